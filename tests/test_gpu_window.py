"""Sliding-window blocks with a ring-buffer KV cache (position p in slot p % cap, cap =
window + 1) and hybrid stacks (every other block windowed), through the C ABI.

A ring cache only changes where keys and values are stored: the decode attention visits
the same positions in the same order as with a linear cache, so a ring decode step must
give results bit-identical to the linear one on the same history, and the linear step is
checked against the oracle. A ring prefill (fresh sequences) forms its keys in the
workspace like a cacheless prefill and then stores the last cap positions."""
import numpy as np
import pytest
import torch

import sparse_moe_block_amd as Z
from oracle import zaya_oracle as O
from tests.zaya_harness import DEV, BlockRun, check_routing_exact, check_taps, compare, stream_bound, to_np
from zaya_synth import CONFIGS, block_weights, stack_weights, token_ids

pytestmark = pytest.mark.gpu

W = 100
CAP = W + 1


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _ring_from_linear(K, lens, cap):
    """Ring slots holding each sequence's last cap positions; never-written slots are NaN."""
    B, nkv, _, d = K.shape
    R = torch.full((B, nkv, cap, d), float("nan"), dtype=K.dtype, device=K.device)
    for b, L in enumerate(lens):
        for p in range(max(0, L - cap), L):
            R[b, :, p % cap] = K[b, :, p]
    return R


def test_bf16_ring_decode_equals_linear_and_oracle():
    cfg = CONFIGS["decode"].replace(name="decode_ring", batch=5, kv_len=333, sliding_window=W)
    lens = [333, 50, 100, 101, 257]  # shorter than, equal to and wrapped past the ring
    run = BlockRun(cfg)
    run.inp["cache_len"] = torch.tensor(lens, dtype=torch.int32)
    run.cache["cache_len"] = lens
    run.cache["cache_len_dev"] = run.inp["cache_len"].to(DEV)
    conv0, prev0 = run.cache["conv_state"].clone(), run.cache["prev_hs"].clone()
    ring = {"K": _ring_from_linear(run.cache["K"], lens, CAP), "V": _ring_from_linear(run.cache["V"], lens, CAP),
            "conv_state": conv0, "prev_hs": prev0, "cache_len": lens, "cache_len_dev": run.cache["cache_len_dev"],
            "ring": True}
    run.run()
    ref = run.oracle()
    r = check_routing_exact(run, ref)
    t = check_taps(run, ref)
    print(cfg.name, r, {k: (round(v["max"], 6), round(v["rel_rms"], 6)) for k, v in t.items()}, flush=True)
    x_out = torch.full_like(run.x_out, float("nan"))
    s_out = torch.full_like(run.s_out, float("nan"))
    print(f"[gpu] ring decode cfg={cfg.name} cap={CAP} lens={lens}", flush=True)
    Z.zaya_block_decode(cfg, run.w, cfg.batch, run.x, run.s_in, x_out, s_out, ring, None, run.ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(x_out), _bits(run.x_out)) and torch.equal(_bits(s_out), _bits(run.s_out))
    for b, L in enumerate(lens):
        assert torch.equal(_bits(ring["K"][b, :, L % CAP]), _bits(run.cache["K"][b, :, L]))
        assert torch.equal(_bits(ring["V"][b, :, L % CAP]), _bits(run.cache["V"][b, :, L]))
    assert torch.equal(_bits(ring["conv_state"]), _bits(run.cache["conv_state"]))
    assert torch.equal(_bits(ring["prev_hs"]), _bits(run.cache["prev_hs"]))


def test_bf16_ring_prefill_then_decode():
    S = 300
    cfg = CONFIGS["prefill"].replace(name="prefill_ring", batch=2, seq=S, sliding_window=W)
    run = BlockRun(cfg)  # no cache: keys in the workspace
    run.run()
    B, nkv, d, C, H = cfg.batch, cfg.num_kv_heads, cfg.head_dim, cfg.conv_channels, cfg.hidden_size
    dt = cfg.torch_dtype
    ring = {"K": torch.full((B, nkv, CAP, d), float("nan"), dtype=dt, device=DEV),
            "V": torch.full((B, nkv, CAP, d), float("nan"), dtype=dt, device=DEV),
            "conv_state": torch.full((B, C, 2), float("nan"), dtype=dt, device=DEV),
            "prev_hs": torch.full((B, H), float("nan"), dtype=dt, device=DEV),
            "cache_len": [0] * B, "ring": True}
    x_out = torch.full_like(run.x_out, float("nan"))
    s_out = torch.full_like(run.s_out, float("nan"))
    print(f"[gpu] ring prefill cfg={cfg.name} S={S} cap={CAP}", flush=True)
    Z.zaya_block_prefill(cfg, run.w, B, S, run.x, run.s_in, x_out, s_out, ring, None, run.ws)
    torch.cuda.synchronize()
    assert torch.equal(_bits(x_out), _bits(run.x_out)) and torch.equal(_bits(s_out), _bits(run.s_out))
    keys, vals = run.taps["attention_keys"], run.taps["attention_values"]  # [B, nkv, S, d]
    for p in range(S - CAP, S):
        assert torch.equal(_bits(ring["K"][:, :, p % CAP]), _bits(keys[:, :, p]))
        assert torch.equal(_bits(ring["V"][:, :, p % CAP]), _bits(vals[:, :, p]))
    # one decode step on the ring against the oracle's decode on the linear history
    dcfg = cfg.replace(name="prefill_ring_dec", seq=1, kv_len=S, decode=True)
    g = torch.Generator().manual_seed(11)
    xd = torch.randn((B, 1, H), generator=g)
    sd = torch.randn((B, 1, cfg.router_hidden), generator=g).to(dt)
    xo = torch.full((B, 1, H), float("nan"), device=DEV)
    so = torch.full((B, 1, cfg.router_hidden), float("nan"), device=DEV, dtype=dt)
    conv_pre, prev_pre = ring["conv_state"].clone(), ring["prev_hs"].clone()
    ring["cache_len"] = [S] * B
    ws = torch.empty(Z.zaya_block_workspace_bytes(dcfg, B, 1, True), dtype=torch.uint8, device=DEV)
    cls = torch.full((B, 1), -7, dtype=torch.int32, device=DEV)
    print(f"[gpu] ring decode after prefill cfg={dcfg.name}", flush=True)
    Z.zaya_block_decode(dcfg, run.w, B, xd.to(DEV), sd.to(DEV), xo, so, ring, {"expert_classes": cls}, ws)
    torch.cuda.synchronize()
    Kl = torch.zeros((B, nkv, S + 1, d))
    Vl = torch.zeros((B, nkv, S + 1, d))
    Kl[:, :, :S], Vl[:, :, :S] = keys.float().cpu(), vals.float().cpu()
    cache = dict(K=Kl.numpy(), V=Vl.numpy(), conv_state=conv_pre.float().cpu().numpy(),
                 prev_hs=prev_pre.float().cpu().numpy(), cache_len=np.array([S] * B))
    w = {k: v.float().numpy() for k, v in run.w_host.items()}
    ref = O.block_forward(dcfg, w, xd.numpy().astype(np.float64), sd.float().numpy(), cache,
                          force_cls=cls.cpu().numpy().reshape(-1))  # routing teacher-forced to the GPU's
    compare("layer_output", to_np(xo).reshape(B, H), ref["layer_output"], "bf16",
            bound=stream_bound("bf16", ref["attention_output"], ref["layer_output"], ref["mlp_output"], w["m_rs"]))
    compare("router_state", to_np(so).reshape(B, -1), ref["router_state"], "bf16")
    compare("new key", to_np(ring["K"][:, :, S % CAP]), ref["attention_keys"][:, :, 0], "bf16")


@pytest.mark.parametrize("window_layers", [1, 2])
def test_tiny_fp32_hybrid_stack(window_layers):
    cfg = CONFIGS["tiny"].replace(name=f"tiny_hybrid{window_layers}", num_layers=4, batch=2, seq=40,
                                  sliding_window=7, window_layers=window_layers)
    sw_h = stack_weights(cfg)
    blocks_h = [block_weights(cfg, i) for i in range(cfg.num_layers)]
    ids = token_ids(cfg)
    sw = {k: v.to(DEV) for k, v in sw_h.items()}
    blocks = [{k: v.to(DEV) for k, v in b.items()} for b in blocks_h]
    B, S = cfg.batch, cfg.seq
    taps = [dict(layer_output=torch.full((B, S, cfg.hidden_size), float("nan"), device=DEV)) for _ in blocks]
    logits = torch.full((B, S, cfg.vocab_size), float("nan"), device=DEV)
    ws = torch.empty(Z.zaya_stack_workspace_bytes(cfg, B, S), dtype=torch.uint8, device=DEV)
    print(f"[gpu] hybrid stack cfg={cfg.name}", flush=True)
    Z.zaya_stack_forward(cfg, sw, blocks, B, S, ids.to(DEV), logits, None, taps, ws)
    torch.cuda.synchronize()
    npb = [{k: v.float().numpy() for k, v in b.items()} for b in blocks_h]
    ref = O.stack_forward(cfg, {k: v.float().numpy() for k, v in sw_h.items()}, lambda i: npb[i], ids.numpy())
    full = O.stack_forward(cfg.replace(sliding_window=-1), {k: v.float().numpy() for k, v in sw_h.items()},
                           lambda i: npb[i], ids.numpy())
    for l in range(cfg.num_layers):
        compare(f"layer_output[{l}]", to_np(taps[l]["layer_output"]), ref["layer_outputs"][l], "f32", scaled=False)
    compare("logits", to_np(logits).reshape(-1, cfg.vocab_size), ref["logits"], "f32")
    # the window matters here: the GPU is far from the full-attention stack
    assert np.abs(to_np(logits).reshape(-1, cfg.vocab_size) - full["logits"].reshape(-1, cfg.vocab_size)).max() > 1e-2
