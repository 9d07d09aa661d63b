"""A multi-block decode step captured in a HIP graph (through torch.cuda.CUDAGraph) gives
bit-identical results to the same calls made eagerly, on every replay.

The library allocates nothing and launches only kernels and device-to-device copies on
the caller's stream, with every host-side decision taken from the call's arguments, so
a captured step replays exactly what the eager step ran. Replays are interleaved with
unrelated eager GPU work and synchronisations, and each replay starts from the same
cache state (the step writes K/V at position cache_len and updates conv_state and
prev_hs in place), so each must reproduce the eager outputs bit for bit."""
import pytest
import torch

import sparse_moe_block_amd as Z
from tests.zaya_harness import DEV, pack_if_needed
from zaya_synth import CONFIGS, _device_stream, block_weights_device

pytestmark = pytest.mark.gpu

L_BLOCKS = 4


def _caches(cfg, n_blocks):
    B, nkv, d, H, C = cfg.batch, cfg.num_kv_heads, cfg.head_dim, cfg.hidden_size, cfg.conv_channels
    cap = cfg.kv_len + 1
    out = []
    for l in range(n_blocks):
        def rnd(name, shape):
            g = _device_stream(0, cfg.name + "_graph", l, name, DEV)
            return torch.randn(shape, generator=g, device=DEV).to(cfg.torch_dtype)
        K = torch.zeros((B, nkv, cap, d), device=DEV, dtype=cfg.torch_dtype)
        V = torch.zeros_like(K)
        K[:, :, :cfg.kv_len] = rnd("K", (B, nkv, cfg.kv_len, d))
        V[:, :, :cfg.kv_len] = rnd("V", (B, nkv, cfg.kv_len, d))
        out.append({"K": K, "V": V, "conv_state": rnd("conv", (B, C, 2)), "prev_hs": rnd("prev", (B, H)),
                    "cache_len": [cfg.kv_len] * B,
                    "cache_len_dev": torch.full((B,), cfg.kv_len, dtype=torch.int32, device=DEV)})
    return out


def test_graph_captured_decode_step_is_bit_identical_to_eager():
    cfg = CONFIGS["decode"]
    B, H, R = cfg.batch, cfg.hidden_size, cfg.router_hidden
    blocks = [pack_if_needed(cfg, block_weights_device(cfg, l)) for l in range(L_BLOCKS)]
    caches = _caches(cfg, L_BLOCKS)
    pos = cfg.kv_len
    g0 = _device_stream(0, cfg.name + "_graph", -1, "x", DEV)
    xs = [torch.randn((B, H), generator=g0, device=DEV)] + [torch.empty((B, H), device=DEV) for _ in range(L_BLOCKS)]
    ss = [torch.randn((B, R), generator=g0, device=DEV).to(cfg.torch_dtype)] + \
         [torch.empty((B, R), device=DEV, dtype=cfg.torch_dtype) for _ in range(L_BLOCKS)]
    ws = torch.empty(Z.zaya_block_workspace_bytes(cfg, B, 1, True), dtype=torch.uint8, device=DEV)
    pristine = [{k: c[k].clone() for k in ("conv_state", "prev_hs")} for c in caches]

    def restore():
        for c, p in zip(caches, pristine):
            c["conv_state"].copy_(p["conv_state"])
            c["prev_hs"].copy_(p["prev_hs"])
            c["K"][:, :, pos].zero_()
            c["V"][:, :, pos].zero_()
        for t in xs[1:]:
            t.fill_(float("nan"))
        for t in ss[1:]:
            t.fill_(float("nan"))

    def step():
        for l in range(L_BLOCKS):
            Z.zaya_block_decode(cfg, blocks[l], B, xs[l], ss[l], xs[l + 1], ss[l + 1], caches[l], workspace=ws)

    def snapshot():
        out = {f"x{l}": xs[l + 1].clone() for l in range(L_BLOCKS)}
        out.update({f"s{l}": ss[l + 1].clone() for l in range(L_BLOCKS)})
        for l, c in enumerate(caches):
            out[f"conv{l}"] = c["conv_state"].clone()
            out[f"prev{l}"] = c["prev_hs"].clone()
            out[f"K{l}"] = c["K"][:, :, pos].clone()
            out[f"V{l}"] = c["V"][:, :, pos].clone()
        return out

    restore()
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    eager = snapshot()
    assert all(torch.isfinite(v.float()).all() for v in eager.values())

    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        restore()
        # unrelated eager work between replays
        a = torch.randn((512, 512), device=DEV)
        (a @ a).sum().item()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k, v in eager.items():
            assert torch.equal(v.view(torch.uint8) if v.dtype != torch.float32 else v.view(torch.int32),
                               got[k].view(torch.uint8) if v.dtype != torch.float32 else got[k].view(torch.int32)), \
                f"replay {rep}: {k} differs from the eager step"
        print(f"replay {rep}: {len(eager)} tensors bit-identical", flush=True)


def test_graph_replay_with_grown_cache_length_matches_oracle():
    """A decode step captured at cache length 1000 and replayed after the caller advanced
    the device-side lengths to 1100 (a graph cannot see the host array): the attention
    covered 4 chunks of 256 keys (1024 positions) at capture, so the replay must derive
    longer chunks from the device lengths to reach all 1101 keys. Checked against the
    oracle's decode at length 1100 (routing teacher-forced to the replay's, R1 bit-exact)."""
    import numpy as np
    from oracle import zaya_oracle as O
    from tests.zaya_harness import compare, np_weights, stream_bound, to_np, upload_weights
    from zaya_synth import block_inputs, block_weights
    L_new, L_cap = 1100, 1000
    cfg = CONFIGS["decode"].replace(name="decode_graph_grow", batch=4, kv_len=L_new)
    B, H, R, E = cfg.batch, cfg.hidden_size, cfg.router_hidden, cfg.num_experts
    w_host = block_weights(cfg)
    inp = block_inputs(cfg)  # K/V filled to 1100 positions, cap 1101
    w = upload_weights(w_host, cfg)
    cache = {k: inp[k].to(DEV).contiguous() for k in ("K", "V", "conv_state", "prev_hs")}
    cache["cache_len"] = [L_cap] * B
    cache["cache_len_dev"] = torch.full((B,), L_cap, dtype=torch.int32, device=DEV)
    x, s_in = inp["x"].to(DEV), inp["s_in"].to(DEV)
    xo = torch.full((B, 1, H), float("nan"), device=DEV)
    so = torch.full((B, 1, R), float("nan"), device=DEV, dtype=cfg.torch_dtype)
    taps = {"router_logits": torch.full((B, 1, E + 1), float("nan"), device=DEV, dtype=cfg.torch_dtype),
            "expert_classes": torch.full((B, 1), -7, device=DEV, dtype=torch.int32)}
    ws = torch.empty(Z.zaya_block_workspace_bytes(cfg, B, 1, True), dtype=torch.uint8, device=DEV)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    print(f"[gpu] capture decode at cache length {L_cap}, replay at {L_new}", flush=True)
    with torch.cuda.graph(graph):  # capture only: nothing runs until the replay
        Z.zaya_block_decode(cfg, w, B, x, s_in, xo, so, cache, taps, ws)
    torch.cuda.synchronize()
    cache["cache_len_dev"].fill_(L_new)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    npw = np_weights(w_host)
    gcls = taps["expert_classes"].cpu().numpy().reshape(-1)
    lg = to_np(taps["router_logits"]).reshape(B, E + 1)
    cls, _, _ = O.select(lg, npw["bal_bias"].astype(np.float64), O.rnd_bf16)
    assert np.array_equal(cls, gcls)
    ocache = {k: inp[k].float().numpy() for k in ("K", "V", "conv_state", "prev_hs")}
    ocache["cache_len"] = np.full(B, L_new)
    ref = O.block_forward(cfg, npw, inp["x"].numpy().astype(np.float64), inp["s_in"].float().numpy(), ocache,
                          force_cls=gcls)
    r = compare("layer_output", to_np(xo).reshape(B, H), ref["layer_output"], "bf16",
                bound=stream_bound("bf16", ref["attention_output"], ref["layer_output"], ref["mlp_output"],
                                   npw["m_rs"]))
    compare("router_state", to_np(so).reshape(B, R), ref["router_state"], "bf16")
    compare("new key at 1100", to_np(cache["K"][:, :, L_new]), ref["attention_keys"][:, :, 0], "bf16")
    compare("conv_state", to_np(cache["conv_state"]), ref["conv_state"], "bf16")
    print("replay at grown cache length:", r, flush=True)
