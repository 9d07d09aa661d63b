"""GPU parity of zaya_stack_forward (embedding, blocks with the router state carried
from block to block, final norm, tied lm_head) against the CPU oracle."""
import numpy as np
import pytest
import torch

import sparse_moe_block_amd as Z
from oracle import zaya_oracle as O
from tests.zaya_harness import DEV, TOL, compare, pack_if_needed, stream_bound, to_np
from zaya_synth import (CONFIGS, block_weights, block_weights_device, stack_weights, stack_weights_device,
                        token_ids)

pytestmark = pytest.mark.gpu


def _taps(cfg):
    B, S, H, R, E = cfg.batch, cfg.seq, cfg.hidden_size, cfg.router_hidden, cfg.num_experts
    dt = cfg.torch_dtype
    return dict(layer_output=torch.full((B, S, H), float("nan"), device=DEV),
                router_state=torch.full((B, S, R), float("nan"), device=DEV, dtype=dt),
                router_logits=torch.full((B, S, E + 1), float("nan"), device=DEV, dtype=dt),
                expert_classes=torch.full((B, S), -7, device=DEV, dtype=torch.int32))


def _run_stack(cfg, sw, blocks, ids, taps):
    B, S = cfg.batch, cfg.seq
    logits = torch.full((B, S, cfg.vocab_size), float("nan"), device=DEV, dtype=cfg.torch_dtype)
    ws = torch.empty(Z.zaya_stack_workspace_bytes(cfg, B, S), dtype=torch.uint8, device=DEV)
    print(f"[gpu] stack cfg={cfg.name} L={cfg.num_layers} B={B} S={S} V={cfg.vocab_size}", flush=True)
    Z.zaya_stack_forward(cfg, sw, blocks, B, S, ids, logits, None, taps, ws)
    torch.cuda.synchronize()
    return logits


def test_tiny_fp32_stack_end_to_end():
    cfg = CONFIGS["tiny"].replace(name="tiny_stack", num_layers=3, batch=2, seq=24)
    sw_h = stack_weights(cfg)
    blocks_h = [block_weights(cfg, i) for i in range(cfg.num_layers)]
    ids = token_ids(cfg)
    sw = {k: v.to(DEV) for k, v in sw_h.items()}
    blocks = [{k: v.to(DEV) for k, v in b.items()} for b in blocks_h]
    taps = [_taps(cfg) for _ in range(cfg.num_layers)]
    logits = _run_stack(cfg, sw, blocks, ids.to(DEV), taps)
    npb = [{k: v.float().numpy() for k, v in b.items()} for b in blocks_h]
    ref = O.stack_forward(cfg, {k: v.float().numpy() for k, v in sw_h.items()}, lambda i: npb[i], ids.numpy())
    for l in range(cfg.num_layers):
        compare(f"layer_output[{l}]", to_np(taps[l]["layer_output"]), ref["layer_outputs"][l], "f32", scaled=False)
        compare(f"router_state[{l}]", to_np(taps[l]["router_state"]), ref["router_states"][l], "f32")
    compare("logits", to_np(logits).reshape(-1, cfg.vocab_size), ref["logits"], "f32")


class _HostView:
    """Host copies of one block's device weights, made on first use; the expert stacks
    are copied one expert at a time (the oracle only touches the experts it routes to)."""

    class _Experts:
        def __init__(self, t):
            self.t, self.cache = t, {}

        def __getitem__(self, e):
            if e not in self.cache:
                self.cache[e] = self.t[e].float().cpu().numpy()
            return self.cache[e]

    def __init__(self, w):
        self.w, self.cache = w, {}

    def __getitem__(self, k):
        if k not in self.cache:
            t = self.w[k]
            self.cache[k] = self._Experts(t) if k in ("W_gu", "W_dn") else t.float().cpu().numpy()
        return self.cache[k]


def test_full_stack_workload_blockwise():
    """The 40-block stack (batch 4 x 2048 tokens, vocab 262144): every block of two
    sequences (the first and the last) is checked on a 256-token causal prefix plus rows
    sampled over the whole 2048 tokens (the window of every later token's attention is
    its whole prefix, so these rows reach every key tile). Each block's oracle starts from
    the GPU's own layer input and router state with routing teacher-forced to the GPU's
    choice (so errors do not compound over 40 blocks); routing is bit-exact against the
    oracle's selection of the GPU's logits on every token of both sequences; the head is
    checked on the GPU's last stream at the same rows. The end-to-end oracle (no teacher
    forcing, on a short prefix) is reported, not gated."""
    import time
    cfg = CONFIGS["stack"]
    B, S, L, H = cfg.batch, cfg.seq, cfg.num_layers, cfg.hidden_size
    torch.manual_seed(0)
    sw = stack_weights_device(cfg)
    blocks = [block_weights_device(cfg, i) for i in range(L)]
    ids_h = token_ids(cfg)
    taps = [_taps(cfg) for _ in range(L)]
    t0 = time.time()
    # the library reads the packed expert layout; the oracle below reads the row-major one
    logits = _run_stack(cfg, sw, [pack_if_needed(cfg, b) for b in blocks], ids_h.to(DEV), taps)
    torch.cuda.empty_cache()
    seqs = [0, B - 1]
    bcfg = cfg.replace(batch=len(seqs), seq=S)
    rng = np.random.default_rng(7)
    tsel = np.unique(np.concatenate([np.arange(256), [511, 512, 1023, 1024, S - 2, S - 1],
                                     rng.choice(np.arange(256, S), 18, replace=False)]))
    rows = np.concatenate([j * S + tsel for j in range(len(seqs))])
    emb = sw["embed"].float().cpu().numpy()
    swh = {"embed": emb, "emb_shift": sw["emb_shift"].float().cpu().numpy(),
           "emb_scale": sw["emb_scale"].float().cpu().numpy(), "final_g": sw["final_g"].float().cpu().numpy()}
    _, x = O.embed(bcfg, swh, ids_h[seqs].numpy())
    s = None
    worst = {}
    for l in range(L):
        view = _HostView(blocks[l])
        cls = taps[l]["expert_classes"][seqs].cpu().numpy().reshape(-1)
        lg = to_np(taps[l]["router_logits"][seqs]).reshape(len(seqs) * S, -1)
        c2, _, _ = O.select(lg, view["bal_bias"].astype(np.float64), O.rnd_bf16)
        assert np.array_equal(c2, cls), f"block {l}: routing differs from the selection of the GPU's logits"
        ref = O.block_forward(bcfg, view, x, s, None, rows=rows, force_cls=cls)
        g_out = to_np(taps[l]["layer_output"][seqs]).reshape(len(seqs) * S, H)
        g_st = to_np(taps[l]["router_state"][seqs]).reshape(len(seqs) * S, -1)
        r1 = compare(f"block {l} layer_output", g_out[rows], ref["layer_output"], "bf16",
                     bound=stream_bound("bf16", ref["attention_output"], ref["layer_output"], ref["mlp_output"],
                                        view["m_rs"]))
        r2 = compare(f"block {l} router_state", g_st[rows], ref["router_state"], "bf16")
        worst[l] = (r1["max_abs"], r2["max"])
        x = g_out.reshape(len(seqs), S, H)  # the next block starts from the GPU's stream
        s = g_st.reshape(len(seqs), S, -1)
        if l % 10 == 9:
            print(f"  blocks 0..{l} match on {len(rows)} rows ({time.time() - t0:.0f} s)", flush=True)
    # the head (a 262144-wide product per row) on 16 of the rows, spread over both sequences
    hrows = rows[np.linspace(0, len(rows) - 1, 16).astype(int)]
    _, lg_ref = O.lm_head(bcfg, swh, x.reshape(-1, H)[hrows].reshape(1, len(hrows), H))
    compare("logits (head on the GPU's last stream)", to_np(logits[seqs]).reshape(len(seqs) * S, -1)[hrows],
            lg_ref.reshape(len(hrows), -1), "bf16")
    # end to end (reported): the oracle's own stream through all 40 blocks on a prefix
    k = 4
    views = [_HostView(b) for b in blocks]
    e2e = O.stack_forward(cfg.replace(batch=1, seq=k), swh, lambda i: views[i], ids_h[:1, :k].numpy())
    err = np.abs(to_np(logits[0, :k]) - e2e["logits"])
    print(f"end-to-end logits (oracle without teacher forcing, {k} tokens): max |err| {err.max():.3e}, "
          f"rms {np.sqrt(np.mean(err ** 2)):.3e}; worst block-local layer_output |err| "
          f"{max(v[0] for v in worst.values()):.3e}"
          f", router_state {max(v[1] for v in worst.values()):.3e} ({time.time() - t0:.0f} s)", flush=True)
