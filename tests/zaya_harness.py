"""Shared helpers for the GPU parity tests: upload seeded inputs, run the HIP path
through the C ABI with taps, run the CPU oracle on the same values, compare."""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch

import sparse_moe_block_amd as Z
from oracle import zaya_oracle as O
from zaya_synth import ZayaConfig, block_inputs, block_weights

DEV = "cuda"

# tolerances: bf16 per-element |gpu - oracle| <= 2e-2 * max(1, |oracle|) (bf16 spacing grows
# with magnitude, so a one-ulp difference on a value of 4 is 3e-2) and relative RMS <= 1e-2;
# fp32 configurations 1e-4 for both.
TOL = {"bf16": (2e-2, 1e-2), "f32": (1e-4, 1e-4)}


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def compare(name: str, got: np.ndarray, ref: np.ndarray, act: str) -> Dict[str, float]:
    got = np.asarray(got, np.float64).reshape(ref.shape)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    scaled = err / np.maximum(1.0, np.abs(ref))
    mx = float(scaled.max()) if err.size else 0.0
    den = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    rel = float(np.sqrt(np.mean(err * err)) / den) if den > 0 else float(np.sqrt(np.mean(err * err)) if err.size else 0)
    atol, rtol = TOL[act]
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert mx <= atol, f"{name}: max scaled error {mx:.3e} > {atol}"
    assert rel <= rtol, f"{name}: relative RMS error {rel:.3e} > {rtol}"
    return {"max": mx, "rel_rms": rel}


def upload_weights(w: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    return {k: v.to(DEV).contiguous() for k, v in w.items()}


def np_weights(w: Dict[str, torch.Tensor]) -> Dict[str, np.ndarray]:
    """Oracle view of the weights: float32 arrays (bf16 values are exact in fp32)."""
    return {k: v.float().numpy() for k, v in w.items()}


class BlockRun:
    """One block call on the GPU with all taps, plus the host copies the oracle needs."""

    def __init__(self, cfg: ZayaConfig, w_host=None, inp=None, seed: int = 0, taps: bool = True,
                 decode: Optional[bool] = None):
        self.cfg = cfg
        self.w_host = block_weights(cfg, seed=seed) if w_host is None else w_host
        self.inp = block_inputs(cfg, seed=seed) if inp is None else inp
        self.decode = cfg.decode if decode is None else decode
        self.w = upload_weights(self.w_host)
        B, S, H, R = cfg.batch, cfg.seq, cfg.hidden_size, cfg.router_hidden
        nh, nkv, d, E, I = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.num_experts, cfg.moe_intermediate_size
        T = B * S
        dt = cfg.torch_dtype
        self.x = self.inp["x"].to(DEV)
        self.s_in = self.inp["s_in"].to(DEV) if "s_in" in self.inp else None
        self.x_out = torch.full((B, S, H), float("nan"), device=DEV)
        self.s_out = torch.full((B, S, R), float("nan"), device=DEV, dtype=dt)
        self.cache = None
        if self.decode or cfg.kv_len > 0:
            self.cache = {k: self.inp[k].to(DEV).contiguous() for k in ("K", "V", "conv_state", "prev_hs")}
            self.cache["cache_len"] = [int(v) for v in self.inp["cache_len"]]
            self.cache["cache_len_dev"] = self.inp["cache_len"].to(DEV)
        self.taps = None
        if taps:
            f = lambda *s: torch.full(s, float("nan"), device=DEV, dtype=dt)
            i32 = lambda *s: torch.full(s, -7, device=DEV, dtype=torch.int32)
            self.taps = dict(
                attention_norm_output=f(B, S, H), attention_queries=f(B, nh, S, d), attention_keys=f(B, nkv, S, d),
                attention_values=f(B, nkv, S, d), attention_premix=f(B, S, nh * d), attention_output=f(B, S, H),
                layer_mid=torch.full((B, S, H), float("nan"), device=DEV), mlp_norm_output=f(B, S, H),
                router_logits=f(B, S, E + 1), expert_classes=i32(B, S), expert_indices=i32(B, S),
                expert_weights=f(B, S), bucket_offsets=i32(E + 1), bucket_ids=i32(T), mlp_neurons=f(T, I),
                routed_output=f(B, S, H), mlp_output=f(B, S, H))
        nbytes = Z.zaya_block_workspace_bytes(cfg, B, S, self.decode)
        assert nbytes > 0
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)

    def run(self):
        cfg = self.cfg
        print(f"[gpu] block {'decode' if self.decode else 'prefill'} cfg={cfg.name} B={cfg.batch} S={cfg.seq} "
              f"kv_len={cfg.kv_len} window={cfg.sliding_window}", flush=True)
        if self.decode:
            Z.zaya_block_decode(cfg, self.w, cfg.batch, self.x, self.s_in, self.x_out, self.s_out, self.cache,
                                self.taps, self.ws)
        else:
            Z.zaya_block_prefill(cfg, self.w, cfg.batch, cfg.seq, self.x, self.s_in, self.x_out, self.s_out,
                                 self.cache, self.taps, self.ws)
        torch.cuda.synchronize()
        return self

    # --- oracle side
    def oracle(self, rows=None, force_gpu_routing: bool = True):
        cfg = self.cfg
        w = np_weights(self.w_host)
        x = self.inp["x"].numpy().astype(np.float64)
        s = self.inp["s_in"].float().numpy() if "s_in" in self.inp else None
        cache = None
        if cfg.kv_len > 0:
            cache = {k: self.inp[k].float().numpy() for k in ("K", "V", "conv_state", "prev_hs")}
            cache["cache_len"] = self.inp["cache_len"].numpy()
        fc = self.taps["expert_classes"].cpu().numpy().reshape(-1) if force_gpu_routing else None
        return O.block_forward(cfg, w, x, s, cache, rows=rows, force_cls=fc)


def check_routing_exact(run: BlockRun, ref: dict) -> dict:
    """R1: the oracle's selection applied to the GPU's own logits reproduces the GPU's
    class, index, weight, bucket offsets and ids bit for bit. R2: where the oracle's
    own top-2 margin is wider than the logit error, its decision equals the GPU's."""
    cfg, t = run.cfg, run.taps
    E = cfg.num_experts
    rnd = O.rounder(cfg.act_dtype)
    lg = to_np(t["router_logits"]).reshape(-1, E + 1)
    bb = run.w_host["bal_bias"].numpy().astype(np.float64)
    cls, idx, wt = O.select(lg, bb, rnd)
    g_cls = t["expert_classes"].cpu().numpy().reshape(-1)
    g_idx = t["expert_indices"].cpu().numpy().reshape(-1)
    g_w = to_np(t["expert_weights"]).reshape(-1)
    assert np.array_equal(cls, g_cls), f"class mismatch at {np.nonzero(cls != g_cls)[0][:10]}"
    assert np.array_equal(idx, g_idx)
    assert np.array_equal(wt, g_w), f"weight mismatch at {np.nonzero(wt != g_w)[0][:10]}"
    offs, ids = O.buckets(g_cls, E)
    g_offs = t["bucket_offsets"].cpu().numpy()
    assert np.array_equal(offs, g_offs), (offs, g_offs)
    g_ids = t["bucket_ids"].cpu().numpy()[: offs[-1]]
    assert np.array_equal(ids, g_ids)
    # R2 on the rows the oracle computed
    rows = ref["rows"]
    o_lg = ref["router_logits"]
    o_cls, _, _ = O.select(o_lg, bb, rnd)
    l32 = O.rnd_f32(o_lg)
    sig = O.rnd_f32(O.rnd_f32(O.softmax(l32)) + bb)
    srt = np.sort(sig, axis=-1)
    margin = srt[:, -1] - srt[:, -2]
    lerr = np.max(np.abs(lg[rows] - o_lg), axis=-1)
    # a logit error e moves each softmax entry by at most ~e * (its value) <= e
    decisive = margin > 2 * lerr + 1e-7
    mism = (o_cls != g_cls[rows])
    assert not np.any(mism & decisive), f"decisive routing mismatch at rows {rows[mism & decisive][:10]}"
    return {"near_ties": int(np.sum(~decisive)), "mismatch_near_ties": int(np.sum(mism & ~decisive)),
            "routed": int(offs[-1]), "skipped": int(np.sum(g_cls == E))}


def check_taps(run: BlockRun, ref: dict, skip=()) -> dict:
    cfg, t, act = run.cfg, run.taps, run.cfg.act_dtype
    B, S = cfg.batch, cfg.seq
    rows = ref["rows"]
    res = {}
    bidx, tidx = rows // S, rows % S

    def rowsel(a, last):  # [B, S, last] -> rows
        return to_np(a).reshape(B * S, last)[rows]

    H = cfg.hidden_size
    res["attention_norm_output"] = compare("attention_norm_output",
                                           rowsel(t["attention_norm_output"], H),
                                           ref["attention_norm_output"].reshape(B * S, H)[rows], act)
    q = to_np(t["attention_queries"])  # [B, nh, S, d]
    res["attention_queries"] = compare("attention_queries", q[bidx, :, tidx], ref["attention_queries"][bidx, :, tidx],
                                       act)
    res["attention_keys"] = compare("attention_keys", to_np(t["attention_keys"]), ref["attention_keys"], act)
    res["attention_values"] = compare("attention_values", to_np(t["attention_values"]), ref["attention_values"], act)
    for name, last in (("attention_premix", cfg.num_heads * cfg.head_dim), ("attention_output", H), ("layer_mid", H),
                       ("mlp_norm_output", H), ("router_logits", cfg.num_experts + 1), ("routed_output", H),
                       ("mlp_output", H)):
        if name in skip:
            continue
        res[name] = compare(name, rowsel(t[name], last), ref[name], act)
    res["router_state"] = compare("router_state", to_np(run.s_out).reshape(B * S, -1)[rows], ref["router_state"], act)
    res["layer_output"] = compare("layer_output", to_np(run.x_out).reshape(B * S, H)[rows], ref["layer_output"], act)
    # neurons: GPU rows are in bucket order
    offs = t["bucket_offsets"].cpu().numpy()
    ids = t["bucket_ids"].cpu().numpy()[: offs[-1]]
    pos = np.full(B * S, -1)
    pos[ids] = np.arange(len(ids))
    routed_rows = rows[pos[rows] >= 0]
    if len(routed_rows):
        g = to_np(t["mlp_neurons"])[pos[routed_rows]]
        # Stage-local: the oracle's expert on the GPU's own MoE input rows. The neurons pass
        # four act-dtype roundings (gate, up, activation, product), which turn one-ulp
        # differences upstream into several ulps at |x| ~ 1; end to end they are held to the
        # relative RMS bound, and the block's outputs above to both bounds.
        w = np_weights(run.w_host)
        xin = to_np(t["mlp_norm_output"]).reshape(B * S, H)[routed_rows]
        cls = t["expert_classes"].cpu().numpy().reshape(-1)[routed_rows]
        loc = np.empty_like(g)
        rnd = O.rounder(act)
        for e in np.unique(cls):
            sel = cls == e
            loc[sel] = O.expert(cfg, w, int(e), xin[sel], rnd)[1]
        res["mlp_neurons"] = compare("mlp_neurons", g, loc, act)
        r = ref["mlp_neurons"][np.searchsorted(rows, routed_rows)]
        err = np.abs(g - r)
        e2e = float(np.sqrt(np.mean(err * err)) / max(float(np.sqrt(np.mean(r * r))), 1e-30))
        assert e2e <= TOL[act][1], f"mlp_neurons end to end: relative RMS error {e2e:.3e} > {TOL[act][1]}"
        res["mlp_neurons_e2e"] = {"max": float((err / np.maximum(1.0, np.abs(r))).max()), "rel_rms": e2e}
    return res
