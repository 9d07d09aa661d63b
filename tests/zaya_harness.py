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


def compare(name: str, got: np.ndarray, ref: np.ndarray, act: str, scaled: bool = True,
            bound: Optional[np.ndarray] = None, outliers_per_million: Optional[float] = None) -> Dict[str, float]:
    """Max and relative-RMS error of got against ref. scaled: the max bound applies to
    |err| / max(1, |ref|) (act-dtype tensors, whose spacing grows with magnitude); False:
    a plain absolute bound. bound: an element-wise bound on |err| instead (the fp32
    stream, see stream_bound; queries and keys, see cca_bound); "max" then reports the
    largest |err| / bound. outliers_per_million (with bound): the scaled contract bound
    must also hold on all but that many elements per million (at least one)."""
    got = np.asarray(got, np.float64).reshape(ref.shape)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    den = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    rel = float(np.sqrt(np.mean(err * err)) / den) if den > 0 else float(np.sqrt(np.mean(err * err)) if err.size else 0)
    atol, rtol = TOL[act]
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if bound is not None:
        bound = np.broadcast_to(np.asarray(bound, np.float64), err.shape)
        ratio = err / bound
        mx = float(ratio.max()) if err.size else 0.0
        assert mx <= 1.0, (f"{name}: error {err.ravel()[ratio.argmax()]:.3e} exceeds its bound "
                           f"{bound.ravel()[ratio.argmax()]:.3e}")
        assert rel <= rtol, f"{name}: relative RMS error {rel:.3e} > {rtol}"
        out = {"max": mx, "rel_rms": rel, "max_abs": float(err.max()) if err.size else 0.0}
        if outliers_per_million is not None:
            over = int(np.sum(err / np.maximum(1.0, np.abs(ref)) > atol))
            allowed = max(1, int(math.ceil(outliers_per_million * err.size / 1e6)))
            assert over <= allowed, f"{name}: {over} elements above the contract bound (at most {allowed})"
            out["over_contract"] = over
        return out
    scaled = err / np.maximum(1.0, np.abs(ref)) if scaled else err
    mx = float(scaled.max()) if err.size else 0.0
    assert mx <= atol, f"{name}: max scaled error {mx:.3e} > {atol}"
    assert rel <= rtol, f"{name}: relative RMS error {rel:.3e} > {rtol}"
    return {"max": mx, "rel_rms": rel}


def stream_bound(act: str, A, stream, M=None, rs_m=None) -> np.ndarray:
    """Element-wise bound on the fp32 stream's error. The stream's own arithmetic is the
    same fp32 operations on both sides ("The stream is float32 whatever the load"); only
    the act-dtype contributions differ: the attention merge's A in layer_mid
    h = (x + rb_a) rs_a + A, and in layer_output (h + rb_m) rs_m + M also M, with h's
    error scaled by rs_m. Each contribution is held to tol max(1, |c|) (its own bound as
    an act-dtype tensor), so the stream is held to the sum, plus two fp32 spacings of
    the result for the final roundings."""
    atol = TOL[act][0]
    b = atol * np.maximum(1.0, np.abs(np.asarray(A, np.float64)))
    if M is not None:
        b = np.abs(np.asarray(rs_m, np.float64)) * b + atol * np.maximum(1.0, np.abs(np.asarray(M, np.float64)))
    return b + 2.0 ** -22 * np.abs(np.asarray(stream, np.float64))


def ulp(x, act: str) -> np.ndarray:
    """Spacing of the act dtype at |x| (bf16: 8 significant bits, fp32: 24)."""
    bits = 8 if act == "bf16" else 24
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - (bits - 1))


def neuron_bound(cfg, w, e: int, x_gpu: np.ndarray, x_ref: np.ndarray, act: str):
    """Element-wise bound on |GPU neuron - oracle neuron| for rows of expert e whose MoE
    inputs are x_gpu on the GPU and x_ref in the oracle.

    The neuron is n = rnd(a u), a = rnd(silu(g)), g = rnd(x W_g^T), u = rnd(x W_u^T).
    Two roundings of values that differ by D differ by at most D plus one spacing at the
    larger magnitude, so, step by step:
      dG, dU  = |(x_gpu - x_ref) W^T| (the upstream input difference, exact in fp64)
                + the GPU's fp32 accumulation bound (K/32 + 31) 2^-24 sum|x||w| (one
                32-term MFMA sum per K-slice, K/32 slices chained);
      dg      = dG + ulp(|g| + dG), du likewise;
      da      = 1.1 dg + ulp(|a| + 1.1 dg) + 1e-5 |a|  (|silu'| < 1.1; the last term
                covers the GPU's fp32 exponential);
      dn      = (|a| + da) du + |u| da + ulp(|n| + ...)  (a'u' - au = a'(u'-u) + u(a'-a)).
    Returns (oracle neurons, bound)."""
    I = cfg.moe_intermediate_size
    rnd = O.rounder(act)
    Wgu = O.expert_weight(cfg, w, "W_gu", e).astype(np.float64)
    xr = np.asarray(x_ref, np.float64)
    xg = np.asarray(x_gpu, np.float64)
    K = xr.shape[1]
    exact = xr @ Wgu.T
    d_in = np.abs((xg - xr) @ Wgu.T)
    acc = (K / 32 + 31) * 2.0 ** -24 * (np.abs(xg) @ np.abs(Wgu).T)
    dGU = d_in + acc
    g, u = rnd(exact[:, :I]), rnd(exact[:, I:])
    dG, dU = dGU[:, :I], dGU[:, I:]
    a = rnd(O.silu(g))
    n = rnd(a * u)
    dg = dG + ulp(np.abs(g) + dG, act)
    du = dU + ulp(np.abs(u) + dU, act)
    da = 1.1 * dg + ulp(np.abs(a) + 1.1 * dg, act) + 1e-5 * np.abs(a)
    dn0 = (np.abs(a) + da) * du + np.abs(u) * da
    return n, dn0 + ulp(np.abs(n) + dn0, act)


def cca_bound(cfg, w, xn_gpu, xn_ref, cache_len, conv_state, prev_hs, act: str):
    """Oracle queries and keys and an element-wise bound on |GPU - oracle| for them.

    The chain ("Queries and keys are convolved, normed to √head_dim and the keys
    scaled"): projections P = rnd(xn W^T) of the q/k channels; the convolution (kernel 3
    in fp32 on P, or the two-stage form y1 = rnd(depthwise(P)), y2 = rnd(grouped(y1)));
    the residual of the projections; X = conv + residual; n = X / |X|; rotary; times
    sqrt(d) (keys also temp); rounded. Two roundings of values that differ by D differ by
    at most D plus one spacing at the larger magnitude, so step by step:
      dP   = |(xn_gpu - xn_ref) W^T| + (H/32 + 31) 2^-24 sum|xn||w| + ulp (0 for history);
      dY   = kernel 3: sum_j |cw_j| dP(t-2+j) + 4 2^-24 (|cb| + sum_j |cw_j x|);
             two stages: dy1 = |w1_0| dP(t-1) + |w1_1| dP(t) + slack + ulp(y1), then
             dy2 = sum |W2| dy1 over the group's two taps + (2d/32 + 31) 2^-24 sum|W2 y1| + ulp(y2);
      dX   = dY + the residual's share of dP ((dPq + dPk)/2 for a query head, its mean
             over the group for the key head);
      dn_i = dX_i / (|X| - |dX|) + |X_i| |dX| / (|X| (|X| - |dX|))   (|dX| the 2-norm);
      rotary mixes the pair: da' = dn_a + dn_b (|cos|, |sin| <= 1);
      out  = s dn' + 1e-5 s (fp32 norm/rotary slack) + ulp, s = sqrt(d) (keys temp sqrt(d)).
    Returns (Q [B, nh, S, d], K [B, nkv, S, d], bound Q, bound K)."""
    rnd = O.rounder(act)
    B, S, H = xn_ref.shape
    nh, nkv, d, r = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.rope_dim
    G = nh // nkv
    C = (nh + nkv) * d
    tr = {}
    cca = O.cca_project(cfg, w, xn_ref, cache_len, conv_state, prev_hs, rnd, trace=tr)
    Wqk = np.asarray(w["W_qkv"][:C], np.float64)
    eps32 = 2.0 ** -24
    bq = np.empty((B, nh, S, d))
    bk = np.empty((B, nkv, S, d))
    temp = np.asarray(w["temp"], np.float64)
    for b in range(B):
        xr = np.asarray(xn_ref[b], np.float64)
        xg = np.asarray(xn_gpu[b], np.float64)
        exact = xr @ Wqk.T
        d_in = np.abs((xg - xr) @ Wqk.T) + (H / 32 + 31) * eps32 * (np.abs(xg) @ np.abs(Wqk).T)
        dP = d_in + ulp(np.abs(exact) + d_in, act)  # [S, C]
        t = tr["seq"][b]
        if cfg.conv_k == 3:
            ext = np.abs(np.concatenate([t["hist"], t["cin"]], axis=0))
            dext = np.concatenate([np.zeros((2, C)), dP], axis=0)
            cw = np.abs(np.asarray(w["conv_w"], np.float64))
            cb = np.abs(np.asarray(w["conv_b"], np.float64))
            dY = sum(cw[:, j][None] * dext[j:j + S] for j in range(3))
            dY += 4 * eps32 * (cb[None] + sum(cw[:, j][None] * ext[j:j + S] for j in range(3)))
        else:
            x = np.abs(np.concatenate([t["hist"][0][None], t["cin"]], axis=0))  # rows -1 .. S-1
            dx = np.concatenate([np.zeros((1, C)), dP], axis=0)
            w1 = np.abs(np.asarray(w["conv_w"], np.float64))
            b1 = np.abs(np.asarray(w["conv_b"], np.float64))
            y1 = t["y1"]  # rows -1 .. S-1
            dy1 = w1[:, 0][None] * dx[0:S] + w1[:, 1][None] * dx[1:S + 1]
            dy1 += 4 * eps32 * (b1[None] + w1[:, 0][None] * x[0:S] + w1[:, 1][None] * x[1:S + 1])
            dy1 += ulp(np.abs(y1[1:]) + dy1, act)
            dy1e = np.concatenate([np.zeros((1, C)), dy1], axis=0)
            W2 = np.abs(np.asarray(w["conv2_w"], np.float64))
            b2 = np.abs(np.asarray(w["conv2_b"], np.float64))
            ay1 = np.abs(y1)
            dY = np.empty((S, C))
            acc = np.empty((S, C))
            for g in range(nh + nkv):
                cs = slice(g * d, (g + 1) * d)
                dY[:, cs] = dy1e[0:S, cs] @ W2[cs, 0, :].T + dy1e[1:S + 1, cs] @ W2[cs, 1, :].T
                acc[:, cs] = b2[cs][None] + ay1[0:S, cs] @ W2[cs, 0, :].T + ay1[1:S + 1, cs] @ W2[cs, 1, :].T
            dY += (2 * d / 32 + 31) * eps32 * acc
            dY += ulp(np.abs(t["conv"]) + dY, act)
        dPq = dP[:, :nh * d].reshape(S, nh, d)
        dPk = dP[:, nh * d:].reshape(S, nkv, d)
        drq = np.stack([(dPq[:, h] + dPk[:, h // G]) / 2 for h in range(nh)], axis=1)
        drk = np.stack([drq[:, g * G:(g + 1) * G].mean(axis=1) for g in range(nkv)], axis=1)
        for X, dX, scale, out, bnd in (
                (t["qt"], dY[:, :nh * d].reshape(S, nh, d) + drq, np.full(nh, math.sqrt(d)), cca["Q"][b], bq[b]),
                (t["kt"], dY[:, nh * d:].reshape(S, nkv, d) + drk, temp * math.sqrt(d), cca["K"][b], bk[b])):
            nX = np.linalg.norm(X, axis=-1, keepdims=True)
            ne = np.linalg.norm(dX, axis=-1, keepdims=True)
            gap = np.where(nX > ne, nX - ne, np.nan)  # a bound needs |X| > |dX| (nan fails the check)
            dn = dX / gap + np.abs(X) * ne / (nX * gap)
            if r:
                half = r // 2
                pair = dn[..., :half] + dn[..., half:r]
                dn = dn.copy()
                dn[..., :half] = pair
                dn[..., half:r] = pair
            sc = np.abs(scale)[None, :, None]
            e = (sc * dn + 1e-5 * sc).transpose(1, 0, 2)  # [heads, S, d]
            bnd[...] = e + ulp(np.abs(out) + e, act)
    return cca["Q"], cca["K"], bq, bk


def pack_if_needed(cfg, w: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    """Device weights in the expert layout the configuration names: with expert_layout
    "packed" the library's zaya_pack_experts lays out the row-major W_gu / W_dn."""
    if getattr(cfg, "expert_layout", "rows") != "packed":
        return w
    out = Z.packed_expert_weights(cfg, w)
    torch.cuda.synchronize()
    return out


def upload_weights(w: Dict[str, torch.Tensor], cfg) -> Dict[str, torch.Tensor]:
    return pack_if_needed(cfg, {k: v.to(DEV).contiguous() for k, v in w.items()})


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
        self.w = upload_weights(self.w_host, cfg)
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
        # the fp32 stream (layer_mid) is held to the bound of its act-dtype contribution
        bnd = stream_bound(act, ref["attention_output"], ref["layer_mid"]) if name == "layer_mid" else None
        res[name] = compare(name, rowsel(t[name], last), ref[name], act, bound=bnd)
    res["router_state"] = compare("router_state", to_np(run.s_out).reshape(B * S, -1)[rows], ref["router_state"], act)
    res["layer_output"] = compare("layer_output", to_np(run.x_out).reshape(B * S, H)[rows], ref["layer_output"], act,
                                  bound=stream_bound(act, ref["attention_output"], ref["layer_output"],
                                                     ref["mlp_output"], np_weights({"m_rs": run.w_host["m_rs"]})["m_rs"]))
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
        # End to end: relative RMS as every tap, and element by element the bound that
        # one rounding flip per act-dtype rounding plus the measured difference of the
        # MoE inputs allow (neuron_bound), evaluated on the oracle's own intermediates.
        ri = np.searchsorted(rows, routed_rows)
        r = ref["mlp_neurons"][ri]
        xr = ref["mlp_norm_output"].reshape(-1, H)[ri]
        err = np.abs(g - r)
        e2e = float(np.sqrt(np.mean(err * err)) / max(float(np.sqrt(np.mean(r * r))), 1e-30))
        assert e2e <= TOL[act][1], f"mlp_neurons end to end: relative RMS error {e2e:.3e} > {TOL[act][1]}"
        worst = 0.0
        for e in np.unique(cls):
            sel = cls == e
            _, bound = neuron_bound(cfg, w, int(e), xin[sel], xr[sel], act)
            ratio = err[sel] / bound
            worst = max(worst, float(ratio.max()))
            assert np.all(err[sel] <= bound), (
                f"mlp_neurons end to end, expert {e}: |err| exceeds the derived bound "
                f"(worst ratio {ratio.max():.3f} at |err| {err[sel].ravel()[ratio.argmax()]:.3e})")
        res["mlp_neurons_e2e"] = {"max": float((err / np.maximum(1.0, np.abs(r))).max()), "rel_rms": e2e,
                                  "max_abs": float(err.max()), "worst_err_over_bound": worst}
    return res
