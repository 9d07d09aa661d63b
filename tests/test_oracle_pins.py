"""Pins of the CPU oracle to things other than itself: library routines on the
special cases that reduce to them, closed forms, invariants, brute force on tiny
inputs, and the pages' own checks. CPU only."""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import zaya_oracle as O
from zaya_synth import CONFIGS, block_inputs, block_weight_shapes, block_weights

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def npw(w):
    return {k: v.float().numpy().astype(np.float64) for k, v in w.items()}


def tiny(**kw):
    base = dict(seq=16)
    base.update(kw)
    return CONFIGS["tiny"].replace(**base)


def run_block(cfg, w=None, inp=None, **kw):
    w = npw(block_weights(cfg)) if w is None else w
    inp = block_inputs(cfg) if inp is None else inp
    x = inp["x"].numpy().astype(np.float64)
    s = inp["s_in"].float().numpy() if "s_in" in inp else None
    cache = None
    if cfg.kv_len > 0:
        cache = {k: inp[k].float().numpy() for k in ("K", "V", "conv_state", "prev_hs")}
        cache["cache_len"] = inp["cache_len"].numpy()
    return O.block_forward(cfg, w, x, s, cache, **kw)


# --------------------------------------------------------------------------- rounding

def test_rnd_bf16_matches_torch_conversion():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal(200000) * np.exp2(rng.integers(-140, 120, 200000))).astype(np.float32)
    x = np.concatenate([x, np.float32([0.0, -0.0, 1e-45, 3.4e38, -3.4e38, np.inf, -np.inf])])
    ours = O.rnd_bf16(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy().astype(np.float64)
    np.testing.assert_array_equal(ours, ref)


def test_rnd_bf16_ties_to_even_on_every_midpoint():
    # every finite positive bf16 value b and its successor; the midpoint must go to the even one
    bits = np.arange(0x0000, 0x7F7F, dtype=np.uint32)
    lo = (bits << 16).view(np.float32).astype(np.float64)
    hi = ((bits + 1) << 16).view(np.float32).astype(np.float64)
    mid = (lo + hi) / 2
    got = O.rnd_bf16(mid)
    even = np.where(bits % 2 == 0, lo, hi)
    np.testing.assert_array_equal(got, even)
    np.testing.assert_array_equal(O.rnd_bf16(lo), lo)  # fixed points
    # just off the midpoint goes to the nearer neighbour
    np.testing.assert_array_equal(O.rnd_bf16(np.nextafter(mid, lo)), lo)
    np.testing.assert_array_equal(O.rnd_bf16(np.nextafter(mid, hi)), hi)


# --------------------------------------------------------------------------- primitives

def test_rmsnorm_is_torch_rms_norm_without_rounding():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 96)) * 3
    g = 1 + 0.1 * rng.standard_normal(96)
    ours = O.rmsnorm(x, g, 1e-5, O.rounder("f64"))
    ref = F.rms_norm(torch.from_numpy(x), (96,), weight=torch.from_numpy(g), eps=1e-5).numpy()
    np.testing.assert_allclose(ours, ref, rtol=1e-13, atol=0)


def test_rmsnorm_unit_mean_square_and_scale_invariance():
    rng = np.random.default_rng(3)
    x = O.rnd_bf16(rng.standard_normal((7, 2048)) * 5)
    y = O.rmsnorm(x, np.ones(2048), 1e-5, O.rnd_bf16)
    np.testing.assert_allclose(np.mean(y * y, axis=-1), 1.0, atol=5e-3)
    # a power-of-two scale changes nothing (eps aside)
    y2 = O.rmsnorm(x * 8.0, np.ones(2048), 1e-5 * 64, O.rnd_bf16)
    np.testing.assert_array_equal(y, y2)


def test_linear_brute_force():
    rng = np.random.default_rng(4)
    x, W, b = rng.standard_normal((3, 5)), rng.standard_normal((4, 5)), rng.standard_normal(4)
    ref = np.zeros((3, 4))
    for i in range(3):
        for j in range(4):
            acc = 0.0
            for k in range(5):
                acc += x[i, k] * W[j, k]
            ref[i, j] = acc + b[j]
    np.testing.assert_allclose(O.linear(x, W, O.rounder("f64"), b), ref, rtol=1e-14, atol=1e-14)


def test_gelu_and_silu_are_torch_functions():
    x = np.linspace(-8, 8, 1001)
    t = torch.from_numpy(x)
    np.testing.assert_allclose(O.gelu_erf(x), F.gelu(t).numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(O.silu(x), F.silu(t).numpy(), rtol=1e-14, atol=1e-15)


def test_conv_is_torch_depthwise_conv1d_with_left_history():
    rng = np.random.default_rng(5)
    S, C = 11, 6
    cin, hist = rng.standard_normal((S, C)), rng.standard_normal((2, C))
    cw, cb = rng.standard_normal((C, 3)), rng.standard_normal(C)
    y, _ = O.causal_conv3(cin, hist, cw, cb)
    ext = torch.from_numpy(np.concatenate([hist, cin]).T[None])  # [1, C, S+2]
    ref = F.conv1d(ext, torch.from_numpy(cw)[:, None, :], torch.from_numpy(cb), groups=C)[0].T
    np.testing.assert_allclose(y, ref.numpy(), rtol=1e-14, atol=1e-14)


def test_conv_impulse_response():
    S, C, t0, c0 = 9, 4, 3, 2
    cin = np.zeros((S, C))
    cin[t0, c0] = 1.0
    cw = np.arange(12, dtype=np.float64).reshape(C, 3) + 1
    y, _ = O.causal_conv3(cin, np.zeros((2, C)), cw, np.zeros(C))
    expect = np.zeros((S, C))
    expect[t0, c0], expect[t0 + 1, c0], expect[t0 + 2, c0] = cw[c0, 2], cw[c0, 1], cw[c0, 0]
    np.testing.assert_array_equal(y, expect)


def test_rope_is_complex_rotation_and_relative():
    rng = np.random.default_rng(6)
    d, r, theta = 16, 8, 1e4
    x = rng.standard_normal((5, d))
    pos = np.array([0, 1, 7, 100, 4096])
    y = O.rope_rotate(x, pos, r, theta)
    half = r // 2
    z = x[:, :half] + 1j * x[:, half:r]
    om = theta ** (-np.arange(half) * 2.0 / r)
    zr = z * np.exp(1j * pos[:, None] * om[None, :])
    np.testing.assert_allclose(y[:, :half], zr.real, atol=1e-12)
    np.testing.assert_allclose(y[:, half:r], zr.imag, atol=1e-12)
    np.testing.assert_array_equal(y[:, r:], x[:, r:])  # dims past rope_dim untouched
    np.testing.assert_array_equal(y[0], x[0])  # position 0 is the identity
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    a = O.rope_rotate(q[None], [37], r, theta) @ O.rope_rotate(k[None], [5], r, theta).T
    b = O.rope_rotate(q[None], [1037], r, theta) @ O.rope_rotate(k[None], [1005], r, theta).T
    np.testing.assert_allclose(a, b, rtol=1e-10)


def test_softmax_select_weight_identity_from_the_page():
    # probs = logits.float().softmax(-1); probs.gather(-1, idx).to(w.dtype) == w
    rng = np.random.default_rng(7)
    logits = O.rnd_bf16(rng.standard_normal((500, 17)) * 2)
    cls, idx, wt = O.select(logits, np.zeros(17), O.rnd_bf16)
    probs = torch.from_numpy(logits.astype(np.float32)).softmax(-1)
    keep = cls != 16
    g = probs.gather(-1, torch.from_numpy(idx[:, None]))[:, 0].to(torch.bfloat16).double().numpy()
    torch.testing.assert_close(torch.from_numpy(wt[keep]), torch.from_numpy(g[keep]))
    assert np.all(wt[~keep] == 0) and np.all(idx[~keep] == 0)
    assert np.all(wt[keep] < 1)


def test_select_trained_biases_never_pick_skip():
    rng = np.random.default_rng(8)
    logits = O.rnd_bf16(rng.standard_normal((4000, 17)) * 3)
    logits[:, 16] += 6  # make skip the raw favourite
    bb = np.zeros(17)
    bb[16], bb[3] = -1.0, 0.1
    cls, _, _ = O.select(logits, bb, O.rnd_bf16)
    assert np.all(cls != 16)


def test_select_ties_go_to_lowest_index():
    logits = np.zeros((3, 5))
    logits[1, [2, 3]] = 4.0
    logits[2, [4, 1]] = 4.0
    cls, idx, wt = O.select(logits, np.zeros(5), O.rnd_f32)
    assert list(cls) == [0, 2, 1]
    # bias can break a tie: expert 3 preferred by 2^-10
    cls2, _, _ = O.select(logits[1:2], np.array([0, 0, 0, 2.0 ** -10, 0]), O.rnd_f32)
    assert cls2[0] == 3
    # skip is the last class; when it wins, index and weight are zero
    l3 = np.array([[0, 0, 0, 0, 9.0]])
    c3, i3, w3 = O.select(l3, np.zeros(5), O.rnd_f32)
    assert (c3[0], i3[0], w3[0]) == (4, 0, 0.0)


def test_buckets_brute_force_and_invariants():
    rng = np.random.default_rng(9)
    E = 6
    cls = rng.integers(0, E + 1, 300)
    offs, ids = O.buckets(cls, E)
    assert offs[0] == 0 and np.all(np.diff(offs) >= 0)
    assert offs[-1] == np.sum(cls != E) == len(ids)
    assert len(set(ids.tolist())) == len(ids)
    for e in range(E):
        seg = ids[offs[e]:offs[e + 1]]
        assert list(seg) == [t for t in range(300) if cls[t] == e]


# --------------------------------------------------------------------------- CCA

def test_cca_residual_closed_form_with_zero_conv():
    cfg = tiny(act_dtype="f64", rope_dim=0, num_kv_heads=2, num_heads=4, seq=6)
    w = npw(block_weights(cfg))
    w["conv_w"][:] = 0
    w["conv_b"][:] = 0
    w["temp"][:] = 1
    rng = np.random.default_rng(10)
    xn = rng.standard_normal((1, 6, cfg.hidden_size))
    r = O.cca_project(cfg, w, xn, [0], None, None, O.rounder("f64"))
    d, G = cfg.head_dim, 2
    P = xn[0] @ w["W_qkv"].T
    Pq = P[:, :4 * d].reshape(6, 4, d)
    Pk = P[:, 4 * d:6 * d].reshape(6, 2, d)
    for h in range(4):
        qt = (Pq[:, h] + Pk[:, h // G]) / 2
        np.testing.assert_allclose(r["Q"][0, h], math.sqrt(d) * qt / np.linalg.norm(qt, axis=-1, keepdims=True),
                                   rtol=1e-12, atol=1e-12)
    for g in range(2):
        kt = (Pq[:, g * G:(g + 1) * G].mean(axis=1) + Pk[:, g]) / 2
        np.testing.assert_allclose(r["K"][0, g], math.sqrt(d) * kt / np.linalg.norm(kt, axis=-1, keepdims=True),
                                   rtol=1e-12, atol=1e-12)


def test_qk_norms_and_temperature():
    cfg = tiny(act_dtype="f64", num_kv_heads=2, temp_range=(0.8, 12.9))
    w = npw(block_weights(cfg))
    rng = np.random.default_rng(11)
    xn = rng.standard_normal((2, 16, cfg.hidden_size))
    r = O.cca_project(cfg, w, xn, [0, 5], np.ones((2, cfg.conv_channels, 2)), np.ones((2, cfg.hidden_size)),
                      O.rounder("f64"))
    d = cfg.head_dim
    np.testing.assert_allclose(np.linalg.norm(r["Q"], axis=-1), math.sqrt(d), rtol=1e-12)
    for g in range(2):
        np.testing.assert_allclose(np.linalg.norm(r["K"][:, g], axis=-1), w["temp"][g] * math.sqrt(d), rtol=1e-12)


def test_temperature_zero_zeroes_keys_and_makes_attention_uniform():
    cfg = tiny()
    w = npw(block_weights(cfg))
    w["temp"][:] = 0
    out = run_block(cfg, w)
    assert np.all(out["attention_keys"] == 0)
    V = out["attention_values"][0, 0]  # [S, d]
    prefix_mean = np.cumsum(V, axis=0) / np.arange(1, cfg.seq + 1)[:, None]
    prem = out["attention_premix"].reshape(cfg.seq, cfg.num_heads, cfg.head_dim)
    for h in range(cfg.num_heads):
        np.testing.assert_allclose(prem[:, h], O.rnd_f32(prefix_mean), rtol=0, atol=1e-6)


def test_value_halves_current_then_delayed():
    cfg = tiny(num_kv_heads=2, num_heads=4)
    w = npw(block_weights(cfg))
    (_, _), (_, _), (vc0, vc1), (vd0, vd1) = O.split_qkv_rows(cfg)
    w["W_qkv"][vd0:vd1] = w["W_qkv"][vc0:vc1]  # delayed == current projection
    out = run_block(cfg, w)
    V = out["attention_values"][0]
    half = cfg.head_dim // 2
    np.testing.assert_array_equal(V[:, 1:, half:], V[:, :-1, :half])
    assert np.all(V[:, 0, half:] == 0)  # fresh sequence: no previous token
    w["W_qkv"][vd0:vd1] = 0
    out = run_block(cfg, w)
    assert np.all(out["attention_values"][0][:, :, half:] == 0)


# --------------------------------------------------------------------------- attention

def _attn_inputs(nh=4, nkv=2, S=9, d=8, seed=12):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((nh, S, d)), rng.standard_normal((nkv, S, d)), rng.standard_normal((nkv, S, d))


def test_attention_matches_torch_sdpa():
    Q, K, V = _attn_inputs()
    cfg = tiny()
    ours = O.attention(cfg, Q, K, V, np.arange(9), O.rounder("f64"))
    Kr = torch.from_numpy(K).repeat_interleave(2, dim=0)
    Vr = torch.from_numpy(V).repeat_interleave(2, dim=0)
    ref = F.scaled_dot_product_attention(torch.from_numpy(Q), Kr, Vr, is_causal=True)
    np.testing.assert_allclose(ours, ref.numpy().transpose(1, 0, 2), rtol=1e-12, atol=1e-12)


def test_attention_brute_force_with_window_and_cache_offset():
    Q, K, V = _attn_inputs(S=7)
    L = 7
    q_pos = np.array([3, 4, 5, 6])  # last four tokens are new; three cached before them
    Qn = Q[:, 3:]
    for W in (-1, 0, 1, 2, 10):
        cfg = tiny(sliding_window=W)
        ours = O.attention(cfg, Qn, K, V, q_pos, O.rounder("f64"))
        for h in range(4):
            g = h // 2
            for i, p in enumerate(q_pos):
                vis = [j for j in range(L) if j <= p and (W < 0 or p - j <= W)]
                s = [sum(Qn[h, i, k] * K[g, j, k] for k in range(8)) / math.sqrt(8) for j in vis]
                m = max(s)
                e = [math.exp(v - m) for v in s]
                z = sum(e)
                o = [sum(e[a] / z * V[g, j, k] for a, j in enumerate(vis)) for k in range(8)]
                np.testing.assert_allclose(ours[i, h], o, rtol=1e-12, atol=1e-12)


def test_window_special_cases():
    Q, K, V = _attn_inputs(S=9)
    f = O.rounder("f64")
    full = O.attention(tiny(), Q, K, V, np.arange(9), f)
    np.testing.assert_array_equal(O.attention(tiny(sliding_window=9), Q, K, V, np.arange(9), f), full)
    w0 = O.attention(tiny(sliding_window=0), Q, K, V, np.arange(9), f)
    for h in range(4):
        np.testing.assert_allclose(w0[:, h], V[h // 2], rtol=1e-14)


# --------------------------------------------------------------------------- merges (the page's identity)

def test_contribution_identity_from_the_page():
    cfg = tiny()
    w = npw(block_weights(cfg))
    out = run_block(cfg, w)
    x = torch.from_numpy(out["layer_input"].astype(np.float32)).reshape(-1, cfg.hidden_size)
    attn = torch.from_numpy(out["attention_output"].astype(np.float32))
    mlp = torch.from_numpy(out["mlp_output"].astype(np.float32))
    o = torch.from_numpy(out["layer_output"].astype(np.float32))
    t = {k: torch.from_numpy(w[k].astype(np.float32)) for k in ("a_rb", "a_rs", "m_rb", "m_rs")}
    h = (x + t["a_rb"]) * t["a_rs"] + attn
    torch.testing.assert_close((h + t["m_rb"]) * t["m_rs"] + mlp, o)


def test_merge_is_plain_add_at_initial_values():
    rng = np.random.default_rng(13)
    x = O.rnd_f32(rng.standard_normal((4, 32)))
    o = O.rnd_bf16(rng.standard_normal((4, 32)))
    A, h = O.merge(o, x, np.zeros(32), np.ones(32), np.zeros(32), np.ones(32), O.rnd_bf16)
    np.testing.assert_array_equal(A, o)
    np.testing.assert_array_equal(h, O.rnd_f32(x + o))


def test_zeroing_attention_output_leaves_scaled_stream():
    cfg = tiny()
    w = npw(block_weights(cfg))
    out = run_block(cfg, w, override_attention_output=0.0)
    x = out["layer_input"].reshape(-1, cfg.hidden_size).astype(np.float32)
    ref = (x + w["a_rb"].astype(np.float32)) * w["a_rs"].astype(np.float32)
    np.testing.assert_array_equal(out["layer_mid"], ref.astype(np.float64))


# --------------------------------------------------------------------------- router / MoE

def test_router_state_scale_zero_equals_block_zero():
    cfg = tiny()
    w = npw(block_weights(cfg))
    w["r_rss"][:] = 0
    a = run_block(cfg, w)
    b = run_block(cfg.replace(has_router_state=False), w)
    np.testing.assert_array_equal(a["router_logits"], b["router_logits"])


def test_moe_forced_to_one_expert_is_a_dense_swiglu():
    cfg = tiny(act_dtype="f64")
    w = npw(block_weights(cfg))
    e = 2
    out = run_block(cfg, w, force_cls=np.full(cfg.seq, e))
    hn = torch.from_numpy(out["mlp_input"])
    I = cfg.moe_intermediate_size
    Wg, Wu, Wd = (torch.from_numpy(a) for a in (w["W_gu"][e, :I], w["W_gu"][e, I:], w["W_dn"][e]))
    dense = (F.silu(hn @ Wg.T) * (hn @ Wu.T)) @ Wd.T
    wt = torch.from_numpy(out["expert_weights"])[:, None]
    np.testing.assert_allclose(out["routed_output"], (wt * dense).numpy(), rtol=1e-12, atol=1e-14)


def test_ablating_an_expert_changes_exactly_its_tokens():
    cfg = tiny(bal_bias="normal")
    w = npw(block_weights(cfg))
    clean = run_block(cfg, w)
    idx, wt = clean["expert_indices"], clean["expert_weights"]
    for e in range(cfg.num_experts):
        abl = run_block(cfg, w, ablate=e)
        chose = (idx == e) & (wt > 0)
        assert np.array_equal((abl["mlp_output"] != clean["mlp_output"]).any(-1), chose)
        # at those tokens mlp_output falls back to rnd(rnd(hsb) * hss)
        hb = O.rnd_f32(w["m_hsb"] * w["m_hss"])
        assert np.all(abl["mlp_output"][chose] == hb[None, :])


def test_skip_tokens_get_only_the_merge_bias():
    cfg = tiny()
    w = npw(block_weights(cfg))
    w["bal_bias"][:] = 0
    w["bal_bias"][cfg.num_experts] = 2.0  # everyone skips
    out = run_block(cfg, w)
    assert np.all(out["expert_classes"] == cfg.num_experts)
    assert np.all(out["expert_indices"] == 0) and np.all(out["expert_weights"] == 0)
    assert np.all(out["routed_output"] == 0)
    assert len(out["bucket_ids"]) == 0
    np.testing.assert_array_equal(out["mlp_output"], np.broadcast_to(O.rnd_f32(w["m_hsb"] * w["m_hss"]),
                                                                      out["mlp_output"].shape))


# --------------------------------------------------------------------------- whole block

def test_causality_future_tokens_do_not_change_the_past():
    cfg = tiny(seq=24)
    w = npw(block_weights(cfg))
    inp = block_inputs(cfg)
    a = run_block(cfg, w, inp)
    inp2 = {k: v.clone() for k, v in inp.items()}
    inp2["x"][:, 10:] += torch.randn_like(inp2["x"][:, 10:])
    inp2["s_in"][:, 10:] = 0.5
    b = run_block(cfg, w, inp2)
    H = cfg.hidden_size
    for k in ("attention_premix", "layer_mid", "router_logits", "layer_output"):
        np.testing.assert_array_equal(a[k][:10], b[k][:10])
    np.testing.assert_array_equal(a["attention_queries"][:, :, :10], b["attention_queries"][:, :, :10])
    assert not np.array_equal(a["layer_output"][10:], b["layer_output"][10:])


def test_batch_independence():
    cfg = tiny(batch=3, seq=8)
    w = npw(block_weights(cfg))
    inp = block_inputs(cfg)
    full = run_block(cfg, w, inp)
    c1 = cfg.replace(batch=1)
    for b in range(3):
        one = {k: v[b:b + 1] for k, v in inp.items()}
        o = run_block(c1, w, one)
        np.testing.assert_allclose(o["layer_output"], full["layer_output"][b * 8:(b + 1) * 8], rtol=0, atol=1e-6)


def test_decode_with_state_equals_prefill():
    """Prefill S tokens, hand K/V, conv_state and prev_hs over, decode token S: the
    result equals the last token of a prefill of S+1 tokens."""
    cfg = tiny(seq=12, num_kv_heads=2, num_heads=4)
    w = npw(block_weights(cfg))
    inp = block_inputs(cfg)
    full = run_block(cfg, w, inp)
    S = 11
    pre = run_block(cfg.replace(seq=S), w, {k: (v[:, :S] if k in ("x", "s_in") else v) for k, v in inp.items()})
    cap = 12
    K = np.zeros((1, 2, cap, cfg.head_dim))
    V = np.zeros_like(K)
    K[:, :, :S], V[:, :, :S] = pre["attention_keys"], pre["attention_values"]
    cache = dict(K=K, V=V, conv_state=pre["conv_state"], prev_hs=pre["prev_hs"], cache_len=np.array([S]))
    dcfg = cfg.replace(seq=1, kv_len=S, decode=True)
    dec = O.block_forward(dcfg, w, inp["x"][:, S:].numpy().astype(np.float64),
                          inp["s_in"][:, S:].float().numpy(), cache)
    for k in ("attention_premix", "layer_mid", "router_logits", "layer_output", "mlp_output"):
        np.testing.assert_allclose(dec[k][0], full[k][S], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(dec["attention_queries"][0, :, 0], full["attention_queries"][0, :, S], atol=1e-5)
    np.testing.assert_allclose(dec["conv_state"], full["conv_state"], atol=1e-6)


# --------------------------------------------------------------------------- shapes vs the pages' numbers

def _golden():
    vals = {}
    for line in open(os.path.join(GOLDEN, "page_constants.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            vals[k] = v
    return vals


def test_parameter_tally_reproduces_total_size():
    """Our layout of every tensor but the conv, plus the printout's two convolutions
    (depthwise k2 and grouped k2 with 10 groups, both with bias), the per-block router
    state scale (blocks 1..39), the temperatures, balancing biases and the embedding
    shift/scale, gives exactly half the published byte count of the bf16 checkpoint."""
    g = _golden()
    L, V = int(g["num_hidden_layers"]), int(g["vocab_size"])
    cfg = CONFIGS["prefill"]
    sh = block_weight_shapes(cfg)
    per_block = sum(int(np.prod(s)) for k, s in sh.items() if k not in ("conv_w", "conv_b", "r_rss"))
    C = int(g["conv_channels"])
    conv = (C * 2 + C) + (C * (C // int(g["conv_groups"])) * 2 + C)
    total = L * (per_block + conv) + (L - 1) * cfg.router_hidden
    total += V * cfg.hidden_size + 2 * cfg.hidden_size + cfg.hidden_size  # embed, shift/scale, final norm
    assert total * 2 == int(g["total_size_bytes"])
    assert V * cfg.hidden_size * 2 == int(g["embed_bytes"])


def test_shapes_match_the_printout_and_kv_bytes():
    g = _golden()
    cfg = CONFIGS["prefill"]
    assert cfg.hidden_size == int(g["hidden_size"]) and cfg.head_dim == int(g["head_dim"])
    assert cfg.num_heads == int(g["num_attention_heads"]) and cfg.num_kv_heads == int(g["num_key_value_heads"])
    assert cfg.num_experts == int(g["num_experts"]) and cfg.moe_intermediate_size == int(g["moe_intermediate_size"])
    assert cfg.rope_dim == cfg.head_dim * float(g["partial_rotary_factor"])
    assert cfg.conv_channels == int(g["conv_channels"])
    q, k, vc, vd = O.split_qkv_rows(cfg)
    assert (q[1] - q[0], k[1] - k[0], vc[1] - vc[0], vd[1] - vd[0]) == (
        int(g["q_proj_out"]), int(g["k_proj_out"]), int(g["v_proj_current_out"]), int(g["v_proj_delayed_out"]))
    assert cfg.num_experts + 1 == int(g["router_classes"]) and cfg.router_hidden == int(g["router_hidden"])
    kv = cfg.num_kv_heads * cfg.head_dim * 2 * 2 * int(g["num_hidden_layers"])  # K and V, bf16
    assert kv == int(g["kv_cache_kib_per_token"]) * 1024


def test_router_matches_torch_modules_without_rounding():
    """down_proj (+bias) + router_states_scale * state, then RMSNorm(256) -> fc1 ->
    GELU -> fc2 -> GELU -> out_proj built from torch's own modules."""
    cfg = tiny(act_dtype="f64")
    w = npw(block_weights(cfg))
    rng = np.random.default_rng(14)
    hn = rng.standard_normal((10, cfg.hidden_size))
    s = rng.standard_normal((10, cfg.router_hidden))
    u, logits = O.router(cfg, w, hn, s, O.rounder("f64"))
    t = {k: torch.from_numpy(v) for k, v in w.items()}
    ut = F.linear(torch.from_numpy(hn), t["r_Wd"], t["r_bd"]) + t["r_rss"] * torch.from_numpy(s)
    z = F.rms_norm(ut, (cfg.router_hidden,), weight=t["r_norm_g"], eps=cfg.rms_norm_eps)
    a = F.gelu(F.linear(F.gelu(F.linear(z, t["r_W1"], t["r_b1"])), t["r_W2"], t["r_b2"]))
    np.testing.assert_allclose(u, ut.numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(logits, F.linear(a, t["r_Wout"]).numpy(), rtol=1e-12, atol=1e-13)


def test_embedding_shift_scale_and_tied_head():
    from zaya_synth import stack_weights, token_ids
    cfg = tiny(act_dtype="f64", seq=5)
    sw = npw(stack_weights(cfg))
    ids = token_ids(cfg).numpy()
    te, x = O.embed(cfg, sw, ids)
    np.testing.assert_allclose(te, (sw["embed"][ids] + sw["emb_shift"]) * sw["emb_scale"], rtol=1e-15)
    sw1 = dict(sw, emb_shift=np.zeros_like(sw["emb_shift"]), emb_scale=np.ones_like(sw["emb_scale"]))
    np.testing.assert_array_equal(O.embed(cfg, sw1, ids)[0], sw["embed"][ids])
    xf, logits = O.lm_head(cfg, sw, x)
    ref = F.rms_norm(torch.from_numpy(x), (cfg.hidden_size,), weight=torch.from_numpy(sw["final_g"]), eps=1e-5)
    np.testing.assert_allclose(logits, (ref @ torch.from_numpy(sw["embed"]).T).numpy(), rtol=1e-11, atol=1e-12)


def test_stack_carries_router_state_from_block_to_block():
    from zaya_synth import stack_weights, token_ids
    cfg = tiny(seq=6, num_layers=2)
    sw = npw(stack_weights(cfg))
    blocks = [npw(block_weights(cfg, i)) for i in range(2)]
    ids = token_ids(cfg).numpy()
    res = O.stack_forward(cfg, sw, lambda i: blocks[i], ids)
    _, x0 = O.embed(cfg, sw, ids)
    b0 = O.block_forward(cfg, blocks[0], x0, None)  # block 0: no carried state
    np.testing.assert_array_equal(res["layer_outputs"][0].reshape(-1, cfg.hidden_size), b0["layer_output"])
    s0 = b0["router_state"].reshape(1, 6, -1)
    b1 = O.block_forward(cfg, blocks[1], b0["layer_output"].reshape(1, 6, -1), s0)
    np.testing.assert_array_equal(res["layer_outputs"][1].reshape(-1, cfg.hidden_size), b1["layer_output"])
    b1n = O.block_forward(cfg, blocks[1], b0["layer_output"].reshape(1, 6, -1), None)
    assert not np.array_equal(b1n["router_logits"], b1["router_logits"])
