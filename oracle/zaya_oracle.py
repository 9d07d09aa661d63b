"""CPU oracle for the ZAYA1 decoder-block forward.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import or call this
module; only the tests, the smoke check and the CPU-baseline leg of the benchmark
do. It shares no code with the HIP implementation.

What it computes is the plain definition of the block, written out step by step:
values that the model holds in its load dtype ("act": bfloat16 or float32) are
kept in float64 holding act-representable numbers; every contraction accumulates
in float64; ``rnd`` (round-to-nearest-even to the act dtype) is applied only at
the tensor boundaries the pages name; the residual stream is float32 and its
arithmetic is done op by op in float32.

Sources (all on the nnterp encyclopedia page for ``nnterp.families.zaya``,
"ZAYA1", unless stated):
  * "The Notes / The block, in order" and "From the family module": the block
    order and the merge formula;
  * "The stream is float32 whatever the load": float32 stream, norms cast the
    stream to the weight dtype first, embedding shift/scale before the cast;
  * "Queries and keys are convolved, normed to √head_dim and the keys scaled":
    the CCA projection, residual, value halves, QK norm, temperature, rotary;
  * "One expert per token, chosen beside a skip class" and the family module's
    mixture paragraph: router, state carry, selection, skip;
  * "Printout" and "Config": module shapes, eps, partial rotary factor;
  * "The API / support()": the tap names and layouts returned here.

Readings where the pages are silent or ambiguous are listed in the repository's
design notes; each is flagged at the line that takes it ("reading: ...").

Parity vs the trained ZAYA1 model is unpinned (no weights or reference
activations exist here); every function is pinned by the tests under
``tests/test_oracle_*.py`` against closed forms, invariants, brute force and the
pages' own identities, except two orderings that rest on the pages' wording alone
(parity unpinned: no check can tell them from the alternatives without the trained
model): ``embed`` adds the shift before it multiplies by the scale ("after its shift
and scale"), and ``stream_norm`` rounds the float32 stream to the act dtype before
it norms it ("cast the stream to their weight's dtype before they norm it").
"""
from __future__ import annotations

import math
from typing import Callable, Dict, Optional

import numpy as np
from scipy.special import erf as _erf


# ---------------------------------------------------------------------------
# rounding
# ---------------------------------------------------------------------------

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def rnd_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    bfloat16 has 8 significant bits and float32's exponent range: for |x| in
    [2^(e-1), 2^e) the spacing is 2^(e-8); below the smallest normal 2^-126 the
    spacing stays 2^-133. Dividing by a power of two is exact, and ``np.rint``
    rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    q = np.ldexp(1.0, e - 8)
    y = np.rint(x / q) * q
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, x), y)
    return np.where(np.isfinite(x), y, x)


def rnd_f32(x) -> np.ndarray:
    """Round float64 values to float32 (IEEE round-to-nearest-even), kept as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def rounder(act: str) -> Callable[[np.ndarray], np.ndarray]:
    if act == "bf16":
        return rnd_bf16
    if act == "f32":
        return rnd_f32
    if act == "f64":  # no rounding at all: used by the tests to check exact invariants
        return lambda a: np.asarray(a, dtype=np.float64)
    raise ValueError(f"unknown act dtype {act!r}")


def f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# primitives
# ---------------------------------------------------------------------------

def rmsnorm(x, g, eps, rnd):
    """ZayaRMSNorm on act-dtype input: rnd(g * rnd(x / sqrt(mean(x^2) + eps))).

    Llama-form norm (the family module says the block sits in Llama's
    containers): normalise in high precision, cast back to the load dtype, then
    multiply by the gain in the load dtype. eps = 1e-5 ("Config": rms_norm_eps).
    """
    x = f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = rnd(x / np.sqrt(ms + eps))
    return rnd(f64(g) * y)


def stream_norm(x_stream, g, eps, rnd):
    """Norm of the float32 stream: cast to the weight dtype first, then ZayaRMSNorm.

    ("The stream is float32 whatever the load": the input, post-attention and
    final norms cast the stream to their weight's dtype before norming.)
    """
    return rmsnorm(rnd(f64(x_stream)), g, eps, rnd)


def linear(x, W, rnd, b=None):
    """rnd(x W^T + b): one rounding after a float64 accumulation."""
    y = f64(x) @ f64(W).T
    if b is not None:
        y = y + f64(b)
    return rnd(y)


def gelu_erf(x):
    """GELU with approximate='none' ("Printout": router_mlp.act_fn)."""
    x = f64(x)
    return 0.5 * x * (1.0 + _erf(x / math.sqrt(2.0)))


def silu(x):
    """SiLU ("Printout": experts.act_fn is SiLUActivation; "Config": hidden_act silu)."""
    x = f64(x)
    return x / (1.0 + np.exp(-x))


def softmax(x, axis=-1):
    x = f64(x)
    m = np.max(x, axis=axis, keepdims=True)
    z = np.exp(x - m)
    return z / np.sum(z, axis=axis, keepdims=True)


def merge(o, r_stream, hsb, hss, rb, rs, rnd):
    """ZayaResidualScaling: (o + hsb) * hss + (r + rb) * rs.

    "The Notes / The block, in order" and "The contributions are the merges'
    scaled terms": the contribution (o + hidden_states_bias) * hidden_states_scale
    keeps the load dtype (op by op, each op rounded); the stream term is float32
    ("The stream is float32 whatever the load"). Returns (contribution, stream).
    """
    contrib = rnd(rnd(f64(o) + f64(hsb)) * f64(hss))
    t = rnd_f32(f64(r_stream) + f64(rb))
    t = rnd_f32(t * f64(rs))
    return contrib, rnd_f32(t + contrib)


# ---------------------------------------------------------------------------
# compressed convolutional attention projection
# ---------------------------------------------------------------------------

def split_qkv_rows(cfg):
    """Row ranges of the concatenated projection [q_proj ‖ k_proj ‖ v_proj_current ‖ v_proj_delayed]
    ("Printout": ZayaCCAProjection, out_features 1024 / 256 / 128 / 128 at full size)."""
    nh, nkv, d = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    q = (0, nh * d)
    k = (q[1], q[1] + nkv * d)
    vc = (k[1], k[1] + nkv * d // 2)
    vd = (vc[1], vc[1] + nkv * d // 2)
    return q, k, vc, vd


def causal_conv3(cin, hist, cw, cb):
    """Causal depthwise convolution with kernel 3 and bias, one sequence.

    cin: [S, C] new inputs; hist: [2, C] the two previous inputs (t-2, t-1);
    cw: [C, 3]; cb: [C]. Cross-correlation with the current token on the last
    tap: y_t = cb + cw[:,0] x_{t-2} + cw[:,1] x_{t-1} + cw[:,2] x_t.
    ("Queries and keys are convolved ...": mixing over the current and two
    previous tokens; reading: a single kernel-3 depthwise form with a 2-slot state,
    as the decode-state contract on the JANGTQ2 card's "Architecture Summary" implies.)
    """
    S = cin.shape[0]
    ext = np.concatenate([f64(hist), f64(cin)], axis=0)  # [S+2, C]
    cw = f64(cw)
    y = f64(cb)[None, :] + cw[:, 0][None, :] * ext[0:S] + cw[:, 1][None, :] * ext[1:S + 1] \
        + cw[:, 2][None, :] * ext[2:S + 2]
    return y, ext


def causal_conv_two_stage(cin, x_prev, y1_prev, w1, b1, w2, b2, groups, rnd, trace=None):
    """The printout's two causal convolutions over the q/k channels, one sequence.

    ("Printout": conv_qk_depthwise = Conv1d(C, C, kernel 2, groups C) and
    conv_qk_grouped = Conv1d(C, C, kernel 2, groups 10), both with bias; "Queries and
    keys are convolved ...": together they mix the current and two previous tokens.)
      y1_t = rnd(b1 + w1[:,0] x_{t-1} + w1[:,1] x_t)                  (depthwise)
      y2_t = rnd(b2 + W2[:,0,:] y1_{t-1} + W2[:,1,:] y1_t)  per group   (grouped)
    cin: [S, C]; x_prev, y1_prev: [C] the input and the depthwise output one token
    before the call (zeros for a fresh sequence); w1 [C, 2], b1 [C]; w2 [C, 2, C/groups]
    (output channel, tap, input channel of its group), b2 [C]. Tap 0 takes the previous
    token, tap 1 the current one. Reading: each convolution's output is rounded to the
    act dtype (separate modules); the two-slot state holds (x_{t-1}, y1_{t-1}).
    Returns y2 [S, C] and the new state (x_{S-1}, y1_{S-1}). trace: optional dict that
    receives the depthwise outputs y1 of rows t = -1 .. S-1 (for error analysis only).
    """
    S, C = cin.shape
    x = np.concatenate([f64(x_prev)[None], f64(cin)], axis=0)  # rows t = -1 .. S-1
    w1 = f64(w1)
    y1 = rnd(f64(b1)[None] + w1[:, 0][None] * x[0:S] + w1[:, 1][None] * x[1:S + 1])
    y1e = np.concatenate([f64(y1_prev)[None], y1], axis=0)  # rows t = -1 .. S-1
    if trace is not None:
        trace["y1"] = y1e
    gs = C // groups
    y2 = np.empty((S, C))
    w2 = f64(w2)
    for g in range(groups):
        cs = slice(g * gs, (g + 1) * gs)
        y2[:, cs] = f64(b2)[cs][None] + y1e[0:S, cs] @ w2[cs, 0, :].T + y1e[1:S + 1, cs] @ w2[cs, 1, :].T
    return rnd(y2), x[S], y1e[S]


def rope_rotate(x, pos, rope_dim, theta):
    """Rotary embedding on the first ``rope_dim`` dims of the last axis (rotate-half pairing).

    ("Config": partial_rotary_factor 0.5; "Queries and keys are convolved ...":
    rotary turns the first half of each head.) Pair (j, j + r/2) is rotated by
    angle p * theta^(-2j/r). x: [..., S, d]; pos: [S] integer positions.
    """
    x = f64(x).copy()
    half = rope_dim // 2
    j = np.arange(half, dtype=np.float64)
    inv = theta ** (-2.0 * j / rope_dim)
    ang = np.asarray(pos, np.float64)[:, None] * inv[None, :]  # [S, half]
    c, s = np.cos(ang), np.sin(ang)
    a = x[..., :half].copy()
    b = x[..., half:rope_dim].copy()
    x[..., :half] = a * c - b * s
    x[..., half:rope_dim] = b * c + a * s
    return x


def cca_project(cfg, w, xn, cache_len, conv_state, prev_hs, rnd, trace=None):
    """Queries, keys and values of the CCA projection for B sequences.

    xn: [B, S, H] normed input (act values). cache_len: [B] ints. conv_state:
    [B, C, 2] (kernel 3: slot 0 = input t-2, slot 1 = input t-1; the two-stage form,
    conv_k = 2: slot 0 = input t-1, slot 1 = depthwise output t-1). prev_hs: [B, H] the previous token's
    normed input. A sequence with cache_len 0 is fresh: its history is zero
    whatever the state buffers hold (reading).

    Steps ("Queries and keys are convolved, normed to √head_dim and the keys scaled"):
      1. project q, k, v_current, v_delayed (each rounded to act);
      2. convolve the q and k channels causally over time;
      3. residual: each query head adds the mean of its own projection and its
         key head's projection; each key head adds the mean of those query
         residuals over the query heads it serves;
      4. L2-normalise each head to length sqrt(head_dim); keys times temp[g];
      5. rotary on the first rope_dim dims; round to act;
      6. value head g = [current half of token t ‖ delayed half of token t-1].
    Returns Q [B, nh, S, d], K [B, nkv, S, d], V [B, nkv, S, d] and the new states.
    trace: optional dict that receives, per sequence, the convolution's inputs (history
    rows first), its outputs, the depthwise outputs of the two-stage form and the
    pre-norm query and key vectors (for error analysis only; nothing else changes).
    """
    B, S, H = xn.shape
    nh, nkv, d, r = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.rope_dim
    G = nh // nkv
    C = (nh + nkv) * d
    (q0, q1), (k0, k1), (vc0, vc1), (vd0, vd1) = split_qkv_rows(cfg)
    Wqkv = f64(w["W_qkv"])
    P = linear(xn.reshape(B * S, H), Wqkv, rnd).reshape(B, S, -1)
    Pq = P[..., q0:q1].reshape(B, S, nh, d)
    Pk = P[..., k0:k1].reshape(B, S, nkv, d)
    Vc = P[..., vc0:vc1]
    Vd = P[..., vd0:vd1]

    Q = np.empty((B, nh, S, d))
    K = np.empty((B, nkv, S, d))
    V = np.empty((B, nkv, S, d))
    new_conv = np.empty((B, C, 2))
    new_prev = np.empty((B, H))
    temp = f64(w["temp"])
    half = d // 2
    for b in range(B):
        fresh = int(cache_len[b]) == 0
        hist = np.zeros((2, C)) if fresh else f64(conv_state[b]).T  # [2, C]
        cin = np.concatenate([Pq[b].reshape(S, nh * d), Pk[b].reshape(S, nkv * d)], axis=1)
        tb = {} if trace is not None else None
        if cfg.conv_k == 2:  # the printout's two kernel-2 convolutions; state = (x_{t-1}, y1_{t-1})
            y, xl, y1l = causal_conv_two_stage(cin, hist[0], hist[1], w["conv_w"], w["conv_b"], w["conv2_w"],
                                               w["conv2_b"], nh + nkv, rnd, trace=tb)
            ext = np.concatenate([np.zeros((S, C)), xl[None], y1l[None]], axis=0)  # new state rows S, S+1
        else:
            y, ext = causal_conv3(cin, hist, w["conv_w"], w["conv_b"])
        yq = y[:, :nh * d].reshape(S, nh, d)
        yk = y[:, nh * d:].reshape(S, nkv, d)
        # residual (reading: the pre-conv projections are averaged; g(h) = h // G)
        rq = np.empty((S, nh, d))
        for h in range(nh):
            rq[:, h] = (Pq[b, :, h] + Pk[b, :, h // G]) / 2.0
        rk = np.empty((S, nkv, d))
        for g in range(nkv):
            rk[:, g] = np.mean(rq[:, g * G:(g + 1) * G], axis=1)
        qt = yq + rq
        kt = yk + rk
        if trace is not None:
            tb.update(hist=hist, cin=cin, conv=y, qt=qt, kt=kt)
            trace.setdefault("seq", []).append(tb)
        # L2 norm to sqrt(d); keys scaled by temp (reading: norm clamped at 1e-12)
        qn = math.sqrt(d) * qt / np.maximum(np.linalg.norm(qt, axis=-1, keepdims=True), 1e-12)
        kn = math.sqrt(d) * kt / np.maximum(np.linalg.norm(kt, axis=-1, keepdims=True), 1e-12)
        kn = kn * temp[None, :, None]
        pos = int(cache_len[b]) + np.arange(S)
        Q[b] = rnd(rope_rotate(qn.transpose(1, 0, 2), pos, r, cfg.rope_theta))
        K[b] = rnd(rope_rotate(kn.transpose(1, 0, 2), pos, r, cfg.rope_theta))
        # values: current half first (reading), delayed half from the previous token
        vd_prev = np.zeros(nkv * half) if fresh else linear(f64(prev_hs[b])[None], Wqkv[vd0:vd1], rnd)[0]
        vd_shift = np.concatenate([vd_prev[None], Vd[b, :S - 1]], axis=0)  # [S, nkv*half]
        for g in range(nkv):
            V[b, g, :, :half] = Vc[b, :, g * half:(g + 1) * half]
            V[b, g, :, half:] = vd_shift[:, g * half:(g + 1) * half]
        new_conv[b] = ext[S:S + 2].T
        new_prev[b] = f64(xn[b, S - 1])
    return dict(P=P, Q=Q, K=K, V=V, conv_state=new_conv, prev_hs=new_prev)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def attention(cfg, Q, Kall, Vall, q_pos, rnd, rows_t=None):
    """Grouped-query attention, one sequence.

    Q: [nh, S, d]; Kall, Vall: [nkv, L, d] with key j at position j; q_pos: [S].
    Query head h reads key/value head h // (nh/nkv) ("Config": 8 heads over 2 KV
    heads). Scores Q K^T / sqrt(d), masked causally (p_k <= p_q) and, when the
    window W >= 0, to p_q - p_k <= W (reading of the "4097-token window");
    softmax; weighted sum of values ("The API": attention_scores,
    attention_probabilities, attention_head_outputs). rows_t limits the queries.
    Returns O [S', nh, d] rounded to act.
    """
    nh, nkv, d = Q.shape[0], Kall.shape[0], Q.shape[2]
    G = nh // nkv
    L = Kall.shape[1]
    t_idx = np.arange(Q.shape[1]) if rows_t is None else np.asarray(rows_t)
    qp = np.asarray(q_pos)[t_idx]
    kp = np.arange(L)
    mask = kp[None, :] <= qp[:, None]
    if cfg.sliding_window >= 0:
        mask &= (qp[:, None] - kp[None, :]) <= cfg.sliding_window
    O = np.empty((len(t_idx), nh, d))
    for h in range(nh):
        g = h // G
        s = f64(Q[h, t_idx]) @ f64(Kall[g]).T / math.sqrt(d)
        s = np.where(mask, s, -np.inf)
        p = softmax(s, axis=-1)
        O[:, h] = p @ f64(Vall[g])
    return rnd(O)


# ---------------------------------------------------------------------------
# router, selection, experts
# ---------------------------------------------------------------------------

def router(cfg, w, hn, s_in, rnd):
    """ZayaRouter ("One expert per token ..." and "Printout": router/gate).

    u = down_proj(hn) (+ bias); if a carried state is given (every block but the
    first): u += router_states_scale * state. The state handed to the next block
    is u (reading). router_mlp: RMSNorm(256) -> fc1 -> GELU -> fc2 -> GELU ->
    out_proj (reading of the module order). Returns (u, logits [.., E+1]).
    """
    u = linear(hn, w["r_Wd"], rnd, w["r_bd"])
    if s_in is not None:
        u = rnd(u + rnd(f64(w["r_rss"]) * f64(s_in)))
    z = rmsnorm(u, w["r_norm_g"], cfg.rms_norm_eps, rnd)
    a1 = rnd(gelu_erf(linear(z, w["r_W1"], rnd, w["r_b1"])))
    a2 = rnd(gelu_erf(linear(a1, w["r_W2"], rnd, w["r_b2"])))
    logits = linear(a2, w["r_Wout"], rnd)
    return u, logits


def select(logits, bal_bias, rnd):
    """Top-1 choice beside a skip class ("One expert per token, chosen beside a skip class").

    probs = float32 softmax of the float32 logits (computed in float64, rounded
    to float32); the class is the first argmax of probs + balancing_biases (in
    float32). The last class is skip: weight 0 and index 0. Otherwise the weight
    is the chosen class's own softmax entry, not renormalised, in act dtype.
    Returns (cls, idx, w) with cls == E meaning skip.
    """
    l32 = rnd_f32(logits)
    p = rnd_f32(softmax(l32, axis=-1))
    sig = rnd_f32(p + f64(bal_bias))
    cls = np.argmax(sig, axis=-1)  # first index of the maximum
    E = logits.shape[-1] - 1
    skip = cls == E
    idx = np.where(skip, 0, cls)
    pc = np.take_along_axis(p, cls[..., None], axis=-1)[..., 0]
    wt = np.where(skip, 0.0, rnd(pc))
    return cls.astype(np.int64), idx.astype(np.int64), wt


def buckets(cls_flat, num_experts):
    """Token ids grouped by expert, ascending within each expert; skip tokens excluded.

    Returns (offsets [E+1], ids [N_routed]) with offsets the exclusive prefix sum
    of the per-expert counts.
    """
    cls_flat = np.asarray(cls_flat)
    ids, counts = [], []
    for e in range(num_experts):
        sel = np.nonzero(cls_flat == e)[0]
        ids.append(sel)
        counts.append(len(sel))
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return offsets, np.concatenate(ids).astype(np.int64)


def e4m3_value(code):
    """Value of an OCP FP8 E4M3 byte, from the format's definition: bit 7 sign, bits
    6..3 exponent with bias 7, bits 2..0 mantissa; exponent 0 is subnormal
    (mantissa/8 * 2^-6); the all-ones pattern S.1111.111 is NaN (the format has no
    infinities). Exact in float64."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = (1.0 + man / 8.0) * np.exp2(ex.astype(np.float64) - 7.0)
    sub = man / 8.0 * 2.0 ** -6
    v = sign * np.where(ex == 0, sub, normal)
    return np.where((ex == 15) & ((c & 7) == 7), np.nan, v)


def expert_weight(cfg, w, name, e):
    """Weight matrix of expert e in float64: the stored act values, or with FP8 storage
    the E4M3 byte values times their row scales (fp32)."""
    if getattr(cfg, "expert_format", "act") == "fp8":
        q = np.asarray(w[name][e])
        return e4m3_value(q) * f64(np.asarray(w[name + "_scale"][e]))[:, None]
    return w[name][e]


def expert(cfg, w, e, x, rnd):
    """SwiGLU expert e on rows x: down(rnd(silu(gate x)) * up x).

    ("The API": mlp_activation is the activation's output, mlp_neurons what the
    down projection receives; W_gu[e] holds gate rows then up rows.)
    Returns (activation, neurons, y).
    """
    I = cfg.moe_intermediate_size
    Wgu = expert_weight(cfg, w, "W_gu", e)
    G = linear(x, Wgu[:I], rnd)
    U = linear(x, Wgu[I:], rnd)
    act = rnd(silu(G))
    nrn = rnd(act * U)
    y = linear(nrn, expert_weight(cfg, w, "W_dn", e), rnd)
    return act, nrn, y


# ---------------------------------------------------------------------------
# the block
# ---------------------------------------------------------------------------

def block_forward(cfg, w, x, s_in=None, cache=None, rows=None, force_cls=None, ablate=None,
                  override_attention_output=None):
    """One ZAYA1 decoder block over B sequences of S new tokens.

    x: [B, S, H] float32 stream. s_in: [B, S, R] carried router state or None
    (block-0 semantics). cache: dict(K, V [B, nkv, cap, d]; conv_state [B, C, 2];
    prev_hs [B, H]; cache_len [B]) or None for fresh sequences.
    rows: optional flat token indices (b*S + t) at which to compute everything
    after the attention (all tokens otherwise).
    force_cls: optional [B*S] class per token used instead of the argmax
    (teacher forcing); ablate: optional expert id whose weight is zeroed
    ("Ablating an expert leaves the merge's bias");
    override_attention_output: optional value for the attention contribution
    (for the page's "zeroing attention_output" check).

    Order ("The Notes / The block, in order"):
      h   = merge_a(self_attn(input_layernorm(x)), x)
      out = merge_m(mlp(post_attention_layernorm(h)), h)
    Returns a dict keyed by the tap names of "The API / support()".
    """
    act = cfg.act_dtype
    rnd = rounder(act)
    x = rnd_f32(x)
    B, S, H = x.shape
    nh, nkv, d = cfg.num_heads, cfg.num_kv_heads, cfg.head_dim
    E = cfg.num_experts
    eps = cfg.rms_norm_eps
    if cache is None:
        cache_len = np.zeros(B, np.int64)
        conv_state = np.zeros((B, cfg.conv_channels, 2))
        prev_hs = np.zeros((B, H))
        Kc = Vc = None
    else:
        cache_len = np.asarray(cache["cache_len"], np.int64)
        conv_state, prev_hs = cache["conv_state"], cache["prev_hs"]
        Kc, Vc = cache["K"], cache["V"]

    out = {"layer_input": x}
    xn = stream_norm(x, w["ln1_g"], eps, rnd)
    out["attention_norm_output"] = xn
    cca = cca_project(cfg, w, xn, cache_len, conv_state, prev_hs, rnd)
    out.update(attention_queries=cca["Q"], attention_keys=cca["K"], attention_values=cca["V"],
               qkv=cca["P"], conv_state=cca["conv_state"], prev_hs=cca["prev_hs"])

    all_rows = np.arange(B * S) if rows is None else np.asarray(sorted(rows), np.int64)
    out["rows"] = all_rows
    prem = np.empty((len(all_rows), nh * d))
    for b in range(B):
        sel = all_rows[(all_rows // S) == b]
        if len(sel) == 0:
            continue
        L0 = int(cache_len[b])
        Kall = f64(cca["K"][b]) if L0 == 0 else np.concatenate([f64(Kc[b, :, :L0]), cca["K"][b]], axis=1)
        Vall = f64(cca["V"][b]) if L0 == 0 else np.concatenate([f64(Vc[b, :, :L0]), cca["V"][b]], axis=1)
        O = attention(cfg, cca["Q"][b], Kall, Vall, L0 + np.arange(S), rnd, rows_t=sel - b * S)
        prem[np.searchsorted(all_rows, sel)] = O.reshape(len(sel), nh * d)
    out["attention_premix"] = prem

    xr = x.reshape(B * S, H)[all_rows]
    o = linear(prem, w["W_o"], rnd)
    A, h = merge(o, xr, w["a_hsb"], w["a_hss"], w["a_rb"], w["a_rs"], rnd)
    if override_attention_output is not None:
        A = f64(override_attention_output)
        t = rnd_f32(rnd_f32(xr + f64(w["a_rb"])) * f64(w["a_rs"]))
        h = rnd_f32(t + A)
    out["attention_output"] = A
    out["layer_mid"] = h
    hn = stream_norm(h, w["ln2_g"], eps, rnd)
    out["mlp_norm_output"] = hn
    out["mlp_input"] = hn

    sr = None if s_in is None else f64(s_in).reshape(B * S, -1)[all_rows]
    u, logits = router(cfg, w, hn, sr, rnd)
    out["router_state"] = u
    out["router_logits"] = logits
    cls, idx, wt = select(logits, w["bal_bias"], rnd)
    if force_cls is not None:
        fc = np.asarray(force_cls, np.int64).reshape(-1)[all_rows]
        l32 = rnd_f32(logits)
        p = rnd_f32(softmax(l32, axis=-1))
        cls = fc
        skip = cls == E
        idx = np.where(skip, 0, cls)
        wt = np.where(skip, 0.0, rnd(np.take_along_axis(p, cls[:, None], axis=-1)[:, 0]))
    if ablate is not None:
        wt = np.where(idx == ablate, 0.0, wt)
    out["expert_classes"] = cls
    out["expert_indices"] = idx
    out["expert_weights"] = wt
    if rows is None:
        offs, ids = buckets(cls, E)
        out["bucket_offsets"], out["bucket_ids"] = offs, ids

    I = cfg.moe_intermediate_size
    act_t = np.zeros((len(all_rows), I))
    nrn_t = np.zeros((len(all_rows), I))
    routed = np.zeros((len(all_rows), H))
    for e in range(E):
        sel = np.nonzero(cls == e)[0]
        if len(sel) == 0:
            continue
        a_, n_, y = expert(cfg, w, e, hn[sel], rnd)
        act_t[sel], nrn_t[sel] = a_, n_
        # the slot's weighted output; skip slots (and zero weights) run no expert
        routed[sel] = rnd(wt[sel, None] * y)
    out["mlp_activation"] = act_t
    out["mlp_neurons"] = nrn_t
    out["routed_output"] = routed
    M, o2 = merge(routed, h, w["m_hsb"], w["m_hss"], w["m_rb"], w["m_rs"], rnd)
    out["mlp_output"] = M
    out["layer_output"] = o2
    return out


# ---------------------------------------------------------------------------
# the stack
# ---------------------------------------------------------------------------

def embed(cfg, sw, ids):
    """token_embeddings: rnd(rnd(E[id] + shift) * scale), then cast to float32.

    ("The stream is float32 whatever the load": shift and scale, then the cast;
    reading: shift and scale are [H] vectors applied in that order.)
    """
    rnd = rounder(cfg.act_dtype)
    e = f64(np.asarray(sw["embed"])[np.asarray(ids)])
    te = rnd(rnd(e + f64(sw["emb_shift"])) * f64(sw["emb_scale"]))
    return te, rnd_f32(te)


def lm_head(cfg, sw, x_stream):
    """final norm then the tied head: logits = rnd(norm(x) E^T), no cap or scale
    ("The readout and the tokenizer"; "Config": tie_word_embeddings)."""
    rnd = rounder(cfg.act_dtype)
    xf = stream_norm(x_stream, sw["final_g"], cfg.rms_norm_eps, rnd)
    return xf, linear(xf, sw["embed"], rnd)


def layer_config(cfg, i):
    """Block i's configuration in a stack. ("Queries and keys are convolved ...": the 74B
    preview attends over a 4097-token window on its hybrid_sliding blocks, every other
    block.) Reading: window_layers 1 windows blocks 0, 2, 4, ..., 2 windows blocks 1, 3,
    5, ...; the other blocks attend to the whole prefix; 0 windows every block with
    cfg.sliding_window (which may itself be off)."""
    wl = getattr(cfg, "window_layers", 0)
    if (wl == 1 and i % 2 == 1) or (wl == 2 and i % 2 == 0):
        return cfg.replace(sliding_window=-1)
    return cfg


def stack_forward(cfg, sw, get_block, ids, caches=None):
    """Embedding, ``cfg.num_layers`` blocks with the router state carried from
    block to block (none into block 0), final norm and lm_head.

    get_block(i) returns block i's weights (so the stack never holds them all).
    Returns dict(token_embeddings, layer_outputs [list], final_norm_output, logits).
    """
    te, x = embed(cfg, sw, ids)
    res = {"token_embeddings": te, "layer_outputs": [], "router_states": []}
    s = None
    for i in range(cfg.num_layers):
        c = None if caches is None else caches[i]
        o = block_forward(layer_config(cfg, i), get_block(i), x, s, c)
        x = o["layer_output"].reshape(x.shape)
        s = o["router_state"].reshape(x.shape[0], x.shape[1], -1)
        res["layer_outputs"].append(x)
        res["router_states"].append(s)
    xf, logits = lm_head(cfg, sw, x)
    res["final_norm_output"] = xf
    res["logits"] = logits
    return res
