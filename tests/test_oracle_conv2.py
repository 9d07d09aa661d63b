"""Pins of the oracle's two-stage q/k convolution (the printout's conv_qk_depthwise,
kernel 2, then conv_qk_grouped, kernel 2 with one group per head), used when
conv_k == 2: torch's conv1d composition, a closed-form reduction to a kernel-3
depthwise conv, chunking with the carried state, group locality, and the block-level
decode-after-prefill equality."""
import numpy as np
import torch
import torch.nn.functional as F

from oracle import zaya_oracle as O
from tests.test_oracle_pins import npw, run_block, tiny
from zaya_synth import block_inputs, block_weights

IDENT = lambda v: v  # no rounding: the pins compare exact compositions


def _rand(seed, C=24, S=9, groups=3):
    rng = np.random.default_rng(seed)
    gs = C // groups
    return dict(x=rng.standard_normal((S, C)), w1=rng.standard_normal((C, 2)), b1=rng.standard_normal(C),
                w2=rng.standard_normal((C, 2, gs)), b2=rng.standard_normal(C), groups=groups)


def test_two_stage_is_torch_conv1d_composition():
    a = _rand(0)
    C = a["x"].shape[1]
    y2, _, _ = O.causal_conv_two_stage(a["x"], np.zeros(C), np.zeros(C), a["w1"], a["b1"], a["w2"], a["b2"],
                                       a["groups"], IDENT)
    x = torch.from_numpy(a["x"].T[None])  # [1, C, S]
    y1 = F.conv1d(F.pad(x, (1, 0)), torch.from_numpy(a["w1"][:, None, :]), torch.from_numpy(a["b1"]), groups=C)
    # torch's grouped weight is [C_out, C_in/groups, k]: ours is [C_out, tap, C_in/groups]
    w2t = torch.from_numpy(np.ascontiguousarray(a["w2"].transpose(0, 2, 1)))
    ref = F.conv1d(F.pad(y1, (1, 0)), w2t, torch.from_numpy(a["b2"]), groups=a["groups"])[0].numpy().T
    np.testing.assert_allclose(y2, ref, rtol=1e-12, atol=1e-12)


def test_diagonal_grouped_stage_is_a_kernel3_depthwise_conv():
    # W2[c, tap, c'] = a_tap[c] d(c, c'): y2 = b2 + a0 y1_{t-1} + a1 y1_t, and with
    # y1 = b1 + w0 x_{t-1} + w1 x_t this is the kernel-3 conv with taps
    # (a0 w0, a0 w1 + a1 w0, a1 w1) and bias b2 + (a0 + a1) b1
    a = _rand(1)
    C, gs = a["x"].shape[1], a["w2"].shape[2]
    rng = np.random.default_rng(7)
    a0, a1 = rng.standard_normal(C), rng.standard_normal(C)
    w2 = np.zeros((C, 2, gs))
    for c in range(C):
        w2[c, 0, c % gs] = a0[c]
        w2[c, 1, c % gs] = a1[c]
    xm2, xm1 = rng.standard_normal(C), rng.standard_normal(C)  # inputs two and one tokens back
    y1m1 = a["b1"] + a["w1"][:, 0] * xm2 + a["w1"][:, 1] * xm1
    y2, _, _ = O.causal_conv_two_stage(a["x"], xm1, y1m1, a["w1"], a["b1"], w2, a["b2"], a["groups"], IDENT)
    w0, w1 = a["w1"][:, 0], a["w1"][:, 1]
    cw = np.stack([a0 * w0, a0 * w1 + a1 * w0, a1 * w1], axis=1)
    cb = a["b2"] + (a0 + a1) * a["b1"]
    ref, _ = O.causal_conv3(a["x"], np.stack([xm2, xm1]), cw, cb)
    np.testing.assert_allclose(y2, ref, rtol=1e-12, atol=1e-12)


def test_chunks_with_carried_state_equal_one_pass():
    a = _rand(2, S=13)
    C = a["x"].shape[1]
    for rnd in (IDENT, O.rnd_bf16):
        full, xl, yl = O.causal_conv_two_stage(a["x"], np.zeros(C), np.zeros(C), a["w1"], a["b1"], a["w2"], a["b2"],
                                               a["groups"], rnd)
        p1, x1, y1 = O.causal_conv_two_stage(a["x"][:5], np.zeros(C), np.zeros(C), a["w1"], a["b1"], a["w2"],
                                             a["b2"], a["groups"], rnd)
        p2, x2, y2 = O.causal_conv_two_stage(a["x"][5:], x1, y1, a["w1"], a["b1"], a["w2"], a["b2"], a["groups"], rnd)
        assert np.array_equal(np.concatenate([p1, p2]), full)
        assert np.array_equal(x2, xl) and np.array_equal(y2, yl)
        assert np.array_equal(xl, a["x"][-1])


def test_groups_do_not_mix():
    a = _rand(3)
    C, gs = a["x"].shape[1], a["w2"].shape[2]
    base, _, _ = O.causal_conv_two_stage(a["x"], np.zeros(C), np.zeros(C), a["w1"], a["b1"], a["w2"], a["b2"],
                                         a["groups"], IDENT)
    x = a["x"].copy()
    x[:, gs + 1] += 10.0  # an input channel of group 1
    pert, _, _ = O.causal_conv_two_stage(x, np.zeros(C), np.zeros(C), a["w1"], a["b1"], a["w2"], a["b2"],
                                         a["groups"], IDENT)
    changed = np.any(pert != base, axis=0)
    assert changed[gs:2 * gs].any() and not changed[:gs].any() and not changed[2 * gs:].any()


def test_block_decode_with_two_stage_state_equals_prefill():
    """Prefill S tokens with the two-stage conv, hand K/V, conv_state (last input, last
    depthwise output) and prev_hs over, decode token S: equals a prefill of S+1."""
    cfg = tiny(seq=12, num_kv_heads=2, num_heads=4, conv_k=2, conv_std=0.3, conv2_std=0.3)
    w = npw(block_weights(cfg))
    inp = block_inputs(cfg)
    full = run_block(cfg, w, inp)
    S = 11
    pre = run_block(cfg.replace(seq=S), w, {k: (v[:, :S] if k in ("x", "s_in") else v) for k, v in inp.items()})
    K = np.zeros((1, 2, 12, cfg.head_dim))
    V = np.zeros_like(K)
    K[:, :, :S], V[:, :, :S] = pre["attention_keys"], pre["attention_values"]
    cache = dict(K=K, V=V, conv_state=pre["conv_state"], prev_hs=pre["prev_hs"], cache_len=np.array([S]))
    dec = O.block_forward(cfg.replace(seq=1, kv_len=S, decode=True), w, inp["x"][:, S:].numpy().astype(np.float64),
                          inp["s_in"][:, S:].float().numpy(), cache)
    for k in ("attention_premix", "layer_mid", "layer_output"):
        np.testing.assert_allclose(dec[k][0], full[k][S], rtol=1e-5, atol=1e-6)
    np.testing.assert_allclose(dec["conv_state"], full["conv_state"], atol=1e-6)
    # and the conv matters: the kernel-3 block gives other queries
    k3 = run_block(cfg.replace(conv_k=3), None, inp)
    assert not np.allclose(k3["attention_queries"], full["attention_queries"])
