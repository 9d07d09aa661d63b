"""Pins of the oracle's FP8 E4M3 expert storage: the byte decoder against the values
the format definition fixes, an independent implementation (torch's float8_e4m3fn),
and the rounding-error bound of the stored weights."""
import numpy as np
import torch

from oracle import zaya_oracle as O
from zaya_synth import CONFIGS, block_weights, fp8_rows


def test_e4m3_values_fixed_by_the_format():
    # OCP FP8 E4M3: bias 7, 3 mantissa bits, subnormals at exponent 0, no infinities,
    # NaN only at S.1111.111
    fixed = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x30: 0.5, 0x38: 1.0, 0x3C: 1.5,
             0x40: 2.0, 0x78: 256.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0}
    for code, v in fixed.items():
        assert O.e4m3_value(code) == v, hex(code)
    assert np.isnan(O.e4m3_value(0x7F)) and np.isnan(O.e4m3_value(0xFF))
    assert O.e4m3_value(0x80) == 0.0 and np.signbit(O.e4m3_value(0x80))
    pos = O.e4m3_value(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)  # codes 0x00..0x7E increase
    assert np.array_equal(O.e4m3_value(np.arange(0x80, 0xFF)), -pos)  # sign bit mirrors


def test_e4m3_decoder_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3_value(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


def test_row_storage_error_bound():
    # weights stored as byte x (max|row| / 448): relative error <= 2^-4 (half a mantissa
    # step) in the normal range, absolute error <= 2^-10 x scale among subnormals
    rng = np.random.default_rng(3)
    W = torch.from_numpy(rng.standard_normal((4, 64, 256)).astype(np.float32) * 0.02)
    st = fp8_rows(W, "W")
    q, s = st["W"].numpy(), st["W_scale"].numpy().astype(np.float64)
    deq = O.e4m3_value(q) * s[..., None]
    w = W.numpy().astype(np.float64)
    scaled = np.abs(w) / s[..., None]
    normal = scaled >= 2.0 ** -6
    assert np.all(np.abs(deq - w)[normal] <= 2.0 ** -4 * np.abs(w)[normal] * (1 + 1e-6))
    assert np.all(np.abs(deq - w)[~normal] <= 2.0 ** -10 * np.broadcast_to(s[..., None], w.shape)[~normal] * (1 + 1e-6))
    # the largest magnitude of each row is stored exactly as +-448 x scale
    assert np.all(np.max(np.abs(O.e4m3_value(q)), axis=-1) == 448.0)


def test_fp8_expert_equals_expert_on_the_decoded_weights():
    # the FP8 configuration's expert is the act configuration's expert on the decoded
    # weights (the storage changes the weights, not the expert's arithmetic)
    cfg8 = CONFIGS["tiny"].replace(name="tiny8", act_dtype="bf16", expert_format="fp8")
    w8 = {k: v.float().numpy() for k, v in block_weights(cfg8).items()}
    cfga = cfg8.replace(expert_format="act")
    wa = dict(w8)
    for name in ("W_gu", "W_dn"):
        wa[name] = O.e4m3_value(w8[name].astype(np.int64)) * w8[name + "_scale"][..., None]
    x = O.rnd_bf16(np.random.default_rng(1).standard_normal((5, cfg8.hidden_size)))
    for e in range(cfg8.num_experts):
        r8 = O.expert(cfg8, w8, e, x, O.rnd_bf16)
        ra = O.expert(cfga, wa, e, x, O.rnd_bf16)
        for a, b in zip(r8, ra):
            assert np.array_equal(a, b)
