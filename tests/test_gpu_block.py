"""GPU parity: the HIP block path against the CPU oracle, tap by tap, through the C ABI."""
import numpy as np
import pytest
import torch

from zaya_synth import CONFIGS
from tests.zaya_harness import BlockRun, check_routing_exact, check_taps, to_np

pytestmark = pytest.mark.gpu


def small_bf16(**kw):
    """Full ZAYA1 widths, short sequences: several tiles plus a ragged tail everywhere."""
    base = dict(name="small", batch=2, seq=200)
    base.update(kw)
    return CONFIGS["prefill"].replace(**base)


def _full_check(cfg, rows=None, **kw):
    run = BlockRun(cfg, **kw).run()
    ref = run.oracle(rows=rows)
    r = check_routing_exact(run, ref)
    t = check_taps(run, ref)
    print(cfg.name, r, {k: (round(v["max"], 6), round(v["rel_rms"], 6)) for k, v in t.items()}, flush=True)
    return run, ref, r


def test_tiny_fp32_block():
    _full_check(CONFIGS["tiny"])


def test_tiny_fp32_skips_and_uneven_experts():
    _full_check(CONFIGS["tiny"].replace(name="tiny_bb", bal_bias="normal", seq=50, batch=2, conv_std=0.33))


def test_bf16_full_width_ragged():
    _full_check(small_bf16())


def test_bf16_block_zero_semantics_and_unit_conv():
    _full_check(small_bf16(name="small_b0", has_router_state=False, conv_std=0.33, seq=97, batch=1,
                           gain_std=0.05, bal_bias="normal"))


def test_bf16_sliding_window():
    _full_check(small_bf16(name="small_win", seq=300, batch=1, sliding_window=100))


def test_bf16_chunked_prefill_with_cache():
    _full_check(small_bf16(name="small_cached", seq=77, batch=3, kv_len=130))


def test_bf16_decode_small():
    _full_check(CONFIGS["decode"].replace(name="decode_small", batch=5, kv_len=333))


# The two-stage conv (conv_k 2): depthwise taps at unit scale (std 0.33); the grouped
# stage sums 2 * head_dim inputs, so its unit-gain draw has std 1/sqrt(2 d) (0.0625 at
# d = 128). The fp32 case also runs a gain-5 grouped stage (std 0.33) at fp32 tolerance.
def test_tiny_fp32_two_stage_conv():
    _full_check(CONFIGS["tiny"].replace(name="tiny_conv2", conv_k=2, conv_std=0.33, conv2_std=0.33, seq=50,
                                        batch=2))


def test_bf16_two_stage_conv_ragged():
    _full_check(small_bf16(name="small_conv2", conv_k=2, conv_std=0.33, conv2_std=0.0625))


def test_bf16_two_stage_conv_chunked_with_cache():
    _full_check(small_bf16(name="small_conv2_cached", conv_k=2, conv_std=0.33, conv2_std=0.0625, seq=77, batch=3,
                           kv_len=130))


def test_bf16_two_stage_conv_decode():
    _full_check(CONFIGS["decode"].replace(name="decode_conv2", conv_k=2, conv_std=0.33, conv2_std=0.0625, batch=5,
                                          kv_len=333))


def test_deterministic_rerun():
    cfg = small_bf16(name="small_det", seq=150)
    a = BlockRun(cfg).run()
    out1 = a.x_out.clone()
    taps1 = {k: v.clone() for k, v in a.taps.items()}
    a.run()
    assert torch.equal(out1, a.x_out)
    for k, v in taps1.items():
        assert torch.equal(v.view(torch.uint8) if v.dtype != torch.int32 else v,
                           a.taps[k].view(torch.uint8) if v.dtype != torch.int32 else a.taps[k]), k


def test_all_tokens_skip():
    cfg = CONFIGS["tiny"].replace(name="tiny_skip", seq=40)
    from zaya_synth import block_weights
    w = block_weights(cfg)
    w["bal_bias"][:] = 0
    w["bal_bias"][cfg.num_experts] = 2.0
    run, ref, r = _full_check(cfg, w_host=w)
    assert r["routed"] == 0 and r["skipped"] == cfg.seq


def _sample_rows(T, n=48, seed=5):
    """Rows spread over the whole sequence: the first and last tokens, tile edges, and
    a seeded sample in between."""
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 2, 31, 32, 63, 64, 127, 128, 255, 256, T // 2, T - 33, T - 32, T - 2, T - 1]
    pick = rng.choice(T, size=n, replace=False)
    return np.unique(np.clip(np.concatenate([fixed, pick]), 0, T - 1))


def test_full_prefill_workload_sampled_rows():
    """The benchmark's prefill workload (batch 1, 4096 tokens, full widths) in the same
    launch configuration: every tap on sampled rows, routing bit-exact on all tokens."""
    cfg = CONFIGS["prefill"]
    _full_check(cfg, rows=_sample_rows(cfg.tokens))


def test_full_prefill_two_stage_conv_sampled_rows():
    """The benchmark's prefill workload with the printout's two-stage conv (depthwise k2,
    then grouped k2 per head), batch 1 x 4096 tokens at full widths, in the launch
    configuration the benchmark times: every tap on sampled rows, routing bit-exact."""
    cfg = CONFIGS["prefill_conv2"]
    _full_check(cfg, rows=_sample_rows(cfg.tokens))


def test_full_decode_workload():
    """The benchmark's decode workload: batch 64, one new token each over 8192 cached."""
    _full_check(CONFIGS["decode"])


def test_long_context_window_zipf_sampled_rows():
    """The long-context workload: 32768 tokens, sliding window 4096 (4097 keys), and
    balancing biases calibrated by the oracle (tests/golden/make_longctx_bias.py) so the
    expert load follows Zipf(1.2) with 15% skip. Sampled rows include the window edge."""
    import os
    from zaya_synth import block_weights
    cfg = CONFIGS["longctx"]
    path = os.path.join(os.path.dirname(__file__), "golden", "longctx_bal_bias.txt")
    bb = np.array([float(l) for l in open(path) if l.strip() and not l.startswith("#")])
    w = block_weights(cfg, bal_bias=bb)
    T = cfg.tokens
    rows = np.unique(np.concatenate([_sample_rows(T, n=40), [4095, 4096, 4097, 4098, 8191, 8192, 16384]]))
    run, ref, r = _full_check(cfg, rows=rows, w_host=w)
    offs = run.taps["bucket_offsets"].cpu().numpy()
    counts = np.diff(offs)
    print("long context expert counts:", counts.tolist(), "skip:", T - int(offs[-1]), flush=True)
    # the load is strongly skewed: the first expert carries several times the last one's tokens
    assert counts[0] > 5 * counts[-1] and (T - offs[-1]) > 0.1 * T


def test_fp8_experts_decode_workload():
    """The decode workload with the expert weights stored as FP8 E4M3 bytes and fp32 row
    scales: every row and tap against the oracle on the decoded weights."""
    _full_check(CONFIGS["decode_fp8"])


def test_fp8_experts_prefill_several_token_tiles():
    """FP8 experts on a short prefill, where experts receive more than one 16-token tile."""
    run, ref, r = _full_check(small_bf16(name="small_fp8", expert_format="fp8", batch=2, seq=160))
    counts = np.diff(run.taps["bucket_offsets"].cpu().numpy())
    assert counts.max() > 16
