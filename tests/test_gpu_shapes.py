"""GPU parity across the configuration space the C ABI accepts, at sizes the oracle
finishes in seconds: head_dim 64 and 128, 1 / 2 / 8 query heads per key head, the
largest expert count (31 + skip) and hidden size (4096), expert widths that are not
powers of two, rotary on no dims and on all dims, a single-token prefill, decode over
cache lengths of mixed sizes (0, 1, one tile, one tile + 1, ...), and a windowed prefill
after a cache."""
import pytest
import torch

from tests.zaya_harness import BlockRun, check_routing_exact, check_taps
from zaya_synth import CONFIGS

pytestmark = pytest.mark.gpu


def _check(cfg, lens=None):
    run = BlockRun(cfg)
    if lens is not None:  # per-sequence cache lengths
        run.inp["cache_len"] = torch.tensor(lens, dtype=torch.int32)
        run.cache["cache_len"] = list(lens)
        run.cache["cache_len_dev"] = run.inp["cache_len"].to("cuda")
    run.run()
    ref = run.oracle()
    r = check_routing_exact(run, ref)
    t = check_taps(run, ref)
    print(cfg.name, r, {k: (round(v["max"], 6), round(v["rel_rms"], 6)) for k, v in t.items()}, flush=True)


def _small(**kw):
    base = dict(act_dtype="bf16", batch=2, seq=40, rope_theta=1e6, router_hidden=256, temp_range=(0.8, 2.0))
    base.update(kw)
    return CONFIGS["tiny"].replace(**base)


SHAPES = [
    # name, overrides
    ("d128_g8_e8_i192", dict(hidden_size=512, num_heads=16, num_kv_heads=2, head_dim=128, rope_dim=64,
                             num_experts=8, moe_intermediate_size=192)),
    ("d64_g1_e31_i64", dict(hidden_size=256, num_heads=4, num_kv_heads=4, head_dim=64, rope_dim=32,
                            num_experts=31, moe_intermediate_size=64, seq=33, batch=1)),
    ("d64_g2_h4096_rope0", dict(hidden_size=4096, num_heads=8, num_kv_heads=4, head_dim=64, rope_dim=0,
                                num_experts=3, moe_intermediate_size=128, seq=20, batch=1)),
    ("d128_g1_rope_all", dict(hidden_size=768, num_heads=2, num_kv_heads=2, head_dim=128, rope_dim=128,
                              num_experts=5, moe_intermediate_size=320, seq=70, batch=1)),
    ("fp32_d128_g2", dict(act_dtype="f32", hidden_size=256, num_heads=4, num_kv_heads=2, head_dim=128, rope_dim=64,
                          num_experts=2, moe_intermediate_size=256, seq=17, batch=2, temp_range=(1.0, 1.0))),
    # bf16 head_dim 128 with 2 and 1 query heads per key head, long enough (25 key tiles)
    # that the longest query tiles split over key chunks and are merged
    ("d128_g2_split", dict(hidden_size=512, num_heads=4, num_kv_heads=2, head_dim=128, rope_dim=64,
                           num_experts=4, moe_intermediate_size=128, seq=1600, batch=1)),
    ("d128_g1_split", dict(hidden_size=256, num_heads=2, num_kv_heads=2, head_dim=128, rope_dim=64,
                           num_experts=3, moe_intermediate_size=128, seq=1550, batch=1)),
    # enough rows (2 x 1200, not a whole number of 128-row tiles) that q/k/v and o_proj
    # take the 8-wave 128x192 tile, with widths that are not a whole number of it (q/k/v:
    # 8 + 4 + 2 heads of 128 = 1792 columns; o_proj: 2048), so their last column tiles are
    # ragged; o_proj keeps the model's reduction length (8 heads x 128). The grouped GEMMs'
    # items (fewer than one round of resident workgroups) all run as half/quarter parts.
    ("d128_g2_ragged_wide", dict(hidden_size=2048, num_heads=8, num_kv_heads=4, head_dim=128, rope_dim=64,
                                 num_experts=4, moe_intermediate_size=512, seq=1200, batch=2)),
]


@pytest.mark.parametrize("name,over", SHAPES, ids=[s[0] for s in SHAPES])
def test_shape_variants(name, over):
    _check(_small(name=name, **over))


def test_single_token_prefill_full_width():
    _check(CONFIGS["prefill"].replace(name="prefill_s1", batch=3, seq=1))


def test_decode_mixed_cache_lengths():
    cfg = CONFIGS["decode"].replace(name="decode_mixed", batch=6, kv_len=200)
    _check(cfg, lens=[0, 1, 63, 64, 65, 200])


def test_windowed_prefill_after_cache():
    cfg = CONFIGS["prefill"].replace(name="prefill_win_cached", batch=2, seq=77, kv_len=130, sliding_window=50)
    _check(cfg)


# Decode in bf16 at head_dim 64 (one dim per lane in the weighted sum, keys paired for
# the bf16 dot products), with 1 and 4 query heads per key head and cache lengths of
# mixed sizes, including a fresh sequence and a partial last tile.
@pytest.mark.parametrize("G", [1, 4])
def test_decode_bf16_head_dim_64(G):
    cfg = _small(name=f"decode_d64_g{G}", hidden_size=512, num_heads=4, num_kv_heads=4 // G, head_dim=64,
                 rope_dim=32, num_experts=6,
                 moe_intermediate_size=128, batch=5, seq=1, kv_len=300, decode=True)
    _check(cfg, lens=[0, 1, 64, 129, 300])
