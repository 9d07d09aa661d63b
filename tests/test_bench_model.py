"""The benchmark's host logic: the algorithmic work it divides by (flops and bytes per
stage) against the closed forms of the block's arithmetic, and the one-GPU contract."""
import json
import os
import subprocess
import sys

import pytest

import bench
from zaya_synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_prefill_flops_match_the_closed_form():
    c = CONFIGS["prefill"]
    T, H, d, nh, R, I, E = c.tokens, c.hidden_size, c.head_dim, c.num_heads, c.router_hidden, c.moe_intermediate_size, c.num_experts
    n_r = round(E / (E + 1) * T)  # every class equally likely: 16 of 17 tokens routed
    w = bench.stage_work(c, n_r, E)
    qkv_rows = nh * d + 2 * c.num_kv_heads * d  # q, k, v_current + v_delayed halves
    assert w["qkv_proj"][0] == 2 * T * H * qkv_rows
    assert w["o_proj_merge"][0] == 2 * T * nh * d * H
    # causal: query t sees t + 1 keys; QK and PV are 2 d flops each per (query, key, head)
    assert w["attention"][0] == 4 * d * nh * T * (T + 1) // 2
    assert w["router_down"][0] + w["router_mlp_select"][0] == 2 * T * (H * R + 2 * R * R + (E + 1) * R)
    assert w["expert_gate_up"][0] == 2 * n_r * H * 2 * I
    assert w["expert_down_merge"][0] == 2 * n_r * I * H
    total = sum(v[0] for v in w.values())
    assert abs(total / 1e9 - 179.7) < 0.1  # the scope table's figure for this workload


def test_decode_bytes_are_dominated_by_the_cache():
    c = CONFIGS["decode"]
    w = bench.stage_work(c, 60, 13)
    B, nkv, d = c.batch, c.num_kv_heads, c.head_dim
    kv = 2 * B * nkv * (c.kv_len + 1) * d * 2  # K and V of every visible key, bf16
    assert w["attention"][1] >= kv
    assert w["attention"][1] - kv < 0.01 * kv  # plus queries and outputs only
    # the experts actually used: 13 of them, each [2I, H] + [H, I] bf16
    assert w["expert_gate_up"][1] >= 13 * 2 * c.moe_intermediate_size * c.hidden_size * 2
    assert w["expert_down_merge"][1] >= 13 * c.hidden_size * c.moe_intermediate_size * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]
