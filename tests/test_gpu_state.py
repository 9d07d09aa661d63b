"""The state a block hands to the next decode step, against the oracle.

A call writes its tokens' keys and values into the cache at positions cache_len[b] + t,
and updates conv_state and prev_hs in place ("Queries and keys are convolved, normed to
√head_dim and the keys scaled" on the nnterp page: the convolution mixes the current and
two previous tokens and the value's delayed half reads the previous token; the JANGTQ2
card's "Architecture Summary" lists KV plus conv_state [B, 1280, 2] and prev_hs [B, 2048]
as the decode state). Two kinds of checks:

  * the new conv_state, prev_hs and cache rows after one call, element by element
    against the oracle's new state, for the kernel-3 conv and the printout's two-stage
    conv, over chunk lengths that reach every branch of the state write (one token, two,
    one full 16-token tile, a tile plus one, several tiles with a ragged tail, and the
    4096-token workload), at batch 3 with a fresh sequence in the mix; positions outside
    the written range must be untouched;
  * a GPU prefill of S tokens followed by a GPU decode step that reads the GPU-written
    cache and state, against the oracle's prefill of all S + 1 tokens at the last one
    (every tap), for linear and ring caches and both conv forms.
"""
import numpy as np
import pytest
import torch

import sparse_moe_block_amd as Z
from oracle import zaya_oracle as O
from tests.zaya_harness import (DEV, BlockRun, cca_bound, compare, np_weights, stream_bound, to_np,
                                upload_weights)
from zaya_synth import CONFIGS, block_inputs, block_weights

pytestmark = pytest.mark.gpu

LENS = [0, 5, 130]  # cached tokens per sequence: a fresh one, a short and a longer history


def _bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def _conv_kw(conv_k):
    # unit-scale depthwise taps so a wrong tap or slot is visible; the grouped stage at
    # unit gain 1/sqrt(2 d)
    return dict(conv_k=conv_k, conv_std=0.33, conv2_std=0.0625)


def _state_case(conv_k, S, rows=None):
    kv = max(LENS)
    cfg = CONFIGS["prefill"].replace(name=f"state_k{conv_k}_s{S}", batch=len(LENS), seq=S, kv_len=kv,
                                     decode=S == 1, **_conv_kw(conv_k))
    run = BlockRun(cfg)
    run.inp["cache_len"] = torch.tensor(LENS, dtype=torch.int32)
    run.cache["cache_len"] = list(LENS)
    run.cache["cache_len_dev"] = run.inp["cache_len"].to(DEV)
    before = {k: run.cache[k].clone() for k in ("K", "V", "conv_state", "prev_hs")}
    run.run()
    ref = run.oracle(rows=rows)
    act = cfg.act_dtype
    res = {}
    # conv_state and prev_hs: the whole new state of every sequence
    res["conv_state"] = compare("conv_state", to_np(run.cache["conv_state"]), ref["conv_state"], act)
    res["prev_hs"] = compare("prev_hs", to_np(run.cache["prev_hs"]), ref["prev_hs"], act)
    # the rows written into the cache are the oracle's keys and values at positions L0 + t.
    # Keys (and the queries): every element within the bound derived from one rounding
    # flip per act-dtype rounding of the chain and the measured difference of the normed
    # inputs (cca_bound), and the contract's bound on all but one element per million (a
    # flip of the two-stage conv's output, amplified by the key normalisation, can reach
    # 12 spacings of a key of 0.25 at unit-scale taps). Values (copies of rounded
    # projections): the contract's bound.
    w = np_weights(run.w_host)
    xn_g = to_np(run.taps["attention_norm_output"])
    st = {k: run.inp[k].float().numpy() for k in ("conv_state", "prev_hs")}
    Qr, Kr, bQ, bK = cca_bound(cfg, w, xn_g, ref["attention_norm_output"], np.array(LENS), st["conv_state"],
                               st["prev_hs"], act)
    res["Q"] = compare("queries", to_np(run.taps["attention_queries"]), Qr, act, bound=bQ, outliers_per_million=1)
    for name, tap in (("K", "attention_keys"), ("V", "attention_values")):
        got = run.cache[name]
        for b, L0 in enumerate(LENS):
            res[f"{name}[{b}]"] = compare(f"cache {name} rows of sequence {b}", to_np(got[b, :, L0:L0 + S]),
                                          ref[tap][b], act, bound=bK[b] if name == "K" else None,
                                          outliers_per_million=1 if name == "K" else None)
            # nothing else in the sequence's cache changed
            assert torch.equal(_bits(got[b, :, :L0]), _bits(before[name][b, :, :L0])), (name, b)
            assert torch.equal(_bits(got[b, :, L0 + S:]), _bits(before[name][b, :, L0 + S:])), (name, b)
    # one token after a history: the older slot is the old newer slot, moved bit for bit
    # (kernel 3: inputs t-2, t-1); the two-stage form's slot 0 is the input one token back
    if S == 1 and conv_k == 3:
        for b, L0 in enumerate(LENS):
            if L0 > 0:
                assert torch.equal(_bits(run.cache["conv_state"][b, :, 0]), _bits(before["conv_state"][b, :, 1]))
    print(cfg.name, {k: (round(v["max"], 6), round(v["rel_rms"], 6)) for k, v in res.items()}, flush=True)
    return run, ref


@pytest.mark.parametrize("conv_k", [3, 2])
@pytest.mark.parametrize("S", [1, 2, 16, 17, 77])
def test_state_writes_match_oracle(conv_k, S):
    _state_case(conv_k, S)


@pytest.mark.parametrize("conv_k", [3, 2])
def test_state_writes_match_oracle_4096(conv_k):
    """The benchmark's prefill length (4096 tokens) after the same mixed histories: the
    state comes from the last tile's rows of the projections, not from the tile in LDS."""
    S = 4096
    _state_case(conv_k, S, rows=np.array([b * S + S - 1 for b in range(len(LENS))]))


def _taps_for(cfg, B, S):
    dt = cfg.torch_dtype
    H, nh, nkv, d, E, I = (cfg.hidden_size, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.num_experts,
                           cfg.moe_intermediate_size)
    f = lambda *s: torch.full(s, float("nan"), device=DEV, dtype=dt)
    i32 = lambda *s: torch.full(s, -7, device=DEV, dtype=torch.int32)
    return dict(attention_norm_output=f(B, S, H), attention_queries=f(B, nh, S, d), attention_keys=f(B, nkv, S, d),
                attention_values=f(B, nkv, S, d), attention_premix=f(B, S, nh * d), attention_output=f(B, S, H),
                layer_mid=torch.full((B, S, H), float("nan"), device=DEV), mlp_norm_output=f(B, S, H),
                router_logits=f(B, S, E + 1), expert_classes=i32(B, S), expert_indices=i32(B, S),
                expert_weights=f(B, S), bucket_offsets=i32(E + 1), bucket_ids=i32(B * S), mlp_neurons=f(B * S, I),
                routed_output=f(B, S, H), mlp_output=f(B, S, H))


@pytest.mark.parametrize("conv_k", [3, 2])
@pytest.mark.parametrize("ring", [False, True])
def test_prefill_then_decode_equals_oracle_prefill(conv_k, ring):
    """GPU prefill of S tokens into a cache, then one GPU decode step on the GPU-written
    cache and state, against the oracle's prefill of the S + 1 tokens (fresh) at the last
    token. Linear: cap = S + 1, so the decode writes the cache's last slot. Ring: window
    100, cap 101, with S past the ring so the prefill wraps and the decode overwrites the
    oldest slot."""
    S, B = (77, 2) if not ring else (150, 2)
    W = 100 if ring else -1
    cfg = CONFIGS["prefill"].replace(name=f"pd_k{conv_k}_{'ring' if ring else 'lin'}", batch=B, seq=S + 1,
                                     sliding_window=W, **_conv_kw(conv_k))
    w_host = block_weights(cfg)
    inp = block_inputs(cfg)  # x [B, S+1, H], s_in [B, S+1, R]
    w = upload_weights(w_host, cfg)
    H, R, nkv, d, C = cfg.hidden_size, cfg.router_hidden, cfg.num_kv_heads, cfg.head_dim, cfg.conv_channels
    dt = cfg.torch_dtype
    cap = W + 1 if ring else S + 1
    cache = {"K": torch.full((B, nkv, cap, d), float("nan"), dtype=dt, device=DEV),
             "V": torch.full((B, nkv, cap, d), float("nan"), dtype=dt, device=DEV),
             "conv_state": torch.full((B, C, 2), float("nan"), dtype=dt, device=DEV),
             "prev_hs": torch.full((B, H), float("nan"), dtype=dt, device=DEV),
             "cache_len": [0] * B, "ring": ring}
    x = inp["x"].to(DEV)
    s_in = inp["s_in"].to(DEV)
    pcfg = cfg.replace(seq=S)
    xo = torch.full((B, S, H), float("nan"), device=DEV)
    so = torch.full((B, S, R), float("nan"), device=DEV, dtype=dt)
    ws = torch.empty(Z.zaya_block_workspace_bytes(pcfg, B, S), dtype=torch.uint8, device=DEV)
    print(f"[gpu] prefill {cfg.name} S={S} cap={cap}", flush=True)
    Z.zaya_block_prefill(pcfg, w, B, S, x[:, :S].contiguous(), s_in[:, :S].contiguous(), xo, so, cache, None, ws)
    dcfg = cfg.replace(seq=1, decode=True, kv_len=S)
    cache["cache_len"] = [S] * B
    cache["cache_len_dev"] = torch.full((B,), S, dtype=torch.int32, device=DEV)
    taps = _taps_for(dcfg, B, 1)
    xo1 = torch.full((B, 1, H), float("nan"), device=DEV)
    so1 = torch.full((B, 1, R), float("nan"), device=DEV, dtype=dt)
    ws1 = torch.empty(Z.zaya_block_workspace_bytes(dcfg, B, 1, True), dtype=torch.uint8, device=DEV)
    print(f"[gpu] decode after prefill {cfg.name}", flush=True)
    Z.zaya_block_decode(dcfg, w, B, x[:, S:].contiguous(), s_in[:, S:].contiguous(), xo1, so1, cache, taps, ws1)
    torch.cuda.synchronize()

    # the oracle: one prefill of all S + 1 tokens, evaluated at the last token of each
    # sequence, routing teacher-forced to the GPU decode's choice (checked bit-exact below)
    rows = np.array([b * (S + 1) + S for b in range(B)])
    gcls = taps["expert_classes"].cpu().numpy().reshape(-1)
    fc = np.zeros(B * (S + 1), np.int64)
    fc[rows] = gcls
    npw = np_weights(w_host)
    ref = O.block_forward(cfg, npw, inp["x"].numpy().astype(np.float64), inp["s_in"].float().numpy(), None,
                          rows=rows, force_cls=fc)
    act = cfg.act_dtype
    E = cfg.num_experts
    # R1: the oracle's selection of the GPU's logits is the GPU's routing
    lg = to_np(taps["router_logits"]).reshape(B, E + 1)
    cls, idx, wt = O.select(lg, npw["bal_bias"].astype(np.float64), O.rounder(act))
    assert np.array_equal(cls, gcls)
    assert np.array_equal(wt, to_np(taps["expert_weights"]).reshape(-1))
    res = {}
    t_last = S
    res["attention_norm_output"] = compare("attention_norm_output", to_np(taps["attention_norm_output"]).reshape(B, H),
                                           ref["attention_norm_output"][:, t_last], act)
    for name in ("attention_queries", "attention_keys", "attention_values"):
        res[name] = compare(name, to_np(taps[name])[:, :, 0], ref[name][:, :, t_last], act)
    for name, last in (("attention_premix", cfg.num_heads * d), ("attention_output", H), ("layer_mid", H),
                       ("mlp_norm_output", H), ("router_logits", E + 1), ("routed_output", H), ("mlp_output", H)):
        bnd = stream_bound(act, ref["attention_output"], ref["layer_mid"]) if name == "layer_mid" else None
        res[name] = compare(name, to_np(taps[name]).reshape(B, last), ref[name], act, bound=bnd)
    res["router_state"] = compare("router_state", to_np(so1).reshape(B, R), ref["router_state"], act)
    res["layer_output"] = compare("layer_output", to_np(xo1).reshape(B, H), ref["layer_output"], act,
                                  bound=stream_bound(act, ref["attention_output"], ref["layer_output"],
                                                     ref["mlp_output"], npw["m_rs"]))
    # the decode's own state writes: key/value at position S, and the state after S + 1 tokens
    slot = S % cap
    res["cache K"] = compare("cache K", to_np(cache["K"][:, :, slot]), ref["attention_keys"][:, :, t_last], act)
    res["cache V"] = compare("cache V", to_np(cache["V"][:, :, slot]), ref["attention_values"][:, :, t_last], act)
    res["conv_state"] = compare("conv_state", to_np(cache["conv_state"]), ref["conv_state"], act)
    res["prev_hs"] = compare("prev_hs", to_np(cache["prev_hs"]), ref["prev_hs"], act)
    print(cfg.name, {k: (round(v["max"], 6), round(v["rel_rms"], 6)) for k, v in res.items()}, flush=True)
