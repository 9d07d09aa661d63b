"""The allocation-free decode entry point (zaya_block_decode_noalloc: the workspace is a
static device array of the library) against zaya_block_decode with a caller workspace:
the same kernels run in the same launch configuration, so every output, tap and state
write must be bit-identical. Two calls in a row, the second smaller than the first, so
the second runs on an array that still holds the first call's intermediates."""
import pytest
import torch

import sparse_moe_block_amd as Z
from tests.zaya_harness import DEV, upload_weights
from zaya_synth import CONFIGS, block_inputs, block_weights

pytestmark = pytest.mark.gpu


def _bits(t):
    if t.dtype == torch.float32:
        return t.view(torch.int32)
    if t.dtype == torch.int32:
        return t
    return t.view(torch.int16)


def _taps(cfg):
    B, H, E, R = cfg.batch, cfg.hidden_size, cfg.num_experts, cfg.router_hidden
    dt = cfg.torch_dtype
    f = lambda *s: torch.full(s, float("nan"), device=DEV, dtype=dt)
    i32 = lambda *s: torch.full(s, -7, device=DEV, dtype=torch.int32)
    return dict(attention_premix=f(B, 1, cfg.num_heads * cfg.head_dim), router_logits=f(B, 1, E + 1),
                expert_classes=i32(B, 1), bucket_offsets=i32(E + 1), bucket_ids=i32(B),
                mlp_neurons=f(B, cfg.moe_intermediate_size), mlp_output=f(B, 1, H))


def _one(cfg, lens):
    B, H, R = cfg.batch, cfg.hidden_size, cfg.router_hidden
    w = upload_weights(block_weights(cfg), cfg)
    inp = block_inputs(cfg)
    base = {k: inp[k].to(DEV).contiguous() for k in ("K", "V", "conv_state", "prev_hs")}
    x, s_in = inp["x"].to(DEV), inp["s_in"].to(DEV)
    outs = []
    for mode in ("workspace", "noalloc"):
        cache = {k: v.clone() for k, v in base.items()}
        cache["cache_len"] = list(lens)
        cache["cache_len_dev"] = torch.tensor(lens, dtype=torch.int32, device=DEV)
        xo = torch.full((B, 1, H), float("nan"), device=DEV)
        so = torch.full((B, 1, R), float("nan"), device=DEV, dtype=cfg.torch_dtype)
        taps = _taps(cfg)
        print(f"[gpu] decode {mode} cfg={cfg.name} B={B} lens[:4]={list(lens)[:4]}", flush=True)
        if mode == "workspace":
            ws = torch.empty(Z.zaya_block_workspace_bytes(cfg, B, 1, True), dtype=torch.uint8, device=DEV)
            Z.zaya_block_decode(cfg, w, B, x, s_in, xo, so, cache, taps, ws)
        else:
            Z.zaya_block_decode_noalloc(cfg, w, B, x, s_in, xo, so, cache, taps)
        torch.cuda.synchronize()
        outs.append(dict(x_out=xo, s_out=so, **{f"tap_{k}": v for k, v in taps.items()},
                         **{f"cache_{k}": cache[k] for k in ("K", "V", "conv_state", "prev_hs")}))
    a, b = outs
    assert torch.isfinite(a["x_out"]).all()
    # bucket ids and neurons are defined for the routed tokens only (the first
    # bucket_offsets[E] rows); the rest of those taps holds whatever the buffers held
    n = int(a["tap_bucket_offsets"][-1])
    assert n == int(b["tap_bucket_offsets"][-1])
    for k in ("tap_bucket_ids", "tap_mlp_neurons"):
        a[k], b[k] = a[k][:n], b[k][:n]
    for k in a:
        assert torch.equal(_bits(a[k]), _bits(b[k])), f"{cfg.name}: {k} differs between the two entry points"
    print(f"{cfg.name}: {len(a)} tensors bit-identical", flush=True)


def test_noalloc_decode_equals_workspace_decode_twice():
    # the decode workload (64 sequences over 8192 cached tokens), then a smaller step
    big = CONFIGS["decode"]
    _one(big, [big.kv_len] * big.batch)
    small = CONFIGS["decode"].replace(name="decode_noalloc_small", batch=5, kv_len=333)
    _one(small, [333, 0, 64, 65, 200])


def test_noalloc_rejects_steps_beyond_its_array():
    cfg = CONFIGS["decode"].replace(name="decode_noalloc_big", batch=128)
    need = Z.zaya_block_workspace_bytes(cfg, cfg.batch, 1, True)
    assert need > Z.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(1, device=DEV)
    with pytest.raises(Z.ZayaError) as e:  # rejected before anything else is looked at
        Z.zaya_block_decode_noalloc(cfg, {}, cfg.batch, t, t, t, t, None)
    assert e.value.code == -4 and "static array" in str(e.value)
