"""ZAYA1 decoder-block forward on MI355X (gfx950): Python binding of libzaya.so.

Every function here only marshals arguments into the C ABI of ``include/zaya.h``;
all of the block's arithmetic runs in the library's HIP kernels. PyTorch tensors
are used as device buffers (their ``data_ptr()``), and the current torch stream is
the default stream for launches.

If the shared library is not built, importing still works but every entry point
raises ``ZayaLibraryMissing``: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Mapping, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzaya.so")

ZAYA_F32, ZAYA_BF16 = 0, 1
ZAYA_EXPERTS_ACT, ZAYA_EXPERTS_FP8_E4M3, ZAYA_EXPERTS_ACT_PACKED, ZAYA_EXPERTS_FP8_E4M3_PACKED = 0, 1, 2, 3
# (expert_format, expert_layout) of a configuration -> the C enum
_EXPERT_FORMATS = {("act", "rows"): ZAYA_EXPERTS_ACT, ("fp8", "rows"): ZAYA_EXPERTS_FP8_E4M3,
                   ("act", "packed"): ZAYA_EXPERTS_ACT_PACKED, ("fp8", "packed"): ZAYA_EXPERTS_FP8_E4M3_PACKED}
STATUS = {0: "ZAYA_OK", -1: "ZAYA_EINVAL", -2: "ZAYA_ESHAPE", -3: "ZAYA_EDTYPE", -4: "ZAYA_EWORKSPACE",
          -5: "ZAYA_ECACHE", -6: "ZAYA_EALIAS", -7: "ZAYA_EHIP"}


class ZayaLibraryMissing(RuntimeError):
    pass


class ZayaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class BlockConfig(C.Structure):
    _fields_ = [("hidden", C.c_int), ("n_heads", C.c_int), ("n_kv_heads", C.c_int), ("head_dim", C.c_int),
                ("rope_dim", C.c_int), ("rope_theta", C.c_float), ("conv_k", C.c_int), ("n_experts", C.c_int),
                ("expert_inter", C.c_int), ("router_hidden", C.c_int), ("sliding_window", C.c_int),
                ("rms_eps", C.c_float), ("act_dtype", C.c_int), ("expert_format", C.c_int)]


WEIGHT_FIELDS = ("ln1_g", "W_qkv", "conv_w", "conv_b", "temp", "W_o", "a_hsb", "a_hss", "a_rb", "a_rs", "ln2_g",
                 "r_Wd", "r_bd", "r_rss", "r_norm_g", "r_W1", "r_b1", "r_W2", "r_b2", "r_Wout", "bal_bias", "W_gu",
                 "W_dn", "m_hsb", "m_hss", "m_rb", "m_rs", "W_gu_scale", "W_dn_scale", "conv2_w", "conv2_b")


class BlockWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in WEIGHT_FIELDS]


class CcaCache(C.Structure):
    _fields_ = [("K", C.c_void_p), ("V", C.c_void_p), ("cap", C.c_int), ("conv_state", C.c_void_p),
                ("prev_hs", C.c_void_p), ("cache_len", C.POINTER(C.c_int32)), ("cache_len_dev", C.c_void_p),
                ("ring", C.c_int)]


TAP_FIELDS = ("attention_norm_output", "attention_queries", "attention_keys", "attention_values", "attention_premix",
              "attention_output", "layer_mid", "mlp_norm_output", "router_logits", "expert_classes", "expert_indices",
              "expert_weights", "bucket_offsets", "bucket_ids", "mlp_neurons", "routed_output", "mlp_output",
              "layer_output", "router_state")


class Taps(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in TAP_FIELDS]


class StackConfig(C.Structure):
    _fields_ = [("block", BlockConfig), ("n_layers", C.c_int), ("vocab", C.c_int), ("window_layers", C.c_int)]


class StackWeights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("emb_shift", C.c_void_p), ("emb_scale", C.c_void_p),
                ("final_g", C.c_void_p), ("blocks", C.POINTER(BlockWeights))]


_lib = None


def lib():
    """The loaded libzaya.so (raises ZayaLibraryMissing if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ZayaLibraryMissing(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                                     "python sparse_moe_block_amd/build.py")
        L = C.CDLL(LIB_PATH)
        vp, i, sz = C.c_void_p, C.c_int, C.c_size_t
        L.zaya_block_workspace_bytes.argtypes = [C.POINTER(BlockConfig), i, i, i]
        L.zaya_block_workspace_bytes.restype = sz
        L.zaya_block_prefill.argtypes = [C.POINTER(BlockConfig), C.POINTER(BlockWeights), i, i, vp, vp, vp, vp,
                                         C.POINTER(CcaCache), C.POINTER(Taps), vp, sz, vp]
        L.zaya_block_prefill.restype = i
        L.zaya_block_decode.argtypes = [C.POINTER(BlockConfig), C.POINTER(BlockWeights), i, vp, vp, vp, vp,
                                        C.POINTER(CcaCache), C.POINTER(Taps), vp, sz, vp]
        L.zaya_block_decode.restype = i
        L.zaya_block_decode_noalloc.argtypes = [C.POINTER(BlockConfig), C.POINTER(BlockWeights), i, vp, vp, vp, vp,
                                                C.POINTER(CcaCache), C.POINTER(Taps), vp]
        L.zaya_block_decode_noalloc.restype = i
        L.zaya_stack_workspace_bytes.argtypes = [C.POINTER(StackConfig), i, i]
        L.zaya_stack_workspace_bytes.restype = sz
        L.zaya_stack_forward.argtypes = [C.POINTER(StackConfig), C.POINTER(StackWeights), i, i, vp, vp,
                                         C.POINTER(CcaCache), C.POINTER(Taps), vp, sz, vp]
        L.zaya_stack_forward.restype = i
        L.zaya_pack_experts.argtypes = [C.POINTER(BlockConfig), vp, vp, vp, vp, vp]
        L.zaya_pack_experts.restype = i
        L.zaya_last_error.restype = C.c_char_p
        L.zaya_status_str.argtypes = [i]
        L.zaya_status_str.restype = C.c_char_p
        L.zaya_abi_version.restype = i
        L.zaya_set_stage_events.argtypes = [C.POINTER(C.c_void_p), i]
        L.zaya_set_stage_events.restype = i
        L.zaya_stage_name.argtypes = [i]
        L.zaya_stage_name.restype = C.c_char_p
        L.zaya_probe_mfma_bf16.argtypes = [i, i, vp, vp, C.POINTER(C.c_double)]
        L.zaya_probe_mfma_bf16.restype = i
        L.zaya_probe_hbm_read.argtypes = [vp, sz, i, vp, vp]
        L.zaya_probe_hbm_read.restype = i
        _lib = L
    return _lib


# ----------------------------------------------------------------------------- marshalling

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr() if hasattr(t, "data_ptr") else int(t)


def block_config(cfg) -> BlockConfig:
    """C config from any object with the ZayaConfig attribute names."""
    return BlockConfig(cfg.hidden_size, cfg.num_heads, cfg.num_kv_heads, cfg.head_dim, cfg.rope_dim,
                       float(cfg.rope_theta), getattr(cfg, "conv_k", 3), cfg.num_experts,
                       cfg.moe_intermediate_size, cfg.router_hidden, getattr(cfg, "sliding_window", -1),
                       float(getattr(cfg, "rms_norm_eps", 1e-5)),
                       ZAYA_BF16 if cfg.act_dtype == "bf16" else ZAYA_F32,
                       _EXPERT_FORMATS[(getattr(cfg, "expert_format", "act"), getattr(cfg, "expert_layout", "rows"))])


def block_weights(w: Mapping) -> BlockWeights:
    """Weights by field name; the two expert scale tensors are optional (fp8 experts)."""
    return BlockWeights(*[_ptr(w.get(n)) for n in WEIGHT_FIELDS])


def cca_cache(cache: Optional[Mapping]):
    """(struct, keep-alive) from dict(K, V, conv_state, prev_hs, cache_len [host int list/tensor],
    optional cache_len_dev [device int32 tensor], optional ring [bool: K/V slots hold position p
    at p % cap])."""
    if cache is None:
        return None, None
    lens = [int(v) for v in cache["cache_len"]]
    arr = (C.c_int32 * len(lens))(*lens)
    st = CcaCache(_ptr(cache["K"]), _ptr(cache["V"]), int(cache["K"].shape[2]), _ptr(cache["conv_state"]),
                  _ptr(cache["prev_hs"]), C.cast(arr, C.POINTER(C.c_int32)), _ptr(cache.get("cache_len_dev")),
                  int(bool(cache.get("ring", False))))
    return st, arr


def taps_struct(taps: Optional[Mapping]):
    if not taps:
        return None
    bad = set(taps) - set(TAP_FIELDS)
    if bad:
        raise KeyError(f"unknown taps {sorted(bad)}")
    return Taps(*[_ptr(taps.get(n)) for n in TAP_FIELDS])


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def _check(rc: int):
    if rc != 0:
        raise ZayaError(rc, lib().zaya_last_error().decode())


def _ref(s):
    return C.byref(s) if s is not None else None


# ----------------------------------------------------------------------------- entry points

def zaya_block_workspace_bytes(cfg, B: int, S: int, decode: bool = False) -> int:
    return int(lib().zaya_block_workspace_bytes(C.byref(block_config(cfg)), B, S, int(bool(decode))))


def zaya_stack_workspace_bytes(cfg, B: int, S: int) -> int:
    sc = StackConfig(block_config(cfg), cfg.num_layers, cfg.vocab_size, getattr(cfg, "window_layers", 0))
    return int(lib().zaya_stack_workspace_bytes(C.byref(sc), B, S))


def zaya_block_prefill(cfg, w: Mapping, B: int, S: int, x, s_in, x_out, s_out, cache=None, taps=None,
                       workspace=None, stream=None) -> None:
    """One block forward (see ``zaya_block_prefill`` in include/zaya.h)."""
    L = lib()
    cs, keep = cca_cache(cache)
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = L.zaya_block_prefill(C.byref(block_config(cfg)), C.byref(block_weights(w)), B, S, _ptr(x), _ptr(s_in),
                              _ptr(x_out), _ptr(s_out), _ref(cs), _ref(taps_struct(taps)), _ptr(workspace), ws_bytes,
                              _stream(stream))
    del keep
    _check(rc)


def zaya_block_decode(cfg, w: Mapping, B: int, x, s_in, x_out, s_out, cache, taps=None, workspace=None,
                      stream=None) -> None:
    """One decode step (see ``zaya_block_decode`` in include/zaya.h)."""
    L = lib()
    cs, keep = cca_cache(cache)
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = L.zaya_block_decode(C.byref(block_config(cfg)), C.byref(block_weights(w)), B, _ptr(x), _ptr(s_in),
                             _ptr(x_out), _ptr(s_out), _ref(cs), _ref(taps_struct(taps)), _ptr(workspace), ws_bytes,
                             _stream(stream))
    del keep
    _check(rc)


def zaya_block_decode_noalloc(cfg, w: Mapping, B: int, x, s_in, x_out, s_out, cache, taps=None,
                              stream=None) -> None:
    """One decode step in the library's static scratch array, no workspace (see
    ``zaya_block_decode_noalloc`` in include/zaya.h)."""
    L = lib()
    cs, keep = cca_cache(cache)
    rc = L.zaya_block_decode_noalloc(C.byref(block_config(cfg)), C.byref(block_weights(w)), B, _ptr(x), _ptr(s_in),
                                     _ptr(x_out), _ptr(s_out), _ref(cs), _ref(taps_struct(taps)), _stream(stream))
    del keep
    _check(rc)


NOALLOC_SCRATCH_BYTES = 64 << 20  # ZAYA_NOALLOC_SCRATCH_BYTES


def zaya_stack_forward(cfg, sw: Mapping, blocks: Sequence[Mapping], B: int, S: int, ids, logits,
                       caches: Optional[Sequence[Mapping]] = None, taps: Optional[Sequence[Mapping]] = None,
                       workspace=None, stream=None) -> None:
    """Embedding, ``cfg.num_layers`` blocks, final norm and tied lm_head (see include/zaya.h)."""
    L = lib()
    sc = StackConfig(block_config(cfg), cfg.num_layers, cfg.vocab_size, getattr(cfg, "window_layers", 0))
    bw = (BlockWeights * len(blocks))(*[block_weights(b) for b in blocks])
    swt = StackWeights(_ptr(sw["embed"]), _ptr(sw["emb_shift"]), _ptr(sw["emb_scale"]), _ptr(sw["final_g"]),
                       C.cast(bw, C.POINTER(BlockWeights)))
    keep = []
    cptr = None
    if caches is not None:
        structs = []
        for c in caches:
            s_, k_ = cca_cache(c)
            structs.append(s_)
            keep.append(k_)
        carr = (CcaCache * len(structs))(*structs)
        cptr = C.cast(carr, C.POINTER(CcaCache))
        keep.append(carr)
    tptr = None
    if taps is not None:
        tarr = (Taps * len(taps))(*[taps_struct(t) or Taps() for t in taps])
        tptr = C.cast(tarr, C.POINTER(Taps))
        keep.append(tarr)
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = L.zaya_stack_forward(C.byref(sc), C.byref(swt), B, S, _ptr(ids), _ptr(logits), cptr, tptr, _ptr(workspace),
                              ws_bytes, _stream(stream))
    del keep
    _check(rc)


def zaya_pack_experts(cfg, W_gu, W_dn, W_gu_packed, W_dn_packed, stream=None) -> None:
    """Write the packed expert layout (see ``zaya_pack_experts`` in include/zaya.h)."""
    _check(lib().zaya_pack_experts(C.byref(block_config(cfg)), _ptr(W_gu), _ptr(W_dn), _ptr(W_gu_packed),
                                   _ptr(W_dn_packed), _stream(stream)))


def packed_expert_weights(cfg, w: Mapping, stream=None) -> dict:
    """A copy of the weight dict whose W_gu / W_dn are new device buffers holding the
    packed layout of the given row-major ones (for expert_layout "packed"; act-dtype or
    FP8 codes as the configuration's expert_format says)."""
    import torch
    out = dict(w)
    out["W_gu"] = torch.empty_like(w["W_gu"])
    out["W_dn"] = torch.empty_like(w["W_dn"])
    zaya_pack_experts(cfg, w["W_gu"], w["W_dn"], out["W_gu"], out["W_dn"], stream)
    return out


N_STAGES = 11


def zaya_set_stage_events(events: Optional[Sequence[int]]) -> None:
    """Record the given hipEvent_t handles (N_STAGES + 1 of them) around each stage of the
    block calls made by this thread; None switches recording off."""
    if not events:
        _check(lib().zaya_set_stage_events(None, 0))
        return
    arr = (C.c_void_p * len(events))(*events)
    _check(lib().zaya_set_stage_events(arr, len(events)))


def zaya_stage_name(k: int) -> str:
    return lib().zaya_stage_name(k).decode()


def zaya_probe_mfma_bf16(n_wg: int, iters: int, sink_ptr: int, stream: int) -> float:
    """Enqueue the matrix-core probe (see include/zaya.h); returns the flops it performs."""
    flops = C.c_double(0.0)
    _check(lib().zaya_probe_mfma_bf16(n_wg, iters, C.c_void_p(sink_ptr), C.c_void_p(stream), C.byref(flops)))
    return float(flops.value)


def zaya_probe_hbm_read(src_ptr: int, nbytes: int, n_wg: int, sink_ptr: int, stream: int) -> None:
    """Enqueue the HBM read probe (see include/zaya.h)."""
    _check(lib().zaya_probe_hbm_read(C.c_void_p(src_ptr), nbytes, n_wg, C.c_void_p(sink_ptr), C.c_void_p(stream)))


def abi_version() -> int:
    return int(lib().zaya_abi_version())


__all__ = ["zaya_block_prefill", "zaya_block_decode", "zaya_stack_forward", "zaya_pack_experts", "packed_expert_weights", "zaya_block_workspace_bytes",
           "zaya_stack_workspace_bytes", "ZayaError", "ZayaLibraryMissing", "lib", "abi_version", "LIB_PATH",
           "TAP_FIELDS", "WEIGHT_FIELDS", "zaya_set_stage_events", "zaya_stage_name", "N_STAGES",
           "zaya_probe_mfma_bf16", "zaya_probe_hbm_read"]
