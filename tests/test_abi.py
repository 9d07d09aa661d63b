"""The C-ABI library on the host: it loads, exports every function include/zaya.h
declares, and rejects bad arguments with the documented status codes before anything
touches a device. No call here reaches a kernel launch: every argument set fails host
validation (the pointers are dummies that are never dereferenced)."""
import ctypes as C
import os
import re

import pytest

import sparse_moe_block_amd as Z
from zaya_synth import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zaya.h")
FAKE = 0x7F0000001000  # a 4 KiB-aligned dummy address, never dereferenced by validation


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(Z.LIB_PATH):
        from sparse_moe_block_amd import build as B
        B.build(verbose=False)
    return Z.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\**\s*(zaya_[a-z_]+)\s*\(", text, flags=re.M)))


def header_define(name):
    m = re.search(rf"#define\s+{name}\s+(\d+)", open(HEADER).read())
    return int(m.group(1))


def test_every_declared_function_is_exported(L):
    names = declared_functions()
    assert {"zaya_block_prefill", "zaya_block_decode", "zaya_stack_forward"} <= set(names)
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, f"declared in include/zaya.h but not exported: {missing}"


def test_abi_version_and_stage_names(L):
    assert Z.abi_version() == header_define("ZAYA_ABI_VERSION")
    n = header_define("ZAYA_N_STAGES")
    assert n == Z.N_STAGES
    names = [Z.zaya_stage_name(k) for k in range(n)]
    assert len(set(names)) == n and all(names)
    for code, name in Z.STATUS.items():
        assert L.zaya_status_str(code).decode() == name
    assert L.zaya_status_str(-99).decode() == "ZAYA_UNKNOWN"


def test_stage_event_count_is_checked(L):
    arr = (C.c_void_p * 3)(FAKE, FAKE, FAKE)
    assert L.zaya_set_stage_events(arr, 3) == -1
    assert "events" in L.zaya_last_error().decode()
    assert L.zaya_set_stage_events(None, 0) == 0


def test_workspace_queries(L):
    for name in ("tiny", "prefill", "decode", "longctx"):
        cfg = CONFIGS[name]
        S = 1 if cfg.decode else cfg.seq
        n = Z.zaya_block_workspace_bytes(cfg, cfg.batch, S, cfg.decode)
        assert n > 0 and n % 256 == 0
    st = CONFIGS["stack"]
    assert Z.zaya_stack_workspace_bytes(st, st.batch, st.seq) > Z.zaya_block_workspace_bytes(st, st.batch, st.seq)
    # unsupported shapes and decode with S != 1 give 0
    assert Z.zaya_block_workspace_bytes(CONFIGS["prefill"].replace(head_dim=96), 1, 8) == 0
    assert Z.zaya_block_workspace_bytes(CONFIGS["decode"], 4, 2, True) == 0
    assert Z.zaya_block_workspace_bytes(CONFIGS["prefill"], 0, 8) == 0


BAD_CONFIGS = [
    (dict(head_dim=96), -2, "head_dim"),
    (dict(num_heads=6, num_kv_heads=2), -2, "n_heads"),  # group of 3
    (dict(rope_dim=63), -2, "rope_dim"),
    (dict(rope_dim=256), -2, "rope_dim"),
    (dict(conv_k=4), -2, "conv_k"),
    (dict(conv_k=2, act_dtype="f32", head_dim=128, num_heads=16, num_kv_heads=2), -2, "LDS"),
    (dict(num_experts=32), -2, "n_experts"),
    (dict(hidden_size=2000), -2, "hidden"),
    (dict(moe_intermediate_size=2000), -2, "expert_inter"),
    (dict(router_hidden=128), -2, "router_hidden"),
    (dict(rms_norm_eps=0.0), -2, "rms_eps"),
]


def _args(zcfg, nb, ns, **over):
    """Dummy but non-NULL arguments for zaya_block_prefill; `over` replaces some."""
    a = dict(cfg=C.byref(Z.block_config(zcfg)), w=C.byref(Z.BlockWeights(*([FAKE] * len(Z.WEIGHT_FIELDS)))), B=nb, S=ns,
             x=FAKE, s_in=FAKE + (1 << 32), x_out=FAKE + (2 << 32), s_out=FAKE + (3 << 32), cache=None, taps=None,
             ws=FAKE + (4 << 32), ws_bytes=1 << 40, stream=None)
    a.update(over)
    return a


def _prefill(L, a):
    return L.zaya_block_prefill(a["cfg"], a["w"], a["B"], a["S"], a["x"], a["s_in"], a["x_out"], a["s_out"],
                                a["cache"], a["taps"], a["ws"], a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("over,code,word", BAD_CONFIGS)
def test_unsupported_configs_are_rejected(L, over, code, word):
    cfg = CONFIGS["prefill"].replace(**over)
    rc = _prefill(L, _args(cfg, 1, 8, ws_bytes=0))
    assert rc == code, (rc, L.zaya_last_error())
    assert word in L.zaya_last_error().decode()


def test_argument_errors_have_their_codes(L):
    cfg = CONFIGS["prefill"]
    need = Z.zaya_block_workspace_bytes(cfg, 2, 16)
    cases = [
        (dict(cfg=None), -1),
        (dict(w=None), -1),
        (dict(w=C.byref(Z.BlockWeights(*([FAKE] * 26 + [None] + [FAKE] * (len(Z.WEIGHT_FIELDS) - 27))))), -1),
        (dict(B=0), -1),
        (dict(S=-3), -1),
        (dict(x=None), -1),
        (dict(x_out=None), -1),
        (dict(s_out=None), -1),
        (dict(x_out=FAKE + 64), -6),                           # x_out overlaps x
        (dict(s_in=FAKE + (3 << 32) + 2), -6),                 # router state in/out overlap
        (dict(ws=None, ws_bytes=need), -4),
        (dict(ws_bytes=need - 1), -4),
        (dict(ws=FAKE + (4 << 32) + 128, ws_bytes=need), -4),  # not 256-byte aligned
    ]
    for over, code in cases:
        a = _args(cfg, 2, 16, **over)
        if "ws_bytes" not in over:
            a["ws_bytes"] = 0  # an empty workspace keeps every case short of a launch
        rc = _prefill(L, a)
        assert rc == code, (over, rc, L.zaya_last_error())
        assert L.zaya_last_error().decode()


def test_bad_dtype(L):
    cfg = CONFIGS["prefill"]
    bc = Z.block_config(cfg)
    bc.act_dtype = 7
    rc = _prefill(L, _args(cfg, 1, 8, cfg=C.byref(bc), ws_bytes=0))
    assert rc == -3
    bc = Z.block_config(cfg)
    bc.expert_format = 5
    assert _prefill(L, _args(cfg, 1, 8, cfg=C.byref(bc), ws_bytes=0)) == -3


def test_fp8_experts_validation(L):
    # FP8 experts need bf16 activations and both row-scale tensors
    f32 = CONFIGS["tiny"].replace(expert_format="fp8")
    assert _prefill(L, _args(f32, 1, 8, ws_bytes=0)) == -3
    assert "BF16" in L.zaya_last_error().decode()
    cfg = CONFIGS["decode_fp8"]
    fields = [FAKE] * len(Z.WEIGHT_FIELDS)
    fields[Z.WEIGHT_FIELDS.index("W_dn_scale")] = None
    rc = _prefill(L, _args(cfg, 1, 8, w=C.byref(Z.BlockWeights(*fields)), ws_bytes=0))
    assert rc == -1 and "scale" in L.zaya_last_error().decode()
    # with the scales present, validation reaches the workspace check
    assert _prefill(L, _args(cfg, 1, 8, ws_bytes=0)) == -4
    # act-format experts ignore the scale pointers
    fields = [FAKE] * len(Z.WEIGHT_FIELDS)
    fields[Z.WEIGHT_FIELDS.index("W_gu_scale")] = fields[Z.WEIGHT_FIELDS.index("W_dn_scale")] = None
    assert _prefill(L, _args(CONFIGS["prefill"], 1, 8, w=C.byref(Z.BlockWeights(*fields)), ws_bytes=0)) == -4


def test_two_stage_conv_validation(L):
    # conv_k 2 needs the grouped stage's weight and bias; conv_k 3 ignores them
    cfg = CONFIGS["prefill"].replace(conv_k=2)
    for name in ("conv2_w", "conv2_b"):
        fields = [FAKE] * len(Z.WEIGHT_FIELDS)
        fields[Z.WEIGHT_FIELDS.index(name)] = None
        rc = _prefill(L, _args(cfg, 1, 8, w=C.byref(Z.BlockWeights(*fields)), ws_bytes=0))
        assert rc == -1 and "conv2" in L.zaya_last_error().decode()
        assert _prefill(L, _args(CONFIGS["prefill"], 1, 8, w=C.byref(Z.BlockWeights(*fields)), ws_bytes=0)) == -4
    assert _prefill(L, _args(cfg, 1, 8, ws_bytes=0)) == -4


def test_cache_bounds_are_checked(L):
    cfg = CONFIGS["decode"]
    lens = (C.c_int32 * 3)(10, 100, 5)
    cache = Z.CcaCache(FAKE, FAKE + (5 << 32), 100, FAKE + (6 << 32), FAKE + (7 << 32),
                       C.cast(lens, C.POINTER(C.c_int32)), None)
    bw = Z.BlockWeights(*([FAKE] * len(Z.WEIGHT_FIELDS)))
    rc = L.zaya_block_decode(C.byref(Z.block_config(cfg)), C.byref(bw), 3, FAKE, FAKE + (1 << 32), FAKE + (2 << 32),
                             FAKE + (3 << 32), C.byref(cache), None, FAKE + (4 << 32), 0, None)
    assert rc == -5 and "cache_len[1]" in L.zaya_last_error().decode()
    lens[1] = -1
    rc = L.zaya_block_decode(C.byref(Z.block_config(cfg)), C.byref(bw), 3, FAKE, FAKE + (1 << 32), FAKE + (2 << 32),
                             FAKE + (3 << 32), C.byref(cache), None, FAKE + (4 << 32), 0, None)
    assert rc == -5
    # decode without a cache
    rc = L.zaya_block_decode(C.byref(Z.block_config(cfg)), C.byref(bw), 3, FAKE, FAKE + (1 << 32), FAKE + (2 << 32),
                             FAKE + (3 << 32), None, None, FAKE + (4 << 32), 0, None)
    assert rc == -1
    # in bounds: validation goes on to the workspace check (0 bytes given)
    lens[1] = 99
    rc = L.zaya_block_decode(C.byref(Z.block_config(cfg)), C.byref(bw), 3, FAKE, FAKE + (1 << 32), FAKE + (2 << 32),
                             FAKE + (3 << 32), C.byref(cache), None, FAKE + (4 << 32), 0, None)
    assert rc == -4


def test_ring_cache_validation(L):
    bw = Z.BlockWeights(*([FAKE] * len(Z.WEIGHT_FIELDS)))
    lens = (C.c_int32 * 3)(500, 7, 0)  # a ring may hold sequences longer than its cap

    def decode(cfg, cap, ring=1):
        cache = Z.CcaCache(FAKE, FAKE + (5 << 32), cap, FAKE + (6 << 32), FAKE + (7 << 32),
                           C.cast(lens, C.POINTER(C.c_int32)), None, ring)
        return L.zaya_block_decode(C.byref(Z.block_config(cfg)), C.byref(bw), 3, FAKE, FAKE + (1 << 32),
                                   FAKE + (2 << 32), FAKE + (3 << 32), C.byref(cache), None, FAKE + (4 << 32), 0,
                                   None)

    win = CONFIGS["decode"].replace(sliding_window=100)
    assert decode(win, 101) == -4  # valid: stops at the empty workspace
    assert decode(win, 101, ring=0) == -5  # the same lengths overflow a linear cache
    assert decode(CONFIGS["decode"], 101) == -5 and "window" in L.zaya_last_error().decode()
    assert decode(win, 100) == -5 and "cap" in L.zaya_last_error().decode()
    # prefill into a ring: fresh sequences only
    cache = Z.CcaCache(FAKE, FAKE + (5 << 32), 101, FAKE + (6 << 32), FAKE + (7 << 32),
                       C.cast(lens, C.POINTER(C.c_int32)), None, 1)
    rc = _prefill(L, _args(win.replace(batch=3, seq=16, decode=False), 3, 16, cache=C.byref(cache), ws_bytes=0))
    assert rc == -5 and "fresh" in L.zaya_last_error().decode()
    lens[0] = lens[1] = 0
    assert _prefill(L, _args(win.replace(batch=3, seq=16, decode=False), 3, 16, cache=C.byref(cache),
                             ws_bytes=0)) == -4


def test_stack_validation(L):
    cfg = CONFIGS["stack"]
    bw = (Z.BlockWeights * cfg.num_layers)(*[Z.BlockWeights(*([FAKE] * len(Z.WEIGHT_FIELDS)))
                                             for _ in range(cfg.num_layers)])
    sw = Z.StackWeights(FAKE, FAKE, FAKE, FAKE, C.cast(bw, C.POINTER(Z.BlockWeights)))

    def call(sc, swt=sw, ids=FAKE, logits=FAKE + (1 << 32), ws=FAKE + (2 << 32), ws_bytes=0):
        return L.zaya_stack_forward(C.byref(sc), C.byref(swt), 4, 16, ids, logits, None, None, ws, ws_bytes, None)

    sc = Z.StackConfig(Z.block_config(cfg), 0, cfg.vocab_size)
    assert call(sc) == -2
    sc = Z.StackConfig(Z.block_config(cfg), cfg.num_layers, cfg.vocab_size)
    assert call(sc, ids=None) == -1
    assert call(sc, swt=Z.StackWeights(FAKE, None, FAKE, FAKE, C.cast(bw, C.POINTER(Z.BlockWeights)))) == -1
    assert call(sc) == -4  # everything else valid: the empty workspace is what stops it
    bad = Z.StackConfig(Z.block_config(cfg.replace(head_dim=80)), cfg.num_layers, cfg.vocab_size)
    assert call(bad) == -2
    # the head stores four logits per lane: a vocabulary that is not a multiple of 4 is
    # rejected before any launch (and has no workspace size)
    for v in (262145, 1002, 3):
        assert call(Z.StackConfig(Z.block_config(cfg), cfg.num_layers, v)) == -2
        assert "multiple of 4" in L.zaya_last_error().decode()
        assert Z.zaya_stack_workspace_bytes(cfg.replace(vocab_size=v), 4, 16) == 0
    assert Z.zaya_stack_workspace_bytes(cfg.replace(vocab_size=262272), 4, 16) > 0
    # hybrid stacks: window_layers in {0, 1, 2}
    assert call(Z.StackConfig(Z.block_config(cfg.replace(sliding_window=64)), cfg.num_layers, cfg.vocab_size, 1)) == -4
    bad = Z.StackConfig(Z.block_config(cfg), cfg.num_layers, cfg.vocab_size, 3)
    assert call(bad) == -2 and "window_layers" in L.zaya_last_error().decode()
    assert Z.zaya_stack_workspace_bytes(cfg.replace(window_layers=3), 4, 16) == 0
    # the workspace covers the windowed and the full-attention blocks
    hyb = cfg.replace(sliding_window=64, window_layers=1)
    assert Z.zaya_stack_workspace_bytes(hyb, 4, 2048) >= max(
        Z.zaya_stack_workspace_bytes(cfg, 4, 2048), Z.zaya_stack_workspace_bytes(cfg.replace(sliding_window=64), 4, 2048))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(Z, "LIB_PATH", str(tmp_path / "absent.so"))
    monkeypatch.setattr(Z, "_lib", None)
    with pytest.raises(Z.ZayaLibraryMissing):
        Z.zaya_block_workspace_bytes(CONFIGS["tiny"], 1, 8)


def test_probe_arguments_are_checked(L):
    flops = C.c_double(0.0)
    assert L.zaya_probe_mfma_bf16(0, 10, C.c_void_p(FAKE), None, C.byref(flops)) == -1
    assert L.zaya_probe_mfma_bf16(4, 0, C.c_void_p(FAKE), None, C.byref(flops)) == -1
    assert L.zaya_probe_mfma_bf16(4, 10, None, None, C.byref(flops)) == -1
    assert L.zaya_probe_hbm_read(C.c_void_p(FAKE), 4096, 0, C.c_void_p(FAKE), None) == -1
    assert L.zaya_probe_hbm_read(C.c_void_p(FAKE + 8), 4096, 4, C.c_void_p(FAKE), None) == -1  # misaligned
    assert L.zaya_probe_hbm_read(C.c_void_p(FAKE), 4100, 4, C.c_void_p(FAKE), None) == -1  # not 16-byte whole
    assert L.zaya_probe_hbm_read(None, 4096, 4, C.c_void_p(FAKE), None) == -1


def test_noalloc_decode_rejects_oversized_steps_before_any_device_call(L):
    """The allocation-free decode checks the configuration and that the step fits its
    static array before it looks up the array on a device (nothing here has a GPU)."""
    cfg = CONFIGS["decode"].replace(batch=128)
    need = Z.zaya_block_workspace_bytes(cfg, 128, 1, True)
    assert need > header_define("ZAYA_NOALLOC_SCRATCH_BYTES") == Z.NOALLOC_SCRATCH_BYTES
    assert Z.zaya_block_workspace_bytes(CONFIGS["decode"], 64, 1, True) <= Z.NOALLOC_SCRATCH_BYTES
    rc = L.zaya_block_decode_noalloc(C.byref(Z.block_config(cfg)), None, 128, FAKE, FAKE, FAKE, FAKE, None, None,
                                     None)
    assert rc == -4 and "static array" in L.zaya_last_error().decode()
    bad = Z.block_config(cfg.replace(head_dim=80))
    assert L.zaya_block_decode_noalloc(C.byref(bad), None, 4, FAKE, FAKE, FAKE, FAKE, None, None, None) == -2
    assert L.zaya_block_decode_noalloc(C.byref(Z.block_config(cfg)), None, 0, FAKE, FAKE, FAKE, FAKE, None, None,
                                       None) == -1


def test_pack_experts_validation(L):
    """zaya_pack_experts: a known expert format, no NULL pointer, packed buffers that
    overlap neither the row-major ones nor each other. Every case fails before a launch."""
    cfg = CONFIGS["prefill"]
    E, H, I = cfg.num_experts, cfg.hidden_size, cfg.moe_intermediate_size
    ngu, ndn = E * 2 * I * H * 2, E * H * I * 2
    gu, dn = FAKE, FAKE + ngu  # two dummy row-major buffers, back to back
    pgu, pdn = FAKE + ngu + ndn, FAKE + 2 * ngu + ndn
    pack = lambda c, *p: L.zaya_pack_experts(C.byref(Z.block_config(c)), *[C.c_void_p(v) if v else None for v in p],
                                             None)
    bad = Z.block_config(cfg)
    bad.expert_format = 7
    assert L.zaya_pack_experts(C.byref(bad), C.c_void_p(gu), C.c_void_p(dn), C.c_void_p(pgu), C.c_void_p(pdn),
                               None) == -3
    assert pack(cfg, gu, dn, None, pdn) == -1
    assert pack(cfg, gu, dn, dn + 4096, pdn) == -6  # packed W_gu over the row-major W_dn
    assert pack(cfg, gu, dn, pgu, pgu + ngu - 2) == -6  # the two packed buffers overlap
    assert pack(cfg.replace(hidden_size=2000), gu, dn, pgu, pdn) == -2
