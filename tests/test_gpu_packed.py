"""Packed expert weights (zaya_pack_experts; ZAYA_EXPERTS_ACT_PACKED, ZAYA_EXPERTS_FP8_E4M3_PACKED).

The packed layout only reorders the weight bytes: the layout itself is checked element
by element against its definition in include/zaya.h (an index map built here from
that text), and a block run on packed weights must equal the same block on row-major
weights bit for bit, every output and every tap, since the kernels do the same
arithmetic in the same order. The row-major runs are the path the oracle parity tests
cover at small widths; the full-size workloads run packed."""
import numpy as np
import pytest
import torch

import sparse_moe_block_amd as Z
from tests.zaya_harness import DEV, BlockRun
from zaya_synth import CONFIGS, block_inputs, block_weights

pytestmark = pytest.mark.gpu


def _gateup_rows(I: int) -> np.ndarray:
    """Row of W_gu [2I, H] stored at position (group j, row q) of one expert's packed
    groups: 16-row blocks b = q // 16 alternate gate (even b) and up (odd b), block b
    covering activation columns 64 j + 16 (b // 2) .. + 15."""
    rows = []
    for j in range(I // 64):
        for q in range(128):
            b, w = q // 16, q % 16
            rows.append((I if b % 2 else 0) + 64 * j + 16 * (b // 2) + w)
    return np.array(rows)


def _pack_ref(W: torch.Tensor, rows: np.ndarray) -> torch.Tensor:
    """[E, N, K] row-major -> the packed byte order: per expert, groups of 128 rows (in
    the order `rows` gives), each group slice after slice (128 bytes of every row of
    the group), rows in order within a slice."""
    E, N, K = W.shape
    per = 128 // W.element_size()  # elements in a 128-byte slice
    g = W[:, torch.as_tensor(rows), :]  # [E, N, K] in packed row order
    g = g.reshape(E, N // 128, 128, K // per, per)  # e, group, row, slice, elements
    return g.permute(0, 1, 3, 2, 4).contiguous().reshape(-1)


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_packed_layout_matches_its_definition(act):
    cfg = CONFIGS["tiny"].replace(name="pack_layout", act_dtype=act, num_experts=3, hidden_size=256,
                                  moe_intermediate_size=192, expert_layout="packed")
    E, H, I = cfg.num_experts, cfg.hidden_size, cfg.moe_intermediate_size
    dt = cfg.torch_dtype
    g = torch.Generator().manual_seed(3)
    Wgu = torch.randn((E, 2 * I, H), generator=g).to(dt)
    Wdn = torch.randn((E, H, I), generator=g).to(dt)
    Pgu = torch.full_like(Wgu, float("nan"), device=DEV)
    Pdn = torch.full_like(Wdn, float("nan"), device=DEV)
    print(f"[gpu] pack layout act={act} E={E} H={H} I={I}", flush=True)
    Z.zaya_pack_experts(cfg, Wgu.to(DEV), Wdn.to(DEV), Pgu, Pdn)
    torch.cuda.synchronize()
    ref_gu = _pack_ref(Wgu, _gateup_rows(I))
    ref_dn = _pack_ref(Wdn, np.arange(H))
    assert torch.equal(Pgu.cpu().reshape(-1), ref_gu)
    assert torch.equal(Pdn.cpu().reshape(-1), ref_dn)


def test_packed_fp8_layout_matches_its_definition():
    """FP8 codes: rows in blocks of 16, each block stored 64-byte step after step."""
    cfg = CONFIGS["tiny"].replace(name="pack_layout8", act_dtype="bf16", num_experts=3, hidden_size=256,
                                  moe_intermediate_size=192, expert_format="fp8", expert_layout="packed")
    E, H, I = cfg.num_experts, cfg.hidden_size, cfg.moe_intermediate_size
    g = torch.Generator().manual_seed(5)
    Wgu = torch.randint(0, 256, (E, 2 * I, H), generator=g, dtype=torch.uint8)
    Wdn = torch.randint(0, 256, (E, H, I), generator=g, dtype=torch.uint8)
    Pgu = torch.zeros_like(Wgu, device=DEV)
    Pdn = torch.zeros_like(Wdn, device=DEV)
    print(f"[gpu] pack layout fp8 E={E} H={H} I={I}", flush=True)
    Z.zaya_pack_experts(cfg, Wgu.to(DEV), Wdn.to(DEV), Pgu, Pdn)
    torch.cuda.synchronize()
    ref = lambda W: W.reshape(E, W.shape[1] // 16, 16, W.shape[2] // 64, 64).permute(0, 1, 3, 2, 4).reshape(-1)
    assert torch.equal(Pgu.cpu().reshape(-1), ref(Wgu))
    assert torch.equal(Pdn.cpu().reshape(-1), ref(Wdn))


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.detach().contiguous().view(torch.uint8).cpu()


def _same_run(cfg_rowmajor):
    """The block on row-major and on packed weights, same inputs: outputs and taps equal
    bit for bit."""
    cfg_p = cfg_rowmajor.replace(expert_layout="packed")
    w = block_weights(cfg_rowmajor)
    inp = block_inputs(cfg_rowmajor)
    a = BlockRun(cfg_rowmajor, w_host=w, inp=inp).run()
    b = BlockRun(cfg_p, w_host=w, inp=inp).run()
    assert b.w["W_gu"].data_ptr() != a.w["W_gu"].data_ptr()
    assert torch.equal(_bits(a.x_out), _bits(b.x_out)), "layer output differs"
    assert torch.equal(_bits(a.s_out), _bits(b.s_out)), "router state differs"
    n = int(a.taps["bucket_offsets"][-1])  # routed rows: the bucket-order taps hold only these
    for k in a.taps:
        ta, tb = a.taps[k], b.taps[k]
        if k in ("bucket_ids", "mlp_neurons"):
            ta, tb = ta[:n], tb[:n]
        assert torch.equal(_bits(ta), _bits(tb)), f"tap {k} differs"
    return a


def test_packed_prefill_bit_identical():
    # 600 tokens over 16 experts: row tiles of 128 with ragged tails, every expert group
    _same_run(CONFIGS["prefill"].replace(name="packed_pre", batch=1, seq=600, expert_layout="rows"))


def test_packed_decode_bit_identical():
    _same_run(CONFIGS["decode"].replace(name="packed_dec", kv_len=300, expert_layout="rows"))


def test_packed_fp32_bit_identical():
    _same_run(CONFIGS["tiny"].replace(name="packed_tiny", seq=100, batch=2))


def test_packed_fp8_decode_bit_identical():
    _same_run(CONFIGS["decode_fp8"].replace(name="packed_dec8", kv_len=300, expert_layout="rows"))


def test_packed_fp8_prefill_bit_identical():
    _same_run(CONFIGS["prefill"].replace(name="packed_pre8", batch=1, seq=600, expert_format="fp8",
                                         expert_layout="rows"))
