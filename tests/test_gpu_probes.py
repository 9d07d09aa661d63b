"""The benchmark probes behind the measured ceilings: the HBM read probe must read every
16-byte chunk of its buffer exactly once (checked through the per-thread fold it writes,
recomputed on the host), and the matrix-core probe must run and report the flops its
launch shape implies."""
import numpy as np
import pytest
import torch

import sparse_moe_block_amd as Z

DEV = "cuda"


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes,n_wg", [(1 << 20, 4), ((1 << 20) + 48, 3), (16, 1)])
def test_read_probe_folds_every_chunk_once(nbytes, n_wg):
    rng = np.random.default_rng(nbytes + n_wg)
    host = rng.integers(0, 1 << 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    sink = torch.zeros(n_wg * 256, dtype=torch.float32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    Z.zaya_probe_hbm_read(buf.data_ptr(), nbytes, n_wg, sink.data_ptr(), stream)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    # thread t folds chunks t, t + T, t + 2T, ... (T = 256 n_wg threads): XOR of all words
    T = n_wg * 256
    chunks = host.reshape(-1, 4)
    want = np.zeros(T, dtype=np.uint32)
    for c in range(chunks.shape[0]):
        want[c % T] ^= np.bitwise_xor.reduce(chunks[c])
    np.testing.assert_array_equal(got, want)


@pytest.mark.gpu
def test_mfma_probe_runs_and_counts_flops():
    n_wg, iters = 8, 50
    sink = torch.full((n_wg * 256,), float("nan"), dtype=torch.float32, device=DEV)
    flops = Z.zaya_probe_mfma_bf16(n_wg, iters, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert flops == n_wg * 4 * iters * 8 * 2 * 32 * 32 * 16
    assert torch.isfinite(sink).all()
