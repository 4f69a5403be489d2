"""The measurement probes of libmla_peaks.so compute what their header says: the streaming
read's per-thread XORs fold to the XOR of the whole buffer, the copy is exact, and the matrix-op
loop's per-thread sums equal the closed form for all-equal operands."""
import numpy as np
import pytest
import torch

from helpers import need_gpu

pytestmark = pytest.mark.gpu


def test_read_probe_xor_and_copy_probe():
    need_gpu()
    from head_latent_attention_amd import measure as M
    rng = np.random.default_rng(11)
    n = (3 << 20) // 4 + 36          # not a multiple of the grid stride: the tail loop runs
    host = rng.integers(-2**31, 2**31, size=n, dtype=np.int64).astype(np.int32)
    src = torch.from_numpy(host).cuda()
    for n_wg in (7, 64):
        sink = torch.zeros(n_wg * 256, dtype=torch.int32, device="cuda")
        M.peak_read(src, sink, n_wg)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(sink.cpu().numpy())
        assert got == np.bitwise_xor.reduce(host), n_wg
        dst = torch.zeros_like(src)
        M.peak_copy(src, dst, n_wg)
        torch.cuda.synchronize()
        assert torch.equal(dst, src), n_wg


@pytest.mark.parametrize("shape", [16, 32])
def test_mfma_probe_closed_form(shape):
    need_gpu()
    from head_latent_attention_amd import measure as M
    iters, v = 100, 1.5               # bf16(1.5) = 1.5 exactly; every sum stays an exact float
    for n_wg, threads in ((3, 256), (2, 512)):
        sink = torch.zeros(n_wg * threads, dtype=torch.float32, device="cuda")
        M.peak_mfma_bf16(shape, iters, v, sink, n_wg, threads)
        torch.cuda.synchronize()
        per_op, elems = (32, 16) if shape == 16 else (16, 64)
        expect = iters * per_op * v * v * elems
        assert torch.all(sink == expect), (shape, n_wg, threads, sink[:4].tolist(), expect)
