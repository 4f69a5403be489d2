"""ctypes binding of libmla_peaks.so (include/mla_peaks.h): measured streaming-read, copy and
bf16 matrix-op peaks on the current GPU, for the benchmark's rooflines.  Argument marshalling
and timing only; the probes are HIP kernels."""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int, c_size_t, c_void_p

import torch

PEAKS_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_peaks.so")
SYMBOLS = ("mla_peak_read", "mla_peak_copy", "mla_peak_mfma_bf16")
_lib = None


def load(path: str = PEAKS_LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise ImportError(f"{path} is not built (run __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        lib.mla_peak_read.argtypes = [c_void_p, c_size_t, c_void_p, c_int, c_void_p]
        lib.mla_peak_copy.argtypes = [c_void_p, c_void_p, c_size_t, c_int, c_void_p]
        lib.mla_peak_mfma_bf16.argtypes = [c_int, c_int, c_float, c_void_p, c_int, c_int, c_void_p]
        for name in SYMBOLS:
            getattr(lib, name).restype = c_int
        _lib = lib
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} returned {rc} ({'invalid argument' if rc == -1 else 'HIP error'})")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def peak_read(src: torch.Tensor, sink: torch.Tensor, n_wg: int) -> None:
    assert src.is_cuda and src.is_contiguous() and sink.dtype == torch.int32 and sink.numel() >= n_wg * 256
    _check(load().mla_peak_read(src.data_ptr(), src.numel() * src.element_size(), sink.data_ptr(), n_wg, _stream()),
           "mla_peak_read")


def peak_copy(src: torch.Tensor, dst: torch.Tensor, n_wg: int) -> None:
    assert src.is_cuda and dst.is_cuda and src.is_contiguous() and dst.is_contiguous()
    assert src.numel() * src.element_size() == dst.numel() * dst.element_size()
    _check(load().mla_peak_copy(src.data_ptr(), dst.data_ptr(), src.numel() * src.element_size(), n_wg, _stream()),
           "mla_peak_copy")


def peak_mfma_bf16(shape: int, iters: int, value: float, sink: torch.Tensor, n_wg: int, threads: int) -> None:
    assert sink.dtype == torch.float32 and sink.numel() >= n_wg * threads
    _check(load().mla_peak_mfma_bf16(shape, iters, value, sink.data_ptr(), n_wg, threads, _stream()),
           "mla_peak_mfma_bf16")


def _best_ms(fn, reps: int) -> float:
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    fn()
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return min(a.elapsed_time(b) for a, b in ev)


def measure(read_bytes: int = 2 << 30, copy_bytes: int = 1 << 30, reps: int = 5) -> dict:
    """Best-of-reps rates of one launch of each probe, timed with HIP events on the launch
    stream, over a few launch shapes: streaming read GB/s, copy GB/s (bytes read + written),
    bf16 matrix-op TFLOP/s for both op shapes."""
    out = {}
    src = torch.empty(read_bytes // 4, dtype=torch.int32, device="cuda").fill_(1)
    best = (0.0, 0)
    for n_wg in (1024, 2048, 4096):
        sink = torch.empty(n_wg * 256, dtype=torch.int32, device="cuda")
        ms = _best_ms(lambda: peak_read(src, sink, n_wg), reps)
        best = max(best, (read_bytes / (ms * 1e-3) / 1e9, n_wg))
    out["read_GBps"], out["read_workgroups"] = round(best[0], 1), best[1]
    del src
    a = torch.empty(copy_bytes // 4, dtype=torch.int32, device="cuda").fill_(2)
    b = torch.empty_like(a)
    best = (0.0, 0)
    for n_wg in (1024, 2048, 4096):
        ms = _best_ms(lambda: peak_copy(a, b, n_wg), reps)
        best = max(best, (2 * copy_bytes / (ms * 1e-3) / 1e9, n_wg))
    out["copy_GBps"], out["copy_workgroups"] = round(best[0], 1), best[1]
    del a, b
    for shape, iters in ((16, 20000), (32, 10000)):
        flop_per_wave_iter = 4 * 2 * (16 * 16 * 32 if shape == 16 else 32 * 32 * 16)
        best = (0.0, "")
        for n_wg, threads in ((256, 256), (512, 256), (256, 512), (512, 512)):
            sink = torch.empty(n_wg * threads, dtype=torch.float32, device="cuda")
            ms = _best_ms(lambda: peak_mfma_bf16(shape, iters, 1.0, sink, n_wg, threads), reps)
            flops = n_wg * (threads // 64) * iters * flop_per_wave_iter
            best = max(best, (flops / (ms * 1e-3) / 1e12, f"{n_wg}x{threads}"))
        out[f"mfma_bf16_{shape}_TFLOPs"], out[f"mfma_bf16_{shape}_launch"] = round(best[0], 1), best[1]
    return out
