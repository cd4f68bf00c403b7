"""Binding of libmoe_peaks.so (include/moe_peaks.h): achievable-peak probes.

The functions with the header's names marshal arguments only; measure_*
time a probe with HIP events on the current stream and return the rate it
sustained. They feed the "measured" column the benchmark reports beside the
published MI355X peaks; they compute nothing of the layer.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from ._lib import MOE_OK, MoEError, moe_status_string

PEAKS_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_peaks.so")

MOE_PEAK_MFMA_BF16_32X32X16 = 0
MOE_PEAK_MFMA_BF16_16X16X32 = 1
MOE_PEAK_MFMA_FP8_32X32X64 = 2
MOE_PEAK_MFMA_FP8_16X16X128 = 3
MOE_PEAK_FMA_F32 = 4
FORMS = {
    "bf16_32x32x16": MOE_PEAK_MFMA_BF16_32X32X16,
    "bf16_16x16x32": MOE_PEAK_MFMA_BF16_16X16X32,
    "fp8_32x32x64": MOE_PEAK_MFMA_FP8_32X32X64,
    "fp8_16x16x128": MOE_PEAK_MFMA_FP8_16X16X128,
    "f32_fma": MOE_PEAK_FMA_F32,
}
EXPORTED = ("moe_peak_mfma", "moe_peak_mfma_flops", "moe_peak_stream_read",
            "moe_peak_stream_read_nt", "moe_peak_l2_read", "moe_peak_stream_copy", "moe_probe_fp8_mfma")

_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmoe_peaks.so (built by mixture_experts_layer_40_amd.build);
    raises if it is missing: there is no fallback."""
    global _lib
    path = path or PEAKS_LIB_PATH
    if _lib is not None and path == PEAKS_LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m mixture_experts_layer_40_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.moe_peak_mfma.argtypes = [ctypes.c_int, I32, I32, P, P]
    lib.moe_peak_mfma.restype = ctypes.c_int
    lib.moe_peak_mfma_flops.argtypes = [ctypes.c_int, I32, I32]
    lib.moe_peak_mfma_flops.restype = ctypes.c_double
    lib.moe_peak_stream_read.argtypes = [P, SZ, I32, P, P]
    lib.moe_peak_stream_read.restype = ctypes.c_int
    lib.moe_peak_stream_read_nt.argtypes = [P, SZ, I32, P, P]
    lib.moe_peak_stream_read_nt.restype = ctypes.c_int
    lib.moe_peak_l2_read.argtypes = [P, SZ, I32, I32, P, P]
    lib.moe_peak_l2_read.restype = ctypes.c_int
    lib.moe_peak_stream_copy.argtypes = [P, P, SZ, I32, P]
    lib.moe_peak_stream_copy.restype = ctypes.c_int
    lib.moe_probe_fp8_mfma.argtypes = [P, P, P, P, I32, P]
    lib.moe_probe_fp8_mfma.restype = ctypes.c_int
    _lib = lib
    return lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(name, st):
    if st != MOE_OK:
        raise MoEError(name, st, moe_status_string(st))


def moe_peak_mfma(kind: int, blocks: int, iters: int, out: torch.Tensor):
    _check("moe_peak_mfma", load_library().moe_peak_mfma(kind, blocks, iters, out.data_ptr(),
                                                          _stream()))


def moe_peak_mfma_flops(kind: int, blocks: int, iters: int) -> float:
    return load_library().moe_peak_mfma_flops(kind, blocks, iters)


def moe_peak_stream_read(src: torch.Tensor, nbytes: int, blocks: int, out: torch.Tensor):
    _check("moe_peak_stream_read", load_library().moe_peak_stream_read(
        src.data_ptr(), nbytes, blocks, out.data_ptr(), _stream()))


def moe_peak_stream_read_nt(src: torch.Tensor, nbytes: int, blocks: int, out: torch.Tensor):
    _check("moe_peak_stream_read_nt", load_library().moe_peak_stream_read_nt(
        src.data_ptr(), nbytes, blocks, out.data_ptr(), _stream()))


def moe_peak_l2_read(src: torch.Tensor, region_bytes: int, blocks: int, iters: int,
                     out: torch.Tensor):
    _check("moe_peak_l2_read", load_library().moe_peak_l2_read(
        src.data_ptr(), region_bytes, blocks, iters, out.data_ptr(), _stream()))


def moe_peak_stream_copy(src: torch.Tensor, dst: torch.Tensor, nbytes: int, blocks: int):
    _check("moe_peak_stream_copy", load_library().moe_peak_stream_copy(
        src.data_ptr(), dst.data_ptr(), nbytes, blocks, _stream()))


def moe_probe_fp8_mfma(a: torch.Tensor, b: torch.Tensor, c: torch.Tensor, d: torch.Tensor):
    """D = A B^T + C by one fp8 MFMA per problem: a, b uint8 [n, 32, 64]
    (E4M3 codes; b holds B's columns as rows), c, d fp32 [n, 32, 32]."""
    n = a.shape[0]
    for t, shape in ((a, (n, 32, 64)), (b, (n, 32, 64)), (c, (n, 32, 32)), (d, (n, 32, 32))):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"moe_probe_fp8_mfma: expected a contiguous {shape} tensor")
    _check("moe_probe_fp8_mfma", load_library().moe_probe_fp8_mfma(
        a.data_ptr(), b.data_ptr(), c.data_ptr(), d.data_ptr(), n, _stream()))


def _time_ms(call, reps: int) -> float:
    call()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(reps):
        call()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def measure_mfma(form: str, blocks: int = 1024, iters: int = 2048, reps: int = 5) -> float:
    """TFLOP/s a loop of independent instructions of `form` sustains over
    `blocks` blocks of 8 waves."""
    kind = FORMS[form]
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    ms = _time_ms(lambda: moe_peak_mfma(kind, blocks, iters, out), reps)
    return moe_peak_mfma_flops(kind, blocks, iters) / (ms * 1e-3) / 1e12


def measure_stream(nbytes: int = 1 << 31, read_blocks: int = 4096,
                   copy_blocks: Optional[int] = None, reps: int = 5) -> dict:
    """GB/s of a 16-byte-load streaming read of `nbytes` (plain loads, and
    loads with the non-temporal hint) and of a streaming copy of `nbytes`
    (read + written bytes). The read runs best as a
    grid-stride loop over a few thousand blocks (6.1 TB/s on MI355X, against
    5.5 with one block per 32 KB chunk); the copy, by default, gets one
    block per chunk (5.4-5.5 TB/s, against 5.2-5.3 grid-stride)."""
    if copy_blocks is None:
        copy_blocks = max(1, min((nbytes + 32767) // 32768, 1 << 20))
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.view(torch.int32).random_()
    dst = torch.empty_like(src)
    out = torch.empty(read_blocks * 256, dtype=torch.int32, device="cuda")
    read_ms = _time_ms(lambda: moe_peak_stream_read(src, nbytes, read_blocks, out), reps)
    read_nt_ms = _time_ms(lambda: moe_peak_stream_read_nt(src, nbytes, read_blocks, out), reps)
    copy_ms = _time_ms(lambda: moe_peak_stream_copy(src, dst, nbytes, copy_blocks), reps)
    del src, dst, out
    return {"read_GBs": nbytes / (read_ms * 1e-3) / 1e9,
            "read_nt_GBs": nbytes / (read_nt_ms * 1e-3) / 1e9,
            "copy_GBs": 2.0 * nbytes / (copy_ms * 1e-3) / 1e9}


def measure_l2(region_bytes: int = 65536, blocks: int = 256, iters: int = 400,
               reps: int = 5) -> float:
    """GB/s of L2 hits into the CUs: each of `blocks` blocks (one per CU by
    default) re-reads its own 64 KB (over the 32 KB L1; 2 MB per XCD, under
    its 4 MB L2)."""
    src = torch.ones(region_bytes * blocks // 4, dtype=torch.int32, device="cuda")
    out = torch.empty(blocks * 512, dtype=torch.int32, device="cuda")
    ms = _time_ms(lambda: moe_peak_l2_read(src, region_bytes, blocks, iters, out), reps)
    del src, out
    return region_bytes * blocks * iters / (ms * 1e-3) / 1e9
