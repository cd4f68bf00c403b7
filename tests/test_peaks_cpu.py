"""libmoe_peaks.so (include/moe_peaks.h) on the host: it loads, exports every
declared symbol, reports the work of a loop call in closed form, and rejects
bad arguments before any launch (no GPU is touched here)."""

import ctypes
import re
from pathlib import Path

import pytest

from mixture_experts_layer_40_amd import _lib as L
from mixture_experts_layer_40_amd import peaks as pk

ROOT = Path(__file__).resolve().parents[1]


def test_exports_every_declared_symbol():
    header = (ROOT / "include" / "moe_peaks.h").read_text()
    declared = set(re.findall(r"^(?:int|double)\s+(moe_(?:peak|probe)_\w+)\(", header, re.M))
    assert declared == set(pk.EXPORTED)
    lib = pk.load_library()
    for name in declared:
        assert hasattr(lib, name)


@pytest.mark.parametrize("kind,per_instr,per_iter", [
    (pk.MOE_PEAK_MFMA_BF16_32X32X16, 32 * 32 * 16 * 2, 16),
    (pk.MOE_PEAK_MFMA_BF16_16X16X32, 16 * 16 * 32 * 2, 32),
    (pk.MOE_PEAK_MFMA_FP8_32X32X64, 32 * 32 * 64 * 2, 16),
    (pk.MOE_PEAK_MFMA_FP8_16X16X128, 16 * 16 * 128 * 2, 32),
    (pk.MOE_PEAK_FMA_F32, 64 * 2, 32),
])
def test_loop_flops_closed_form(kind, per_instr, per_iter):
    # blocks x 8 waves x iters x instructions per wave-iteration x flops each
    for blocks, iters in ((1, 1), (3, 7), (1024, 4096)):
        assert pk.moe_peak_mfma_flops(kind, blocks, iters) == blocks * 8 * iters * per_iter * per_instr


def test_bad_arguments_are_rejected_on_the_host():
    lib = pk.load_library()
    fake = ctypes.c_void_p(0x1000)
    odd = ctypes.c_void_p(0x1008)
    assert lib.moe_peak_mfma_flops(5, 1, 1) == 0.0
    assert lib.moe_peak_mfma_flops(0, 0, 1) == 0.0
    assert lib.moe_peak_mfma(5, 1, 1, fake, None) == L.MOE_ERR_SHAPE
    assert lib.moe_peak_mfma(-1, 1, 1, fake, None) == L.MOE_ERR_SHAPE
    assert lib.moe_peak_mfma(0, 0, 1, fake, None) == L.MOE_ERR_SHAPE
    assert lib.moe_peak_mfma(0, 1, 0, fake, None) == L.MOE_ERR_SHAPE
    assert lib.moe_peak_mfma(0, 1, 1, None, None) == L.MOE_ERR_NULL
    rd, cp = lib.moe_peak_stream_read, lib.moe_peak_stream_copy
    assert rd(None, 16, 1, fake, None) == L.MOE_ERR_NULL
    assert rd(fake, 16, 1, None, None) == L.MOE_ERR_NULL
    assert rd(fake, 0, 1, fake, None) == L.MOE_ERR_SHAPE
    assert rd(fake, 24, 1, fake, None) == L.MOE_ERR_SHAPE
    assert rd(odd, 16, 1, fake, None) == L.MOE_ERR_SHAPE
    assert rd(fake, 16, 0, fake, None) == L.MOE_ERR_SHAPE
    rn = lib.moe_peak_stream_read_nt
    assert rn(None, 16, 1, fake, None) == L.MOE_ERR_NULL
    assert rn(fake, 16, 1, None, None) == L.MOE_ERR_NULL
    assert rn(fake, 24, 1, fake, None) == L.MOE_ERR_SHAPE
    assert rn(odd, 16, 1, fake, None) == L.MOE_ERR_SHAPE
    assert rn(fake, 16, 0, fake, None) == L.MOE_ERR_SHAPE
    l2 = lib.moe_peak_l2_read
    assert l2(None, 65536, 1, 1, fake, None) == L.MOE_ERR_NULL
    assert l2(fake, 65536, 1, 1, None, None) == L.MOE_ERR_NULL
    assert l2(fake, 32768, 1, 1, fake, None) == L.MOE_ERR_SHAPE      # not a multiple of 64 KB
    assert l2(fake, 0, 1, 1, fake, None) == L.MOE_ERR_SHAPE
    assert l2(fake, 65536, 0, 1, fake, None) == L.MOE_ERR_SHAPE
    assert l2(fake, 65536, 1, 0, fake, None) == L.MOE_ERR_SHAPE
    assert l2(odd, 65536, 1, 1, fake, None) == L.MOE_ERR_SHAPE
    assert cp(None, fake, 16, 1, None) == L.MOE_ERR_NULL
    assert cp(fake, odd, 16, 1, None) == L.MOE_ERR_SHAPE
    assert cp(fake, ctypes.c_void_p(0x1010), 32, 1, None) == L.MOE_ERR_SHAPE   # overlap
    assert cp(fake, ctypes.c_void_p(0x2000), 40, 1, None) == L.MOE_ERR_SHAPE
    pr = lib.moe_probe_fp8_mfma
    assert pr(None, fake, fake, fake, 1, None) == L.MOE_ERR_NULL
    assert pr(fake, fake, fake, None, 1, None) == L.MOE_ERR_NULL
    assert pr(fake, fake, fake, fake, 0, None) == L.MOE_ERR_SHAPE
    assert pr(odd, fake, fake, fake, 1, None) == L.MOE_ERR_SHAPE
