"""The achievable-peak probes on the GPU: the streaming reads (plain and
non-temporal loads) and the L2 read touch
every word (their per-thread XORs combine to the XOR of the buffer) and the
streaming copy is exact, on sizes that leave a ragged grid-stride tail; the
MFMA and FMA loops give finite, non-zero, run-to-run identical results and a
positive rate."""

import numpy as np
import pytest
import torch

from mixture_experts_layer_40_amd import peaks as pk
from gpu_parity import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n16,blocks", [(1, 1), (1000003, 64), (4 * 256 * 37 + 5, 37)])
def test_stream_read_and_copy_touch_every_word(n16, blocks):
    say(f"[peaks] stream n16={n16} blocks={blocks}")
    gen = torch.Generator(device="cpu").manual_seed(n16)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n16 * 4,), generator=gen, dtype=torch.int64)
    host = host.to(torch.int32)
    src = host.cuda()
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    pk.moe_peak_stream_read(src, n16 * 16, blocks, out)
    out_nt = torch.empty_like(out)
    pk.moe_peak_stream_read_nt(src, n16 * 16, blocks, out_nt)
    dst = torch.zeros_like(src)
    pk.moe_peak_stream_copy(src, dst, n16 * 16, blocks)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == want
    assert np.bitwise_xor.reduce(out_nt.cpu().numpy().view(np.uint32)) == want
    assert torch.equal(dst, src)


@pytest.mark.parametrize("blocks,region_kb,iters", [(1, 64, 1), (3, 128, 3)])
def test_l2_read_touches_every_word(blocks, region_kb, iters):
    say(f"[peaks] l2 read blocks={blocks} region={region_kb} KB iters={iters}")
    n32 = blocks * region_kb * 1024 // 4
    gen = torch.Generator(device="cpu").manual_seed(n32)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n32,), generator=gen, dtype=torch.int64).to(torch.int32)
    out = torch.empty(blocks * 512, dtype=torch.int32, device="cuda")
    pk.moe_peak_l2_read(host.cuda(), region_kb * 1024, blocks, iters, out)
    torch.cuda.synchronize()
    # every word is read `iters` times (odd), so the XORs combine to the buffer's
    assert np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) == \
        np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert pk.measure_l2(blocks=64, iters=20, reps=2) > 0


@pytest.mark.parametrize("form", list(pk.FORMS))
def test_loops_are_finite_and_deterministic(form):
    say(f"[peaks] loop {form}")
    kind = pk.FORMS[form]
    blocks, iters = 16, 64
    a = torch.empty(blocks * 512, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    pk.moe_peak_mfma(kind, blocks, iters, a)
    pk.moe_peak_mfma(kind, blocks, iters, b)
    torch.cuda.synchronize()
    assert torch.isfinite(a).all()
    assert (a != 0).any()
    assert torch.equal(a, b)
    assert pk.measure_mfma(form, blocks=256, iters=64, reps=2) > 0
