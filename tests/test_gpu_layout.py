"""The tiled weight layout: moe_pack_weights moves every byte to the place
include/libmoe.h documents (checked bit for bit against a NumPy relocation
written from that description), and a layer called with the tiled weights
gives bit-identical results to the same layer on the row-major weights (the
relocation changes which bytes a load fetches, not the arithmetic)."""

import numpy as np
import pytest
import torch

import mixture_experts_layer_40_amd as moe
import synth
from gpu_parity import run_steps, say

pytestmark = pytest.mark.gpu


def _tiled_reference(a, b, wb):
    """Relocate [G, N, C*wb] byte arrays as the header describes."""
    G, N, Cb = a.shape
    if b is not None:
        rows = np.empty((G, 2 * N, Cb), dtype=np.uint8)
        for c in range(N // 16):
            rows[:, 32 * c:32 * c + 16] = a[:, 16 * c:16 * c + 16]
            rows[:, 32 * c + 16:32 * c + 32] = b[:, 16 * c:16 * c + 16]
    else:
        rows = a
    R = rows.shape[1]
    stage = 64 * wb                       # bytes of one 64-column stage of a row
    aw = 2 * wb                           # 16-byte pieces per lane per tile
    r4 = rows.reshape(G, R // 32, 32, Cb // stage, stage)
    out = np.empty((G, R // 32, Cb // stage, aw, 64, 16), dtype=np.uint8)
    for lane in range(64):
        r, g = lane % 32, lane // 32
        for v in range(aw):
            lo = 32 * g * wb + 16 * v
            out[:, :, :, v, lane, :] = r4[:, :, r, :, lo:lo + 16]
    return out.reshape(G, -1)


def _bytes(t):
    return t.contiguous().view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("wd", ["bf16", "fp8"])
@pytest.mark.parametrize("G,N,C", [(3, 48, 128), (1, 64, 192), (2, 2048 // 16, 64)])
def test_pack_matches_documented_layout(wd, G, N, C):
    gen = torch.Generator(device="cpu").manual_seed(G * 1000 + N + C)
    if wd == "bf16":
        mk = lambda n: torch.randn((G, n, C), generator=gen).to(torch.bfloat16).cuda()
        wb = 2
    else:
        mk = lambda n: torch.randint(0, 256, (G, n, C), generator=gen, dtype=torch.uint8).cuda()
        wb = 1
    w1, w3 = mk(N), mk(N)
    gu = moe.pack_gate_up(w1, w3, wd)
    want = _tiled_reference(_bytes(w1).reshape(G, N, -1), _bytes(w3).reshape(G, N, -1), wb)
    assert np.array_equal(_bytes(gu).reshape(G, -1), want)
    if N % 32 == 0:
        w2 = mk(N)
        dn = moe.pack_down(w2, wd)
        want = _tiled_reference(_bytes(w2).reshape(G, N, -1), None, wb)
        assert np.array_equal(_bytes(dn).reshape(G, -1), want)


def _cfg(base, **kw):
    name = base + "_" + "_".join(f"{k}{v}" for k, v in sorted(kw.items()))
    return synth.scaled_config(base, name=name, **kw)


LAYOUT_CASES = {
    "v3_gemm": _cfg("v3_prefill_bf16", T=1000, d=1024, E=32, K=4, I=384, Is=256),
    "dsmoe_small": _cfg("dsmoe2024_bf16", T=300, d=256, E=64, K=6, I=192, Is=128),
    "fp8_multi": _cfg("v3_decode_fp8", T=700, d=256, E=16, K=4, I=192, S=2, Is=64),
    "fp8_small": _cfg("v3_decode_fp8", T=64, d=512, E=64, K=8, I=256, Is=256),
    "bm256": _cfg("v3_prefill_bf16", T=2000, d=256, E=16, K=4, I=256, Is=128),
}


@pytest.mark.parametrize("name", list(LAYOUT_CASES))
def test_tiled_layer_is_bit_identical_to_rows(name):
    spec = LAYOUT_CASES[name]
    say(f"[layout] {name}")
    inp = synth.make_inputs(spec, "cuda")
    rows = moe.MoELayer(spec, inp, layout="rows", shared_stream=False)
    tiled = moe.MoELayer(spec, inp, layout="tiled", shared_stream=False)
    assert rows.layout == "rows" and tiled.layout == "tiled"
    _, a = run_steps(spec, inp, bias=inp["bias"], layer=rows)
    _, b = run_steps(spec, inp, bias=inp["bias"], layer=tiled)
    TK = spec.T * spec.K
    assert torch.equal(rows.out_slots[:TK], tiled.out_slots[:TK])
    if spec.S > 0:
        assert torch.equal(rows.y_shared, tiled.y_shared)
    assert torch.equal(a["y"], b["y"])
