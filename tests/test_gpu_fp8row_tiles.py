"""fp8 weights with per-row scales (widened to bf16 in registers) on the
256-token tiles, where a wave owns two weight fragments, against the fp64
oracle: routing bit-exact outside near-ties, permutation exact, outputs
within the bf16 tolerance. Shapes put 200-300 rows on every expert, with a
ragged tail, both weight layouts and both call sequences."""

import pytest

import mixture_experts_layer_40_amd as moe
import synth
from gpu_parity import check_outputs, check_permutation, check_route, oracle_route, run_steps, say

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, d, E, K, I, S, Is, layout, fused
    ("fp8row_tiles_a", 1000, 256, 16, 4, 192, 1, 128, "tiled", True),
    ("fp8row_tiles_b", 777, 320, 8, 3, 256, 0, 0, "rows", False),
    ("fp8row_tiles_c", 1200, 192, 12, 2, 128, 2, 64, "rows", True),
]


@pytest.mark.parametrize("name,T,d,E,K,I,S,Is,layout,fused", CASES, ids=[c[0] for c in CASES])
def test_fp8_row_weights_on_large_tiles(name, T, d, E, K, I, S, Is, layout, fused):
    spec = synth.scaled_config("v3_decode_fp8", name=name, seed=20261206 + T, T=T, d=d, E=E, K=K,
                               I=I, S=S, Is=Is)
    say(f"[fp8row] {name}: T={T} d={d} E={E} K={K} I={I} S={S} Is={Is} rows/expert={T * K / E:.0f} "
        f"layout={layout} fused={fused}")
    inp = synth.make_inputs(spec, "cuda")
    layer = moe.MoELayer(spec, inp, layout=layout, fused=fused, shared_stream=False)
    layer, res = run_steps(spec, inp, bias=inp["bias"], layer=layer)
    r, _ = oracle_route(spec, inp["x"], inp["wr"], inp["bias"])
    n_near = check_route(spec, r, res["idx"], res["gate"], res["load"])
    check_permutation(spec, res["idx"], res["offsets"], res["perm"])
    e_y = check_outputs(spec, layer, inp, res, r)["y_err"]
    say(f"[fp8row] {name}: near-ties={n_near} y_err/rms={e_y:.3e}")
