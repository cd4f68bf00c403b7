"""Seeded random shapes through every path, each checked against the fp64
oracle to the same bar as the hand-picked cases: routing bit-exact outside
near-ties, permutation exact, outputs within the tolerance of their dtype.

The shapes are drawn once from a fixed seed (so a failure names a
reproducible case): expert counts from 1 to 256 (including counts that are
not multiples of 16), top-K from 1 to min(E, 8), hidden and intermediate
sizes of 1 to 8 multiples of 64 (of 128 for the block-scaled fp8 path), 0, 1
or 2 shared experts, 1 to 700 tokens, a few past 4096 (the fused router),
both weight layouts and both call sequences of the bf16 path; a second set
draws the routing options (node-limited groups, the three gate
normalisations) and the pre-MoE RMSNorm with the residual."""

import numpy as np
import pytest

import synth
from gpu_parity import (check_outputs, check_permutation, check_route, oracle_route, run_steps,
                        say)
from test_gpu_fp8block import _layer_check as fp8_block_layer_check
from test_gpu_norm import _check_norm_layer

pytestmark = pytest.mark.gpu

PATHS = ("bf16", "fp8row", "f32", "fp8block")


def _draw(n=64, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        path = PATHS[i % len(PATHS)]
        q = 128 if path == "fp8block" else 64
        E = int(rng.choice([1, 2, 3, 8, 16, 20, 64, 128, 256]))
        K = int(rng.integers(1, min(E, 8) + 1))
        T = int(rng.integers(4096, 4400)) if (path == "bf16" and i % 8 == 0) else int(rng.integers(1, 701))
        d = q * int(rng.integers(1, 5 if T > 4000 else 9))
        I = q * int(rng.integers(1, 7))
        S = int(rng.integers(0, 3))
        Is = q * int(rng.integers(1, 5)) if S else 0
        kw = dict(T=T, d=d, E=E, K=K, I=I, S=S, Is=Is)
        if path == "bf16":
            base = "dsmoe2024_bf16" if rng.random() < 0.3 else "v3_prefill_bf16"
            layout = "tiled" if rng.random() < 0.5 else "rows"
            fused = bool(rng.random() < 0.5) if layout == "rows" else True
        elif path == "fp8row":
            base, layout, fused = "v3_decode_fp8", ("tiled" if rng.random() < 0.5 else "rows"), None
        elif path == "f32":
            base, layout, fused = "tiny_f32", "rows", None
            kw.update(x_std=1.0, w_std=0.05)
        else:
            base, layout, fused = "v3_prefill_fp8b", "tiled", True
        name = f"sweep{i:02d}_{path}"
        spec = synth.scaled_config(base, name=name, seed=20260300 + i, **kw)
        cases.append((name, spec, layout, fused))
    return cases


CASES = _draw()


@pytest.mark.parametrize("name,spec,layout,fused", CASES, ids=[c[0] for c in CASES])
def test_random_shape_matches_oracle(name, spec, layout, fused):
    say(f"[sweep] {name}: T={spec.T} d={spec.d} E={spec.E} K={spec.K} I={spec.I} S={spec.S} "
        f"Is={spec.Is} layout={layout} fused={fused} {spec.weight_dtype}/{spec.act_dtype}")
    inp = synth.make_inputs(spec, "cuda")
    if name.endswith("fp8block"):
        n_near, e_y, _ = fp8_block_layer_check(spec, inp)
    else:
        import mixture_experts_layer_40_amd as moe
        layer = moe.MoELayer(spec, inp, layout=layout, fused=fused, shared_stream=False)
        layer, res = run_steps(spec, inp, bias=inp["bias"], layer=layer)
        r, _ = oracle_route(spec, inp["x"], inp["wr"], inp["bias"])
        n_near = check_route(spec, r, res["idx"], res["gate"], res["load"])
        check_permutation(spec, res["idx"], res["offsets"], res["perm"])
        e_y = check_outputs(spec, layer, inp, res, r)["y_err"]
    say(f"[sweep] {name}: near-ties={n_near} y_err/rms={e_y:.3e}")


def _draw_routing(n=32, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        base = ("v3_prefill_bf16", "dsmoe2024_bf16", "v3_decode_fp8")[i % 3]
        E = int(rng.choice([8, 16, 32, 64, 128, 256]))
        K = int(rng.integers(1, min(E, 8) + 1))
        kw = dict(E=E, K=K, T=int(rng.integers(4096, 4300)) if i % 6 == 0 else int(rng.integers(1, 701)),
                  d=64 * int(rng.integers(1, 5)), I=64 * int(rng.integers(1, 5)),
                  norm=str(rng.choice(["selected", "one_plus", "none"])))
        S = int(rng.integers(0, 3))
        kw.update(S=S, Is=64 * int(rng.integers(1, 4)) if S else 0)
        groups = [G for G in (2, 4, 8, 16) if E % G == 0]
        if rng.random() < 0.6:
            G = int(rng.choice(groups))
            m_min = -(-K // (E // G))                      # M * E/G >= K
            kw.update(n_groups=G, topk_groups=int(rng.integers(m_min, G + 1)))
        else:
            kw.update(n_groups=0, topk_groups=0)
        norm_res = bool(rng.random() < 0.4)
        label = {"v3_prefill_bf16": "v3", "dsmoe2024_bf16": "dsmoe2024", "v3_decode_fp8": "fp8"}[base]
        name = f"route{i:02d}_{label}" + ("_norm" if norm_res else "")
        spec = synth.scaled_config(base, name=name, seed=20260400 + i, **kw)
        cases.append((name, spec, norm_res))
    return cases


ROUTE_CASES = _draw_routing()


@pytest.mark.parametrize("name,spec,norm_res", ROUTE_CASES, ids=[c[0] for c in ROUTE_CASES])
def test_random_routing_options_match_oracle(name, spec, norm_res):
    say(f"[sweep] {name}: T={spec.T} d={spec.d} E={spec.E} K={spec.K} groups={spec.n_groups}/"
        f"{spec.topk_groups} norm={spec.norm} S={spec.S} pre-norm+residual={norm_res}")
    inp = synth.make_inputs(spec, "cuda")
    if norm_res:
        n_near, out = _check_norm_layer(spec, inp)
        e_y = out["y_err"]
    else:
        layer, res = run_steps(spec, inp, bias=inp["bias"])
        r, _ = oracle_route(spec, inp["x"], inp["wr"], inp["bias"])
        n_near = check_route(spec, r, res["idx"], res["gate"], res["load"])
        check_permutation(spec, res["idx"], res["offsets"], res["perm"])
        e_y = check_outputs(spec, layer, inp, res, r)["y_err"]
    say(f"[sweep] {name}: near-ties={n_near} y_err/rms={e_y:.3e}")
