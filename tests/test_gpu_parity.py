"""GPU parity of the whole layer at sizes the oracle finishes in seconds.

Every case runs the HIP path through the C ABI on seeded synthetic inputs and
compares routing (bit-exact up to near-ties), the permutation (bit-exact), the
gathered rows (bit-exact), and the shared, routed and combined outputs (to the
tolerance of the activation dtype) with the fp64 oracle. The shapes span
several tiles with ragged tails, every router path (fused bf16, split-K bf16,
fp32), both score functions and gate normalisations, bf16 and fp8 weights,
and the degenerate cases (K = E, E not a multiple of 16, one token, E = 1).
"""

import numpy as np
import pytest
import torch

import mixture_experts_layer_40_amd as moe
import oracle
import synth
from gpu_parity import (check_outputs, check_permutation, check_route, f64, host, oracle_route,
                        run_steps, say)

pytestmark = pytest.mark.gpu


def _cfg(base, **kw):
    name = base + "_" + "_".join(f"{k}{v}" for k, v in sorted(kw.items()))
    return synth.scaled_config(base, name=name, **kw)


CASES = {
    # the fp32 workload itself
    "tiny_f32": synth.get_config("tiny_f32"),
    # fp32, ragged tokens, 24 experts, S=1
    "f32_ragged": _cfg("tiny_f32", T=77, d=192, E=24, K=3, I=128, Is=64, x_std=1.0, w_std=0.05),
    # 2024 layout: softmax, unnormalised gates, 2 shared experts, split-K router
    "dsmoe_small": _cfg("dsmoe2024_bf16", T=300, d=256, E=64, K=6, I=192, Is=128),
    # V3 routing with bias through the fused router (T >= 4096), ragged tiles
    "v3_fused": _cfg("v3_prefill_bf16", T=4100, d=128, E=256, K=8, I=128, Is=128),
    # multi-tile GEMMs in both axes, M_e ~ 125
    "v3_gemm": _cfg("v3_prefill_bf16", T=1000, d=1024, E=32, K=4, I=384, Is=256),
    # fp8 weights, decode-like token count
    "fp8_small": _cfg("v3_decode_fp8", T=64, d=512, E=64, K=8, I=256, Is=256),
    # fp8 weights with multi-tile token blocks and 2 shared experts
    "fp8_multi": _cfg("v3_decode_fp8", T=700, d=256, E=16, K=4, I=192, S=2, Is=64),
    # > 128 rows per expert: 256-token tiles, several per expert, ragged
    "bm256": _cfg("v3_prefill_bf16", T=2000, d=256, E=16, K=4, I=256, Is=128),
    "fp8_bm256": _cfg("v3_decode_fp8", T=1500, d=320, E=8, K=2, I=128, Is=64),
    # degenerate: K = E, E not a multiple of 16
    "k_eq_e": _cfg("v3_prefill_bf16", T=50, d=64, E=7, K=7, I=64, Is=64),
    "e20": _cfg("v3_prefill_bf16", T=129, d=64, E=20, K=5, I=64, Is=64),
    "one_token": _cfg("v3_prefill_bf16", T=1, d=128, E=256, K=8, I=64, Is=64),
    "one_expert": _cfg("v3_prefill_bf16", T=33, d=64, E=1, K=1, I=64, S=0, Is=0),
    # many slots per token: 64 of 256 experts (a wave's full record of
    # selections), all 256 (every expert holds every token; 5120 pairs, a
    # multi-chunk sort), and 64 under node-limited routing (4 of 8 groups)
    "k64": _cfg("v3_prefill_bf16", T=100, d=128, E=256, K=64, I=64, Is=64),
    "k_eq_e_256": _cfg("v3_prefill_bf16", T=20, d=64, E=256, K=256, I=64, Is=64),
    "k64_grouped": _cfg("v3_prefill_bf16", T=120, d=128, E=256, K=64, I=64, Is=64,
                        n_groups=8, topk_groups=4),
    # node-limited routing: split-K router, fused router (T >= 4096), softmax
    # scores, a single kept group
    "grouped_small": _cfg("v3_prefill_bf16", T=300, d=256, E=64, K=6, I=128, Is=128,
                          n_groups=8, topk_groups=3),
    "grouped_fused": _cfg("v3_grouped_bf16", T=4100, d=128, E=256, K=8, I=128, Is=128),
    "grouped_softmax": _cfg("dsmoe2024_bf16", T=200, d=128, E=64, K=6, I=128, Is=128,
                            n_groups=4, topk_groups=2),
    "grouped_m1": _cfg("v3_prefill_bf16", T=150, d=128, E=32, K=4, I=64, Is=64,
                       n_groups=4, topk_groups=1),
    # the routed slot rows held in bf16 (half their bytes) instead of fp32
    "v3_gemm_bf16_slots": _cfg("v3_prefill_bf16", T=1000, d=1024, E=32, K=4, I=384, Is=256,
                               slot_dtype="bf16"),
    "dsmoe_bf16_slots": _cfg("dsmoe2024_bf16", T=300, d=256, E=64, K=6, I=192, Is=128,
                             slot_dtype="bf16"),
    "fp8_bf16_slots": _cfg("v3_decode_fp8", T=700, d=256, E=16, K=4, I=192, S=2, Is=64,
                           slot_dtype="bf16"),
    # the "1 + sum" gate weighting, split-K and fused (with node-limited) routers
    "oneplus": _cfg("v3_prefill_bf16", T=400, d=256, E=64, K=6, I=128, Is=128, norm="one_plus"),
    "oneplus_grouped_fused": _cfg("v3_grouped_bf16", T=4096, d=128, E=256, K=8, I=64, Is=64,
                                  norm="one_plus"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_layer_parity(name):
    spec = CASES[name]
    say(f"[parity] {name}: {spec}")
    inp = synth.make_inputs(spec, "cuda")
    layer, res = run_steps(spec, inp, bias=inp["bias"])
    r, _ = oracle_route(spec, inp["x"], inp["wr"], inp["bias"])
    n_near = check_route(spec, r, res["idx"], res["gate"], res["load"])
    check_permutation(spec, res["idx"], res["offsets"], res["perm"])
    # the row gather of moe_permute (the fused forward reads x through
    # perm_slot instead): gathered rows are exact copies
    K = spec.K
    layer.permute(layer._cfg(spec.T), inp["x"])
    perm = torch.as_tensor(res["perm"], device="cuda")
    assert torch.equal(layer.x_perm[:spec.T * K], inp["x"][perm // K])
    out = check_outputs(spec, layer, inp, res, r)
    say(f"[parity] {name}: near-ties={n_near} y_err/rms={out['y_err']:.3e}")


def test_call_sequences_agree_bit_for_bit_and_are_deterministic():
    """Separate expert calls on one stream, the shared expert on a second
    stream, and the fused moe_experts path: identical bits, twice over."""
    spec = CASES["v3_gemm"]
    inp = synth.make_inputs(spec, "cuda")
    runs = [run_steps(spec, inp, bias=inp["bias"], side_stream=side, fused=fused)[1]
            for side, fused in ((False, False), (True, False), (True, False), (False, True),
                                (False, True))]
    runs = [{k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in r.items()}
            for r in runs]
    a = runs[0]
    for b in runs[1:]:
        for k in ("idx", "gate", "load", "offsets", "perm"):
            assert np.array_equal(a[k], b[k]), k
        assert torch.equal(a["y"], b["y"])


def test_split_entry_points_equal_expert_ffn():
    spec = CASES["v3_gemm"]
    inp = synth.make_inputs(spec, "cuda")
    layer, res = run_steps(spec, inp, bias=inp["bias"])
    cfg = moe.config_of(spec)
    TK = spec.T * spec.K
    layer.permute(layer._cfg(spec.T), inp["x"])        # fill x_perm
    h = torch.empty((TK, spec.I), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((TK, spec.d), dtype=layer.out_slots.dtype, device="cuda")
    moe.moe_expert_gate_up(cfg, layer.x_perm[:TK], layer.expert_offsets, inp["w1"], inp["w3"], None, None, h)
    moe.moe_expert_down(cfg, h, layer.expert_offsets, layer.perm_slot[:TK], layer.topk_gate, inp["w2"], None, out)
    torch.cuda.synchronize()
    assert torch.equal(out, layer.out_slots[:TK])


def test_bias_changes_selection_not_gates_on_gpu():
    spec = CASES["v3_gemm"]
    inp = synth.make_inputs(spec, "cuda")
    _, a = run_steps(spec, inp, bias=None)
    _, b = run_steps(spec, inp, bias=inp["bias"])
    same = np.all(np.sort(a["idx"], 1) == np.sort(b["idx"], 1), axis=1)
    assert (~same).any()
    for t in np.flatnonzero(same)[:200]:
        ga = dict(zip(a["idx"][t], a["gate"][t]))
        gb = dict(zip(b["idx"][t], b["gate"][t]))
        for e in ga:
            assert abs(ga[e] - gb[e]) <= 1e-6


def test_forced_bias_routes_every_token_to_one_set():
    spec = CASES["v3_gemm"]
    inp = synth.make_inputs(spec, "cuda")
    forced = [3, 17, 5, 30]
    bias = torch.zeros(spec.E, dtype=torch.float32, device="cuda")
    bias[forced] = 10.0
    layer, res = run_steps(spec, inp, bias=bias)
    assert all(set(row) == set(forced) for row in res["idx"].tolist())
    load = res["load"]
    assert load[forced].tolist() == [spec.T] * 4 and load.sum() == spec.T * spec.K
    r, _ = oracle_route(spec, inp["x"], inp["wr"], bias)
    check_route(spec, r, res["idx"], res["gate"], res["load"])
    check_outputs(spec, layer, inp, res, r, rows=np.arange(0, spec.T, 37))


def test_bf16_output_is_the_rounded_fp32_output():
    import dataclasses
    spec = CASES["v3_gemm"]
    inp = synth.make_inputs(spec, "cuda")
    _, a = run_steps(spec, inp, bias=inp["bias"])
    y32 = a["y"].clone()
    spec16 = dataclasses.replace(spec, out_dtype="bf16")
    _, b = run_steps(spec16, inp, bias=inp["bias"])
    assert b["y"].dtype == torch.bfloat16
    assert torch.equal(b["y"], y32.to(torch.bfloat16))


def test_zero_tokens_zero_load():
    spec = CASES["v3_gemm"]
    inp = synth.make_inputs(spec, "cuda")
    layer = moe.MoELayer(spec, inp, max_tokens=16)
    layer.load.fill_(7)
    y = layer.forward(inp["x"][:0], inp["bias"])
    torch.cuda.synchronize()
    assert y.shape == (0, spec.d) and int(layer.load.abs().sum()) == 0


def test_bias_update_matches_oracle():
    E = 256
    rng = np.random.default_rng(5)
    cases = [rng.integers(0, 100, E), np.full(E, 8), np.zeros(E, dtype=np.int64),
             np.r_[np.full(E - 1, 3), 3 + E]]
    bias0 = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    for load in cases:
        b = torch.tensor(bias0, device="cuda")
        ld = torch.tensor(load.astype(np.int32), device="cuda")
        moe.moe_bias_update(E, ld, 1e-3, b)
        torch.cuda.synchronize()
        want = oracle.bias_update(bias0, load)
        assert np.array_equal(b.cpu().numpy().view(np.uint32), want.view(np.uint32))


def test_zipf_trajectory_small():
    """Skewed loads: routing parity on every batch and the bias after each
    moe_bias_update bit-identical to the oracle's step from the same loads."""
    # w_std scaled so the logit noise matches the full-size workload (d = 7168)
    spec = _cfg("zipf_stress_bf16", T=2048, d=256, E=64, K=8, I=64, Is=64, batches=6,
                w_std=0.02 * (7168 / 256) ** 0.5)
    inp = synth.make_inputs(spec, "cuda")
    layer = moe.MoELayer(spec, inp, max_tokens=spec.T)
    bias = torch.zeros(spec.E, dtype=torch.float32, device="cuda")
    ratios = []
    for bt in range(spec.batches):
        x = synth.make_x(spec, "cuda", batch=bt)
        b_before = bias.cpu().numpy().copy()
        layer.forward(x, bias)
        torch.cuda.synchronize()
        idx = layer.topk_idx.cpu().numpy().astype(np.int64)
        gate = layer.topk_gate.cpu().numpy().astype(np.float64)
        load = layer.load.cpu().numpy().astype(np.int64)
        r, _ = oracle_route(spec, x, inp["wr"], bias)
        check_route(spec, r, idx, gate, load)
        layer.bias_update(bias)
        torch.cuda.synchronize()
        want = oracle.bias_update(b_before, load)
        assert np.array_equal(bias.cpu().numpy().view(np.uint32), want.view(np.uint32))
        ratios.append(load.max() / load.mean())
    say(f"[zipf small] max/mean per batch: {np.round(ratios, 2).tolist()}")
    assert ratios[0] > 3.0            # skewed to begin with


@pytest.mark.parametrize("seq_len", [1, 1000, 4099, 5000])
def test_sequence_loads_match_oracle(seq_len):
    """moe_sequence_loads against the oracle's per-sequence counts of its own
    routing: equal on every sequence, up to the (validated) near-tie tokens,
    each of which can move at most K pairs between experts."""
    spec = CASES["v3_fused"]
    inp = synth.make_inputs(spec, "cuda")
    layer, res = run_steps(spec, inp, bias=inp["bias"])
    r, _ = oracle_route(spec, inp["x"], inp["wr"], inp["bias"])
    check_route(spec, r, res["idx"], res["gate"], res["load"])
    nq = -(-spec.T // seq_len)
    got = torch.full((nq, spec.E), -7, dtype=torch.int32, device="cuda")
    moe.moe_sequence_loads(moe.config_of(spec), layer.topk_idx[:spec.T], seq_len, got)
    got = got.cpu().numpy().astype(np.int64)
    want = oracle.sequence_loads(r["sel"], spec.E, seq_len)
    near_per_seq = np.add.reduceat(r["near_tie"].astype(np.int64), np.arange(0, spec.T, seq_len))
    diff = np.abs(got - want).sum(axis=1)
    assert np.all(diff <= 2 * spec.K * near_per_seq), (diff.max(), near_per_seq.max())
    assert np.all(got.sum(axis=1) == np.diff(np.minimum(np.arange(0, nq + 1) * seq_len, spec.T)) * spec.K)
