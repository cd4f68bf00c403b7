"""The steps either side of the layer ("DeepSeekMoE架构解析" section 4.1 and
eq. (12) of section 2.1): the pre-MoE RMSNorm and the residual add.

moe_rmsnorm is computed in double precision and rounded once, so for bf16
activations the GPU's normalised tokens equal the oracle's (float64, rounded
once by its own converter) bit for bit; the layer on those tokens is then
checked like the plain layer (routing bit-exact up to near-ties, outputs to
the tolerance), with y = x + the expert sum."""

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


def _oracle_u(spec, x, w):
    u = oracle.rmsnorm(f64(x), w.detach().cpu().numpy().astype(np.float64))
    if spec.act_dtype == "bf16":
        return oracle.f64_to_bf16_bits(u)
    return u.astype(np.float32)


def _as_device(spec, u_host):
    if spec.act_dtype == "bf16":
        return torch.from_numpy(u_host.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(u_host).cuda()


@pytest.mark.parametrize("base,kw", [
    ("v3_prefill_bf16", dict(T=300, d=256)),
    ("v3_prefill_bf16", dict(T=1024, d=7168)),
    ("dsmoe2024_bf16", dict(T=257, d=2048)),
    ("tiny_f32", dict()),
])
def test_rmsnorm_matches_oracle(base, kw):
    spec = _cfg(base, **kw) if kw else synth.get_config(base)
    inp = synth.make_inputs(spec, "cuda", with_experts=False)
    x, w = inp["x"], inp["norm_w"]
    cfg = moe.config_of(spec)
    u = torch.empty_like(x)
    moe.moe_rmsnorm(cfg, x, w, u)
    inplace = x.clone()
    moe.moe_rmsnorm(cfg, inplace, w, inplace)
    torch.cuda.synchronize()
    want = _oracle_u(spec, x, w)
    got = host(u)
    if spec.act_dtype == "bf16":
        assert np.array_equal(got, want), f"{int((got != want).sum())} of {got.size} differ"
    else:
        # fp32 inputs: the squares' sum may round, in a different order on each
        # side; at most one fp32 step apart
        assert np.all(np.abs(got.view(np.int32).astype(np.int64) - want.view(np.int32)) <= 1)
    assert torch.equal(inplace, u)



def test_rmsnorm_at_bf16_rounding_boundaries():
    """Outputs placed on bf16 rounding midpoints: rows of ones (root =
    sqrt(1 + eps)) with w = midpoint * root, so (x / root) * w lies within a
    float rounding of a midpoint between two bf16 values and its rounding is
    decided below float precision; plus random rows. Both the float-formed
    elements and the ones redone in double must equal the oracle's bit for
    bit, out of place and in place."""
    spec = _cfg("v3_prefill_bf16", T=64, d=256)
    cfg = moe.config_of(spec)
    d = spec.d
    root = np.sqrt(1.0 + 1e-6)
    k = np.arange(d) % 128
    mid = (1.0 + (2 * k + 1) * 2.0 ** -8) * np.where(np.arange(d) < 128, 1.0, -0.5)
    w = torch.from_numpy((mid * root).astype(np.float32)).cuda()
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    x = torch.randn((spec.T, d), device="cuda", generator=g).to(torch.bfloat16)
    x[: spec.T // 2] = 1.0
    u = torch.empty_like(x)
    moe.moe_rmsnorm(cfg, x, w, u)
    inplace = x.clone()
    moe.moe_rmsnorm(cfg, inplace, w, inplace)
    torch.cuda.synchronize()
    want = _oracle_u(spec, x, w)
    got = host(u)
    assert np.array_equal(got, want), f"{int((got != want).sum())} of {got.size} differ"
    assert torch.equal(inplace, u)
    # the ones rows really sit on midpoints: their float64 values are within
    # 2^-20 (relative) of one
    u64 = oracle.rmsnorm(f64(x[: spec.T // 2]), w.cpu().numpy().astype(np.float64))
    assert np.all(np.abs(u64 / mid - 1) < 2.0 ** -20)

CASES = {
    "v3_small": _cfg("v3_prefill_bf16", T=300, d=256, E=64, K=6, I=128, Is=128),
    "v3_fused": _cfg("v3_prefill_bf16", T=4100, d=128, E=256, K=8, I=128, Is=128),
    "fp8_small": _cfg("v3_decode_fp8", T=64, d=512, E=64, K=8, I=256, Is=256),
    "grouped": _cfg("v3_grouped_bf16", T=500, d=256, E=64, K=6, I=128, Is=128,
                    n_groups=8, topk_groups=3),
}


def _check_norm_layer(spec, inp, n_rows=None):
    layer, res = run_steps(spec, inp, bias=inp["bias"],
                           layer=moe.MoELayer(spec, inp, pre_norm=True, residual=True))
    u_host = _oracle_u(spec, inp["x"], inp["norm_w"])
    assert np.array_equal(host(layer.u[:spec.T]), u_host), "normalised tokens differ"
    u_dev = _as_device(spec, u_host)
    r, _ = oracle_route(spec, u_dev, inp["wr"], inp["bias"])
    n_near = check_route(spec, r, res["idx"], res["gate"], res["load"])
    check_permutation(spec, res["idx"], res["offsets"], res["perm"])
    rows = None
    if n_rows is not None:
        rng = np.random.default_rng(0)
        rows = np.sort(np.unique(np.concatenate([rng.choice(spec.T, n_rows, replace=False),
                                                 np.flatnonzero(r["near_tie"])[:4]])))
    out = check_outputs(spec, layer, inp, res, r, x=u_dev, rows=rows, residual=f64(inp["x"]))
    return n_near, out


@pytest.mark.parametrize("name", list(CASES))
def test_layer_with_pre_norm_and_residual(name):
    spec = CASES[name]
    say(f"[norm] {name}")
    inp = synth.make_inputs(spec, "cuda")
    n_near, out = _check_norm_layer(spec, inp)
    say(f"[norm] {name}: near-ties={n_near} y_err/rms={out['y_err']:.3e}")


@pytest.mark.timeout(300)
def test_fullsize_v3_with_pre_norm_and_residual():
    spec = synth.get_config("v3_prefill_bf16")
    inp = synth.make_inputs(spec, "cuda")
    n_near, out = _check_norm_layer(spec, inp, n_rows=12)
    say(f"[norm] full V3: near-ties={n_near} y_err/rms={out['y_err']:.3e}")
