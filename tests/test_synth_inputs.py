"""The seeded input recipe: shapes, storage types, determinism, fp8 codes."""

import json
import os

import numpy as np
import torch

import synth


def test_zipf_amplitude_matches_calibration(golden_dir):
    with open(os.path.join(golden_dir, "zipf_calibration.json")) as f:
        cal = json.load(f)
    assert synth.get_config("zipf_stress_bf16").zipf_A == cal["A"]
    assert 9.5 <= cal["hottest_over_mean"] <= 10.5


def _small(name, **kw):
    return synth.scaled_config(name, **kw)


def test_shapes_and_dtypes_small_configs():
    for name, kw in [("tiny_f32", {}),
                     ("dsmoe2024_bf16", dict(T=40, d=128, I=64, Is=64)),
                     ("v3_decode_fp8", dict(T=8, d=128, E=32, I=64, Is=64)),
                     ("zipf_stress_bf16", dict(T=16, d=128, E=32, I=64, Is=64))]:
        cfg = _small(name, **kw)
        inp = synth.make_inputs(cfg, "cpu")
        T, d, E, I = cfg.T, cfg.d, cfg.E, cfg.I
        assert inp["x"].shape == (T, d) and inp["wr"].shape == (E, d)
        assert inp["w1"].shape == (E, I, d) and inp["w3"].shape == (E, I, d) and inp["w2"].shape == (E, d, I)
        assert inp["w1s"].shape == (cfg.S * cfg.Is, d) and inp["w2s"].shape == (d, cfg.S * cfg.Is)
        if cfg.weight_dtype == "fp8":
            assert inp["w1"].dtype == torch.uint8 and inp["s1"].shape == (E, I) and inp["s2"].shape == (E, d)
            codes = inp["w1"].view(-1)
            assert not bool(((codes & 0x7F) == 0x7F).any())      # no NaN codes
            assert inp["s2s"].shape == (d,)
        if cfg.bias_range is None:
            assert inp["bias"] is None
        else:
            assert float(inp["bias"].abs().max()) <= cfg.bias_range
        if cfg.zipf_s is not None:
            assert bool((inp["x"][:, 0].float() == 1.0).all())


def test_generation_is_deterministic():
    cfg = _small("dsmoe2024_bf16", T=16, d=64, E=8, I=64, Is=64)
    a, b = synth.make_inputs(cfg, "cpu"), synth.make_inputs(cfg, "cpu")
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k
    x1 = synth.make_x(cfg, "cpu", batch=1)
    assert not torch.equal(x1, a["x"])


def test_to_numpy_stored_bf16_bits():
    t = torch.tensor([1.0, -2.0, 0.5], dtype=torch.bfloat16)
    bits = synth.to_numpy_stored(t)
    assert bits.dtype == np.uint16 and bits.tolist() == [0x3F80, 0xC000, 0x3F00]


def test_slot_dtype_of_named_and_reduced_workloads():
    """The full-size bf16 workloads hold their routed slot rows in bf16; a
    reduced shape derived from one goes back to the library default (fp32)
    unless it asks, and the fp32 and fp8 workloads keep fp32."""
    for name in ("v3_prefill_bf16", "v3_grouped_bf16", "zipf_stress_bf16", "v3_ep8_shard_bf16",
                 "dsmoe2024_bf16"):
        assert synth.get_config(name).slot_dtype == "bf16", name
        assert synth.scaled_config(name, T=64).slot_dtype == "f32", name
        assert synth.scaled_config(name, T=64, slot_dtype="bf16").slot_dtype == "bf16", name
    for name in ("tiny_f32", "v3_decode_fp8", "v3_prefill_fp8b"):
        assert synth.get_config(name).slot_dtype == "f32", name
