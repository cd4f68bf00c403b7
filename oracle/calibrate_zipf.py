"""Calibrate the Zipf popularity amplitude A of the skewed-load workload.

The stress workload gives expert e a router-logit offset A * rank(e)^(-1.1)
(carried by a constant input coordinate). This script picks A by bisection so
that, on batch 0 with zero bias, the hottest expert's load is ten times the
mean load, using the oracle's routing on the workload's own synthetic inputs
(generated on the CPU; the GPU draws differ but follow the same distribution,
and the benchmark reports the ratio it actually measures). It writes
tests/golden/zipf_calibration.json.

Run:  python -m oracle.calibrate_zipf [--tokens 8192]
"""

from __future__ import annotations

import argparse
import dataclasses
import json
import os

import numpy as np

from oracle import route, decode_stored


def _load_ratio(cfg, A, x64, wr_bits):
    import synth
    off = synth.generate.zipf_offsets(dataclasses.replace(cfg, zipf_A=A)).numpy()
    wr = wr_bits.copy()
    # bf16 storage of the offsets, as the generator stores them
    import torch
    wr[:, 0] = torch.from_numpy(off).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    r = route(x64, decode_stored(wr), None, cfg.K, cfg.score, cfg.norm)
    load = r["load"]
    return load.max() / load.mean(), load


def main():
    import synth
    ap = argparse.ArgumentParser()
    ap.add_argument("--tokens", type=int, default=8192)
    ap.add_argument("--target", type=float, default=10.0)
    args = ap.parse_args()
    cfg = synth.get_config("zipf_stress_bf16")
    x = synth.make_x(cfg, "cpu", batch=0, T=args.tokens)
    x64 = decode_stored(synth.to_numpy_stored(x))
    inp = synth.make_inputs(cfg, "cpu", with_experts=False)
    wr_bits = synth.to_numpy_stored(inp["wr"])
    lo, hi = 1.0, 5.0
    for _ in range(18):
        mid = 0.5 * (lo + hi)
        ratio, _ = _load_ratio(cfg, mid, x64, wr_bits)
        print(f"A={mid:.5f} hottest/mean={ratio:.3f}", flush=True)
        if ratio < args.target:
            lo = mid
        else:
            hi = mid
    A = round(0.5 * (lo + hi), 4)
    ratio, load = _load_ratio(cfg, A, x64, wr_bits)
    out = {"about": "Zipf(1.1) amplitude A for the skewed-load workload, chosen by oracle routing "
                    "of batch 0 (bias 0) so that hottest/mean load = 10; written by oracle/calibrate_zipf.py",
           "A": A, "tokens": args.tokens, "hottest_over_mean": float(ratio),
           "coldest_over_mean": float(load.min() / load.mean()),
           "second_over_mean": float(np.sort(load)[-2] / load.mean())}
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "tests", "golden", "zipf_calibration.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=2)
    print(json.dumps(out, indent=2))


if __name__ == "__main__":
    main()
