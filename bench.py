"""Throughput of the DeepSeekMoE layer forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu-baseline] [--no-decode]
                    [--no-grouped] [--no-fp8] [--no-stress] [--no-ep8]

One step = one whole layer call on one batch already resident in HBM, in
the call sequence of MoELayer.forward: the shared expert's SwiGLU FFN on a
second stream from the start of the call, and on the caller's stream the
router GEMM + sigmoid + biased top-K + gates + loads, the stable
permutation, the grouped gate/up and down SwiGLU GEMMs over the routed
experts (one launch each, token rows read through the permutation), then,
once both streams are done, the combine. The workload is the V3-shape prefill layer:
T = 8192 tokens, d = 7168, 256 routed experts of intermediate 2048 (top-8,
score + bias selection) plus 1 shared expert, bf16, synthetic seeded inputs,
expert weights relocated once into the tiled layout before timing.

Printed: one JSON line with tokens/s (mean over the timed region, and the
median and minimum of per-step event timings), the roofline of the dominant
kernel (the routed experts' grouped gate/up GEMM, timed live with HIP
events on its stream,
as a fraction of the nominal peaks and of measured ones), the fp64 oracle
timed on a bounded
sample on the host's cores with the GPU's error on those tokens, and the
other workloads: the layer with the pre-MoE RMSNorm and residual, the decode
layer's fraction of HBM peak, node-limited routing (8 groups, top-4), the
fine-grained fp8 prefill layer, one GPU's share of the layer under 8-way
expert parallelism (32 local experts, 2048 rows each), the skewed-load stress run (20 batches
with the bias update, max/mean load per batch), and the tiny fp32 and
2024-layout workloads (tokens/s and TFLOP/s against their peaks).
Measured peaks come from the probes of libmoe_peaks.so (a loop of
independent MFMAs per instruction form, an fp32 FMA loop, a streaming read
and copy; plus torch's copy and the vendor BLAS GEMM for reference), and
every rate in the line is also given as a fraction of them.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import mixture_experts_layer_40_amd as moe  # noqa: E402
from mixture_experts_layer_40_amd import peaks as pk  # noqa: E402
import synth  # noqa: E402

MFMA_BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16
MFMA_FP8_PEAK_TFLOPS = 5000.0      # MI355X dense fp8
HBM_PEAK_GBS = 8000.0              # MI355X HBM3E
WORKLOAD = "v3_prefill_bf16"
DECODE = "v3_decode_fp8"
GROUPED = "v3_grouped_bf16"
FP8B = "v3_prefill_fp8b"
EP8 = "v3_ep8_shard_bf16"
STRESS = "zipf_stress_bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_v3_prefill_traffic.txt")
TRAFFIC_FILE_FP8 = os.path.join(ROOT, "profiles", "gate_up_v3_prefill_fp8_traffic.txt")
MFMA_UTIL_FILE = os.path.join(ROOT, "profiles", "gemm_mfma_util.txt")
DECODE_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_v3_fp8_traffic.txt")
CLOCK_FILE = os.path.join(ROOT, "profiles", "gemm_clock.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "mixture_experts_layer_40_amd", "csrc", f)
                  for f in ("ffn.hip", "gemm_core.hpp", "common.hpp")]
# The call sequence the bf16 / row-scaled fp8 summaries were taken on: the
# shared experts' FFN on the layer's second stream and the routed experts'
# two grouped launches on the caller's. A summary of another sequence
# describes other launches and is not read.
LAYER_SEQUENCE = "shared-ffn-on-second-stream"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_COMMENT = re.compile(r"//[^\n]*|/\*.*?\*/", re.S)


def kernel_source_hash() -> str:
    """Hash of the GEMM kernel sources with comments and whitespace removed:
    a committed counter summary stays valid across edits of comments only,
    and is dropped as soon as any code changes."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            code = _COMMENT.sub(" ", f.read())
        h.update(" ".join(code.split()).encode())
    return h.hexdigest()[:16]


def read_summary(path, sequence=LAYER_SEQUENCE):
    """The key = value lines of a committed summary, if it was taken on the
    current kernel sources (and, with `sequence`, on that call sequence of
    the layer); else None."""
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_src_sha") != kernel_source_hash():
        return None
    if sequence is not None and kv.get("layer_sequence") != sequence:
        return None
    return kv


def measured_mfma_util(path=MFMA_UTIL_FILE):
    """Matrix-core busy percentages of the grouped GEMM launches from the
    committed rocprofv3 counter run (MfmaUtil), if it was taken on the
    current kernel source and call sequence; else an empty dict."""
    kv = read_summary(path)
    if kv is None:
        return {}
    return {k[len("mfma_util_"):]: float(v) for k, v in kv.items() if k.startswith("mfma_util_")}


def measured_clock(path=CLOCK_FILE):
    """Engine clock (GHz) and matrix-core busy share (%) of the grouped GEMM
    launches from the committed rocprofv3 counter run (GRBM_GUI_ACTIVE over
    each dispatch's duration), if it was taken on the current kernel source;
    with the dense bf16 MFMA rate at that clock. Else an empty dict."""
    kv = read_summary(path)
    if kv is None:
        return {}
    out = {}
    for k, v in kv.items():
        if k.startswith("clock_ghz_"):
            name = k[len("clock_ghz_"):]
            ghz = float(v)
            out[name] = {"ghz": ghz, "mfma_busy_pct": float(kv.get("mfma_busy_" + name, "nan")),
                         "bf16_ceiling_TFLOPs": MFMA_BF16_PEAK_TFLOPS * ghz / 2.4}
    return out


def measured_traffic(path=TRAFFIC_FILE):
    """HBM bytes from a committed rocprofv3 counter summary (per gate/up launch,
    or per decode layer call for the decode one), if the counters were taken on
    the current kernel source (and call sequence, except for the fine-grained
    fp8 layer, which keeps the shared experts in its launches); else None."""
    kv = read_summary(path, None if path == TRAFFIC_FILE_FP8 else LAYER_SEQUENCE)
    if kv is None:
        return None
    try:
        return float(kv["decode_gemm_bytes_per_call"] if "decode_gemm_bytes_per_call" in kv
                     else kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timed:
    """HIP events around one library call on the current stream."""

    def __init__(self):
        self.pairs = []

    def __enter__(self):
        self.s = torch.cuda.Event(enable_timing=True)
        self.e = torch.cuda.Event(enable_timing=True)
        self.s.record()
        return self

    def __exit__(self, *exc):
        self.e.record()
        self.pairs.append((self.s, self.e))

    def mean_ms(self):
        return float(np.mean([s.elapsed_time(e) for s, e in self.pairs]))


def gate_up_bytes(spec, shared=True) -> float:
    """Algorithmic HBM bytes of one gate/up launch: W1 and W3 of every routed
    expert (and of the shared experts, when the launch holds them) once, x
    once, H (and the shared H) written once (bf16)."""
    TK, SI = spec.T * spec.K, (spec.S * spec.Is if shared else 0)
    return float(spec.E * 2 * spec.I * spec.d * 2 + 2 * SI * spec.d * 2 + spec.T * spec.d * 2
                 + TK * spec.I * 2 + spec.T * SI * 2)


def gate_up_flops(spec, shared=True) -> float:
    return 4.0 * spec.d * (spec.I * spec.T * spec.K + (spec.S * spec.Is * spec.T if shared else 0))


def layer_step(layer, x, bias, bufs, gate_timer=None):
    """One full layer call (the fused path of MoELayer.forward: the shared
    expert on the layer's second stream, the routed experts on the caller's),
    with the routed experts issued as their two grouped launches so the
    gate/up launch can be bracketed by events on its stream."""
    h, hs, ws_gemm = bufs
    cfg = layer._cfg(x.shape[0])
    residual = x if layer.residual else None
    if layer.pre_norm:
        moe.moe_rmsnorm(cfg, x, layer.w["norm_w"], layer.u[:x.shape[0]])
        x = layer.u[:x.shape[0]]
    T, K, w = cfg.num_tokens, cfg.top_k, layer.w
    TK = T * K
    cur = torch.cuda.current_stream()
    side = layer.side
    if side is not None:
        side.wait_stream(cur)
        with torch.cuda.stream(side):
            layer.shared(cfg, x, stream=side)
    layer.route(x, bias)
    layer.permute(cfg, x, gather=False)
    shared_here = side is None and spec_has_shared(layer)   # else on the side stream
    ecfg = cfg if side is None else layer.routed_cfg(T)

    def gate_up():
        moe.moe_experts_gate_up(ecfg, x, layer.expert_offsets, layer.perm_slot[:TK], w["w1"],
                                w["w3"], w.get("s1"), w.get("s3"),
                                *((w.get("w1s"), w.get("w3s"), w.get("s1s"), w.get("s3s"), h, hs)
                                  if shared_here else (None, None, None, None, h, None)),
                                ws=ws_gemm)
    if gate_timer is not None:
        with gate_timer:
            gate_up()
    else:
        gate_up()
    moe.moe_experts_down(ecfg, h, hs if shared_here else None, layer.expert_offsets,
                         layer.perm_slot[:TK], layer.topk_gate[:T], w["w2"], w.get("s2"),
                         w.get("w2s") if shared_here else None,
                         w.get("s2s") if shared_here else None, layer.out_slots[:TK],
                         layer.y_shared[:T] if shared_here else None, ws=ws_gemm)
    if side is not None:
        cur.wait_stream(side)
    layer.combine(cfg, residual)


def spec_has_shared(layer) -> bool:
    return layer.y_shared is not None


def setup(spec):
    inp = synth.make_inputs(spec, "cuda")
    layer = moe.MoELayer(spec, inp, max_tokens=spec.T, fused=True)
    cfg = layer._cfg(spec.T)
    h = torch.empty((spec.T * spec.K, spec.I), dtype=torch.bfloat16, device="cuda")
    hs = (torch.empty((spec.T, spec.S * spec.Is), dtype=torch.bfloat16, device="cuda")
          if spec.S > 0 else None)
    ws_gemm = torch.empty(max(moe.moe_workspace_size(cfg, moe.MOE_WS_GEMM), 256), dtype=torch.uint8,
                          device="cuda")
    return inp, layer, (h, hs, ws_gemm)


def time_steps(layer, x, bias, bufs, steps, warmup, gate_timer=None, step_ms=None):
    """Seconds per step over `steps` timed steps (host clock around the whole
    timed region, bracketed by synchronisations). With a list `step_ms`, an
    event pair on the stream also brackets each step and its duration is
    appended (for the median and minimum)."""
    for _ in range(warmup):
        layer_step(layer, x, bias, bufs)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)] if step_ms is not None else None
    t0 = time.perf_counter()
    for i in range(steps):
        if ev:
            ev[i].record()
        layer_step(layer, x, bias, bufs, gate_timer)
    if ev:
        ev[steps].record()
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    if ev:
        step_ms.extend(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return sec


def spread(step_ms):
    return {"ms_per_step_median": float(np.median(step_ms)), "ms_per_step_min": float(np.min(step_ms))}


def cpu_baseline(spec, inp, layer, bufs, n_tokens):
    """The fp64 oracle timed on the host's cores: routing of n_tokens tokens
    of the batch (all of them by default: the full layer) and their layer
    outputs, each routed expert's stored weights decoded to fp64 once. The
    stored values are copied to host memory before the timed region. Then,
    untimed, the parity of the GPU's output on the same tokens: every
    selected set equal to the oracle's or, for a near-tie token, one the tie
    leaves open (oracle.selection_valid), and y within 2e-2 x RMS of the
    oracle evaluated on the GPU's set for near-tie tokens."""
    import oracle
    from threadpoolctl import threadpool_info
    T = spec.T
    if n_tokens >= T:
        rows = np.arange(T)
    else:
        rows = np.sort(np.random.default_rng(0).choice(T, n_tokens, replace=False))
    trow = torch.as_tensor(rows, device="cuda")
    host = synth.to_numpy_stored
    x = host(inp["x"][trow])
    wr = host(inp["wr"])
    bias = inp["bias"].cpu().numpy()
    w = {n: host(inp[n]) for n in ("w1", "w3", "w2")}
    sc = {n: None if inp.get(n) is None else inp[n].cpu().numpy() for n in ("s1", "s3", "s2")}
    shared = (host(inp["w1s"]), host(inp["w3s"]), host(inp["w2s"]),
              None if inp.get("s1s") is None else inp["s1s"].cpu().numpy(),
              None if inp.get("s3s") is None else inp["s3s"].cpu().numpy(),
              None if inp.get("s2s") is None else inp["s2s"].cpu().numpy())
    pick = lambda n, e: None if sc[n] is None else sc[n][e]
    bank = oracle.ExpertBank(
        fetch=lambda e: (w["w1"][e], w["w3"][e], w["w2"][e], pick("s1", e), pick("s3", e),
                         pick("s2", e)),
        shared=shared, S=spec.S)
    t0 = time.perf_counter()
    x64 = oracle.decode_stored(x)
    r = oracle.route(x64, oracle.decode_stored(wr), bias.astype(np.float64), spec.K, spec.score,
                     spec.norm)
    y_or = oracle.layer_rows(x64, r["sel"], r["gate"], bank)[0]
    dt = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    n_exp = len(np.unique(r["sel"]))
    what = (f"full layer: all {T} tokens" if len(rows) == T else f"{len(rows)} of {T} tokens")
    baseline = {"value": len(rows) / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
                "sample": f"{what} of the {spec.name} batch (routing, shared expert, {n_exp} routed "
                          f"experts decoded to fp64), {dt:.1f} s"}
    # parity of the same tokens (outside the timed region): one plain layer step
    layer_step(layer, inp["x"], inp["bias"], bufs)
    torch.cuda.synchronize()
    gidx = layer.topk_idx[trow].cpu().numpy().astype(np.int64)
    near = r["near_tie"]
    valid = oracle.selection_valid(r, gidx, spec.K)
    if near.any():
        g_near = oracle.gate_values(r["scores"][near], gidx[near], spec.norm)
        y_or[near] = oracle.layer_rows(x64[near], gidx[near], g_near, bank)[0]
    y_gpu = layer.y[trow].double().cpu().numpy()
    rms = float(np.sqrt(np.mean(y_or ** 2)))
    err = float(np.abs(y_gpu - y_or).max() / rms)
    parity = {"tokens": int(len(rows)), "selections_valid": bool(valid.all()),
              "invalid_selections": int((~valid).sum()), "near_ties": int(near.sum()),
              "max_abs_err_over_rms": err, "tolerance": 2e-2,
              "pass": bool(valid.all() and err <= 2e-2)}
    return baseline, parity


def other_slots_measure(layer, x, bias, bufs, steps, warmup):
    """The same layer step with the routed slot rows in the other dtype: fp32
    (the library default, twice the bytes, no rounding of the routed terms)
    when the workload holds them in bf16, and the other way round."""
    keep = layer.slot_dtype, layer.out_slots
    other = "f32" if keep[0] == "bf16" else "bf16"
    layer.slot_dtype = other
    layer.out_slots = torch.empty(keep[1].shape, dtype=torch.float32 if other == "f32" else torch.bfloat16,
                                  device="cuda")
    try:
        step_ms = []
        sec = time_steps(layer, x, bias, bufs, steps, warmup, None, step_ms)
    finally:
        layer.slot_dtype, layer.out_slots = keep
    return {"slot_dtype": other, "ms_per_step": sec * 1e3, "tokens_per_s": x.shape[0] / sec,
            **spread(step_ms)}


def decode_measure(steps, warmup):
    spec = synth.get_config(DECODE)
    inp, layer, bufs = setup(spec)
    x, bias = inp["x"], inp["bias"]
    step_ms = []
    sec = time_steps(layer, x, bias, bufs, steps, warmup, step_ms=step_ms)
    load = layer.load.cpu().numpy()
    n_active = int((load > 0).sum())
    bytes_ = ((n_active * spec.weight_bytes_per_expert() + spec.shared_weight_bytes())
              + spec.E * spec.d * 2 + spec.E * 4                      # router rows, bias
              + spec.T * spec.d * 2 + spec.T * spec.d * 4)            # x in, y out (fp32)
    gbs = bytes_ / sec / 1e9
    # the same layer call recorded once into a HIP graph and replayed (a
    # decode step is a short launch sequence; replay removes the host's
    # per-launch work between its kernels)
    xg = x.clone()
    graph = layer.capture(xg, bias)
    gsec = per_launch_ms(graph.replay, steps) * 1e-3
    ggbs = bytes_ / gsec / 1e9
    out = {"workload": DECODE, "tokens_per_s": spec.T / sec, "ms_per_step": sec * 1e3,
           "active_experts": n_active, "algorithmic_bytes": int(bytes_), "achieved_GBs": gbs,
           "peak_GBs": HBM_PEAK_GBS, "frac": gbs / HBM_PEAK_GBS, **spread(step_ms),
           "graph_ms_per_step": gsec * 1e3, "graph_tokens_per_s": spec.T / gsec,
           "graph_achieved_GBs": ggbs, "graph_frac": ggbs / HBM_PEAK_GBS,
           # HBM bytes of its two GEMM launches from the committed counter runs
           "gemm_traffic": measured_traffic(DECODE_TRAFFIC_FILE)}
    del inp, layer, bufs, graph, xg
    torch.cuda.empty_cache()
    return out


def per_launch_ms(call, iters=20) -> float:
    """Mean time of one call, from HIP events around `iters` back-to-back
    calls on the current stream (a short kernel timed alone would also count
    the host's launch latency)."""
    call()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(iters):
        call()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / iters


def route_ms(layer, x, bias, iters=20) -> float:
    return per_launch_ms(lambda: layer.route(x, bias), iters)


def sequence_loads_ms(layer, spec, seq_len, iters=20) -> float:
    """Per-sequence expert loads of the last routed batch (sequences of seq_len)."""
    cfg = layer._cfg(spec.T)
    nq = -(-spec.T // seq_len)
    out = torch.empty((nq, spec.E), dtype=torch.int32, device="cuda")
    idx = layer.topk_idx[:spec.T]
    return per_launch_ms(lambda: moe.moe_sequence_loads(cfg, idx, seq_len, out), iters)


def norm_residual_measure(layer, spec, x, bias, bufs, steps, warmup):
    """The same prefill layer between a pre-MoE RMSNorm and the residual add
    (section 4.1, eq. 12): tokens/s and the RMSNorm kernel's own time."""
    layer.pre_norm, layer.residual = True, True
    layer.u = torch.empty_like(x)
    sec = time_steps(layer, x, bias, bufs, steps, warmup)
    cfg = layer._cfg(spec.T)
    u, w = layer.u, layer.w["norm_w"]
    ms = per_launch_ms(lambda: moe.moe_rmsnorm(cfg, x, w, u))
    layer.pre_norm, layer.residual, layer.u = False, False, None
    # algorithmic bytes: x read and u written once (the weight vector is noise)
    nbytes = 2.0 * spec.T * spec.d * x.element_size()
    return {"tokens_per_s": spec.T / sec, "ms_per_step": sec * 1e3, "rmsnorm_ms": ms,
            "rmsnorm_GBs": nbytes / (ms * 1e-3) / 1e9}


def grouped_measure(steps, warmup, plain_route_ms):
    """The V3 prefill layer with node-limited routing (8 groups of 32 experts,
    top-4 groups): layer throughput and the router's own time."""
    spec = synth.get_config(GROUPED)
    inp, layer, bufs = setup(spec)
    x, bias = inp["x"], inp["bias"]
    sec = time_steps(layer, x, bias, bufs, steps, warmup)
    out = {"workload": GROUPED, "groups": spec.n_groups, "topk_groups": spec.topk_groups,
           "tokens_per_s": spec.T / sec, "ms_per_step": sec * 1e3,
           "layer_TFLOPs": spec.flops() / sec / 1e12,
           "layer_frac_mfma_peak": spec.flops() / sec / 1e12 / MFMA_BF16_PEAK_TFLOPS,
           "route_ms": route_ms(layer, x, bias), "route_ms_without_groups": plain_route_ms}
    del inp, layer, bufs
    torch.cuda.empty_cache()
    return out


def ep8_measure(steps, warmup):
    """One GPU's share of the V3 prefill layer under 8-way expert
    parallelism (32 local experts, 2048 routed rows each; the collectives
    that would move those rows are not part of it): the same GEMM flops as
    the single-GPU layer on 1/8 of its weights, so every token tile is full
    and the launches are MFMA-bound."""
    spec = synth.get_config(EP8)
    inp, layer, bufs = setup(spec)
    x, bias = inp["x"], inp["bias"]
    timer = Timed()
    step_ms = []
    sec = time_steps(layer, x, bias, bufs, steps, warmup, timer, step_ms)
    gms = timer.mean_ms()
    tf = spec.flops() / sec / 1e12
    gtf = gate_up_flops(spec, shared=layer.side is None) / (gms * 1e-3) / 1e12
    out = {"workload": EP8, "tokens_per_s": spec.T / sec, "ms_per_step": sec * 1e3,
           **spread(step_ms), "routed_rows": spec.T * spec.K,
           "layer_TFLOPs": tf, "layer_frac_mfma_peak": tf / MFMA_BF16_PEAK_TFLOPS,
           "gate_up_ms": gms, "gate_up_TFLOPs": gtf,
           "gate_up_mfma_frac": gtf / MFMA_BF16_PEAK_TFLOPS}
    log(f"[bench] ep8 shard: {sec*1e3:.3f} ms/step, layer {tf:.0f} TFLOP/s, gate/up {gms:.3f} ms "
        f"({gtf:.0f} TFLOP/s)")
    del inp, layer, bufs
    torch.cuda.empty_cache()
    return out


def fp8_gate_up_bytes(spec) -> float:
    """Algorithmic HBM bytes of one fine-grained fp8 gate/up launch: W1 and W3
    codes of every routed and shared expert once with their 128 x 128 block
    scales, the quantised x and its tile scales once, h and the shared h
    written once as codes with their tile scales."""
    TK, SI, d, I = spec.T * spec.K, spec.S * spec.Is, spec.d, spec.I
    w = (spec.E * 2 * I + 2 * SI) * d * (1 + 4 / (128 * 128))
    return float(w + spec.T * d * (1 + 4 / 128) + (TK * I + spec.T * SI) * (1 + 4 / 128))


def fp8_measure(steps, warmup):
    """The V3 prefill layer in fine-grained fp8 (128 x 128 weight blocks,
    1 x 128 activation tiles; router and combine as in bf16): tokens/s, and
    the gate/up launch against the HBM and fp8 MFMA rooflines."""
    spec = synth.get_config(FP8B)
    inp = synth.make_inputs(spec, "cuda")
    layer = moe.MoELayer(spec, inp, max_tokens=spec.T)
    x, bias = inp["x"], inp["bias"]
    T, K, I, SI = spec.T, spec.K, spec.I, spec.S * spec.Is
    cfg = layer._cfg(T)
    hq = torch.empty((T * K, I), dtype=torch.uint8, device="cuda")
    hs = torch.empty((T * K, I // 128), dtype=torch.float32, device="cuda")
    hsq = torch.empty((T, SI), dtype=torch.uint8, device="cuda")
    hss = torch.empty((T, SI // 128), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(moe.moe_workspace_size(cfg, moe.MOE_WS_GEMM), 256), dtype=torch.uint8,
                     device="cuda")
    w = layer.w

    def step(timer=None):
        layer.route(x, bias)
        layer.permute(cfg, x, gather=False)
        moe.moe_quantize_act(cfg, x, layer.xq[:T], layer.xs[:T])

        def gate_up():
            moe.moe_experts_fp8_gate_up(cfg, layer.xq[:T], layer.xs[:T], layer.expert_offsets,
                                        layer.perm_slot[:T * K], w["w1"], w["s1"], w["s3"],
                                        w["w1s"], w["s1s"], w["s3s"], hq, hs, hsq, hss, ws=ws)
        if timer is not None:
            with timer:
                gate_up()
        else:
            gate_up()
        moe.moe_experts_fp8_down(cfg, hq, hs, hsq, hss, layer.expert_offsets,
                                 layer.perm_slot[:T * K], layer.topk_gate[:T], w["w2"], w["s2"],
                                 w["w2s"], w["s2s"], layer.out_slots[:T * K], layer.y_shared[:T],
                                 ws=ws)
        layer.combine(cfg)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    timer = Timed()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    gms = timer.mean_ms()
    flops, nbytes = gate_up_flops(spec), fp8_gate_up_bytes(spec)
    quant_ms = per_launch_ms(lambda: moe.moe_quantize_act(cfg, x, layer.xq[:T], layer.xs[:T]))
    out = {"workload": FP8B, "tokens_per_s": T / sec, "ms_per_step": sec * 1e3,
           "gate_up_ms": gms, "gate_up_algorithmic_bytes": nbytes,
           "gate_up_GBs": nbytes / (gms * 1e-3) / 1e9,
           "gate_up_hbm_frac": nbytes / (gms * 1e-3) / 1e9 / HBM_PEAK_GBS,
           "gate_up_TFLOPs": flops / (gms * 1e-3) / 1e12,
           "gate_up_mfma_fp8_frac": flops / (gms * 1e-3) / 1e12 / MFMA_FP8_PEAK_TFLOPS,
           "flop_per_byte": flops / nbytes, "quantize_act_ms": quant_ms,
           "gate_up_traffic": measured_traffic(TRAFFIC_FILE_FP8),
           "layer_TFLOPs": spec.flops() / sec / 1e12,
           "layer_frac_mfma_fp8_peak": spec.flops() / sec / 1e12 / MFMA_FP8_PEAK_TFLOPS}
    log(f"[bench] fp8 prefill: {sec*1e3:.3f} ms/step, {T/sec:.0f} tok/s, gate/up {gms:.3f} ms "
        f"({out['gate_up_TFLOPs']:.0f} TFLOP/s, {out['gate_up_GBs']:.0f} GB/s algorithmic)")
    del inp, layer, hq, hs, hsq, hss, ws
    torch.cuda.empty_cache()
    return out


def measured_peaks():
    """Achievable peaks on this GPU, beside the nominal ones. From the probes
    of libmoe_peaks.so: a loop of independent MFMAs of each instruction form
    (8 waves per block, 1024 blocks, operands changing from one instruction
    to the next), an fp32 FMA loop, and a 16-byte-load streaming read (plain
    and non-temporal loads) and copy of 2 GiB. For reference also torch's copy of 1 GiB and the vendor
    BLAS bf16 GEMM at 8192^3. Also the L2 -> CU read rate (each CU
    re-reading 64 KB), against which the GEMMs' L2 -> CU operand traffic
    can be set."""
    loops = {form: pk.measure_mfma(form, blocks=1024, iters=iters)
             for form, iters in (("bf16_32x32x16", 4096), ("bf16_16x16x32", 4096),
                                 ("fp8_32x32x64", 2048), ("fp8_16x16x128", 2048),
                                 ("f32_fma", 16384))}
    stream = pk.measure_stream(1 << 31, reps=10)
    l2 = pk.measure_l2()
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    copy_ms = per_launch_ms(lambda: dst.copy_(src), 10)
    del src, dst
    a = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    b = torch.randn((8192, 8192), device="cuda").to(torch.bfloat16)
    c = torch.empty((8192, 8192), dtype=torch.bfloat16, device="cuda")
    gemm_ms = per_launch_ms(lambda: torch.matmul(a, b, out=c), 10)
    del a, b, c
    torch.cuda.empty_cache()
    return {"mfma_loop_TFLOPs": loops,
            "mfma_bf16_TFLOPs": max(loops["bf16_32x32x16"], loops["bf16_16x16x32"]),
            "mfma_fp8_TFLOPs": max(loops["fp8_32x32x64"], loops["fp8_16x16x128"]),
            "fma_f32_TFLOPs": loops["f32_fma"],
            "stream_read_GBs": stream["read_GBs"], "stream_read_nt_GBs": stream["read_nt_GBs"],
            "stream_copy_GBs": stream["copy_GBs"],
            "l2_read_GBs": l2,
            "copy_GBs": 2.0 * (1 << 30) / (copy_ms * 1e-3) / 1e9,
            "blas_bf16_TFLOPs": 2.0 * 8192 ** 3 / (gemm_ms * 1e-3) / 1e12,
            "copy": "torch copy_ of 2^28 fp32", "blas": "torch.matmul bf16 8192 x 8192 x 8192"}


def attach_measured_fractions(result, peaks):
    """Every rate of the run as a fraction of the measured peak of the same
    resource (best MFMA loop of its dtype, fp32 FMA loop, streaming read),
    beside the fractions of the published peaks already in the line."""
    bf16, fp8, f32 = peaks["mfma_bf16_TFLOPs"], peaks["mfma_fp8_TFLOPs"], peaks["fma_f32_TFLOPs"]
    rd = peaks["stream_read_GBs"]
    result["layer_frac_measured_mfma"] = result["layer_TFLOPs"] / bf16
    rl = result["roofline"]
    rl["frac_of_measured_read"] = rl["achieved"] / rd
    rl["frac_of_measured_copy"] = rl["achieved"] / peaks["copy_GBs"]
    rl["mfma_frac_of_measured_loop"] = rl["mfma_TFLOPs"] / bf16
    rl["mfma_frac_of_own_form_loop"] = rl["mfma_TFLOPs"] / peaks["mfma_loop_TFLOPs"]["bf16_32x32x16"]
    rl["mfma_frac_of_measured_blas"] = rl["mfma_TFLOPs"] / peaks["blas_bf16_TFLOPs"]
    if "decode" in result:
        # the decode GEMMs load their weights with the non-temporal hint:
        # set them against the streaming read of the same load form
        rdn = peaks["stream_read_nt_GBs"]
        result["decode"]["frac_of_measured_read"] = result["decode"]["achieved_GBs"] / rdn
        result["decode"]["graph_frac_of_measured_read"] = result["decode"]["graph_achieved_GBs"] / rdn
    if "fp8_prefill" in result:
        f = result["fp8_prefill"]
        f["gate_up_frac_of_measured_read"] = f["gate_up_GBs"] / rd
        f["gate_up_frac_of_measured_fp8_loop"] = f["gate_up_TFLOPs"] / fp8
        f["layer_frac_measured_fp8_mfma"] = f["layer_TFLOPs"] / fp8
    if "grouped" in result:
        g = result["grouped"]
        g["layer_frac_measured_mfma"] = g["layer_TFLOPs"] / bf16
    if "ep8_shard" in result:
        e = result["ep8_shard"]
        e["layer_frac_measured_mfma"] = e["layer_TFLOPs"] / bf16
        e["gate_up_frac_of_measured_loop"] = e["gate_up_TFLOPs"] / bf16
        e["gate_up_frac_of_own_form_loop"] = e["gate_up_TFLOPs"] / peaks["mfma_loop_TFLOPs"]["bf16_32x32x16"]
    if "stress" in result:
        result["stress"]["frac_of_measured"] = result["stress"]["layer_TFLOPs"] / bf16
    for o in result.get("other_configs", []):
        o["frac_of_measured"] = o["layer_TFLOPs"] / (f32 if o["peak_TFLOPs"] == FP32_VECTOR_PEAK_TFLOPS
                                                     else bf16)


def stress_measure():
    """The skewed-load workload: 20 batches of 32768 tokens whose router rows
    give expert popularity Zipf(1.1) (hottest about 10x the mean), each layer
    call followed by the bias update from zero (gamma 1e-3): tokens/s over the
    20 (forward + update) and each batch's max/mean load."""
    spec = synth.get_config(STRESS)
    inp = synth.make_inputs(spec, "cuda")
    layer = moe.MoELayer(spec, inp, max_tokens=spec.T)
    xs = [inp["x"]] + [synth.make_x(spec, "cuda", batch=b) for b in range(1, spec.batches)]
    bias = torch.zeros(spec.E, dtype=torch.float32, device="cuda")
    layer.forward(xs[0], bias)              # warm-up; the timed run starts from zero bias
    torch.cuda.synchronize()
    bias.zero_()
    loads = []
    t0 = time.perf_counter()
    for x in xs:
        layer.forward(x, bias)
        loads.append(layer.load.clone())
        layer.bias_update(bias)
    torch.cuda.synchronize()
    sec = time.perf_counter() - t0
    ratio = [float(l.max() / l.float().mean()) for l in (t.cpu() for t in loads)]
    upd_ms = per_launch_ms(lambda: moe.moe_bias_update(spec.E, layer.load, 0.0, bias), 20)
    tf = spec.batches * spec.flops() / sec / 1e12
    out = {"workload": STRESS, "batches": spec.batches, "tokens_per_batch": spec.T,
           "tokens_per_s": spec.batches * spec.T / sec, "ms_per_batch": sec * 1e3 / spec.batches,
           "layer_TFLOPs": tf, "peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
           "frac": tf / MFMA_BF16_PEAK_TFLOPS,
           "max_over_mean_load": ratio, "max_violation_first_last": [ratio[0] - 1, ratio[-1] - 1],
           "bias_update_ms": upd_ms}
    log(f"[bench] stress: {out['ms_per_batch']:.2f} ms/batch, max/mean {ratio[0]:.2f} -> {ratio[-1]:.2f}")
    del inp, layer, xs, bias
    torch.cuda.empty_cache()
    return out


FP32_VECTOR_PEAK_TFLOPS = 157.3    # MI355X fp32 vector


def forward_measure(name, steps, warmup):
    """A named workload through MoELayer.forward (its default path), timed
    over `steps` layer calls: tokens/s and layer TFLOP/s against the peak of
    its arithmetic (bf16 MFMA, or fp32 vector for the fp32 layer)."""
    spec = synth.get_config(name)
    inp = synth.make_inputs(spec, "cuda")
    layer = moe.MoELayer(spec, inp, max_tokens=spec.T)
    x, bias = inp["x"], inp["bias"]
    for _ in range(warmup):
        layer.forward(x, bias)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.forward(x, bias)
    torch.cuda.synchronize()
    sec = (time.perf_counter() - t0) / steps
    tf = spec.flops() / sec / 1e12
    peak = FP32_VECTOR_PEAK_TFLOPS if spec.act_dtype == "f32" else MFMA_BF16_PEAK_TFLOPS
    # the same call recorded once into a HIP graph and replayed (no host
    # launch work per call)
    xg = x.clone()
    graph = layer.capture(xg, bias)
    gsec = per_launch_ms(graph.replay, steps) * 1e-3
    del inp, layer, graph, xg
    torch.cuda.empty_cache()
    return {"workload": name, "tokens": spec.T, "tokens_per_s": spec.T / sec,
            "ms_per_step": sec * 1e3, "layer_TFLOPs": tf, "peak_TFLOPs": peak, "frac": tf / peak,
            "graph_ms_per_step": gsec * 1e3, "graph_tokens_per_s": spec.T / gsec}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-tokens", type=int, default=None,
                    help="tokens of the oracle baseline and parity check (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-grouped", action="store_true")
    ap.add_argument("--no-fp8", action="store_true")
    ap.add_argument("--no-stress", action="store_true")
    ap.add_argument("--no-ep8", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="before timing, run one 1 GiB read + 1 GiB write elementwise kernel, "
                         "the known-size reference for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this layer's path is built and timed on a single "
              "MI355X (no expert sharding or collectives); run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    moe.load_library()

    if args.calibrate_copy:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)      # a kernel no other step launches, so counters can select it
        torch.cuda.synchronize()
        del src, dst
        log("[bench] calibration copy: 1 GiB read, 1 GiB written")
    spec = synth.get_config(WORKLOAD)
    log(f"[bench] generating {WORKLOAD} inputs on the GPU")
    inp, layer, bufs = setup(spec)
    x, bias = inp["x"], inp["bias"]
    gate_timer = Timed()
    log(f"[bench] warmup {args.warmup}, timing {args.steps} steps")
    step_ms = []
    sec = time_steps(layer, x, bias, bufs, args.steps, args.warmup, gate_timer, step_ms)
    tokens_per_s = spec.T / sec
    gate_ms = gate_timer.mean_ms()
    shared_in_launch = layer.side is None   # else the shared FFN runs on the second stream
    gate_flops = gate_up_flops(spec, shared_in_launch)
    gate_bytes = gate_up_bytes(spec, shared_in_launch)
    achieved = gate_flops / (gate_ms * 1e-3) / 1e12
    achieved_gbs = gate_bytes / (gate_ms * 1e-3) / 1e9
    layer_tflops = spec.flops() / sec / 1e12
    load = layer.load.cpu().numpy()
    log(f"[bench] {sec*1e3:.3f} ms/step, {tokens_per_s:.0f} tok/s, gate/up {gate_ms:.3f} ms "
        f"({achieved:.0f} TFLOP/s, {achieved_gbs:.0f} GB/s algorithmic)")

    result = {
        "metric": "MoE-layer tokens/s at V3 shape (T=8192) + % MFMA peak; decode % HBM peak",
        "value": tokens_per_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": sec * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD, "tokens": spec.T, "hidden": spec.d, "routed_experts": spec.E,
                   "top_k": spec.K, "inter": spec.I, "shared_experts": spec.S,
                   "shared_inter": spec.Is, "weights": "bf16", "output": "fp32",
                   "slots": layer.slot_dtype, "parallelism": "single GPU"},
        **spread(step_ms),
        "layer_TFLOPs": layer_tflops,
        "layer_frac_mfma_peak": layer_tflops / MFMA_BF16_PEAK_TFLOPS,
        "load_max_over_mean": float(load.max() / load.mean()),
        # The routed experts' gate/up launch does 4*d*I flops per (token,
        # slot) on weights it must stream once: 250 flop/B at this shape,
        # below the MI355X ridge (2500 TFLOP/s / 8 TB/s = 312 flop/B), so the
        # roofline that binds it is HBM; the MFMA view is reported beside it.
        "roofline": {"kernel": ("grouped_gemm_mfma<gate/up, bf16, 256-token tiles, "
                                + ("shared + routed>" if shared_in_launch else "routed>")),
                     "bound": "hbm",
                     "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": measured_traffic(),
                     # traffic is not counted in this run: it comes from the
                     # committed FETCH_SIZE / WRITE_SIZE summary, and is null
                     # unless that was taken on the current kernel sources
                     "traffic_source": ("profiles/gate_up_v3_prefill_traffic.txt (rocprofv3 "
                                        "FETCH_SIZE + WRITE_SIZE, kernel_src_sha "
                                        f"{kernel_source_hash()})"
                                        if measured_traffic() is not None else None),
                     "algorithmic_bytes_per_launch": gate_bytes,
                     "algorithmic_flops_per_launch": gate_flops, "avg_launch_ms": gate_ms,
                     "flop_per_byte": gate_flops / gate_bytes,
                     "mfma_TFLOPs": achieved, "mfma_peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                     "mfma_frac": achieved / MFMA_BF16_PEAK_TFLOPS},
    }
    other = other_slots_measure(layer, x, bias, bufs, args.steps, args.warmup)
    log(f"[bench] the same step with {other['slot_dtype']} slot rows: {other['ms_per_step']:.3f} ms")
    result[f"{other['slot_dtype']}_slots"] = other
    plain_route = route_ms(layer, x, bias)
    result["route_ms"] = plain_route
    result["sequence_loads_ms"] = sequence_loads_ms(layer, spec, seq_len=4096)
    log("[bench] prefill layer with pre-norm and residual")
    result["norm_residual"] = norm_residual_measure(layer, spec, x, bias, bufs, args.steps,
                                                    args.warmup)
    if not args.no_cpu_baseline:
        n_cpu = spec.T if args.cpu_tokens is None else args.cpu_tokens
        log(f"[bench] oracle cpu baseline on {n_cpu} tokens")
        result["cpu_baseline"], result["parity_sample"] = cpu_baseline(spec, inp, layer, bufs,
                                                                       n_cpu)
        log(f"[bench] oracle {result['cpu_baseline']['sample']}; parity {result['parity_sample']}")
    del inp, layer, bufs
    torch.cuda.empty_cache()
    if not args.no_decode:
        log(f"[bench] decode workload {DECODE}")
        result["decode"] = decode_measure(args.steps, args.warmup)
    if not args.no_grouped:
        log(f"[bench] node-limited routing workload {GROUPED}")
        result["grouped"] = grouped_measure(args.steps, args.warmup, plain_route)
    if not args.no_fp8:
        log(f"[bench] fine-grained fp8 workload {FP8B}")
        result["fp8_prefill"] = fp8_measure(args.steps, args.warmup)
    if not args.no_ep8:
        log(f"[bench] one GPU's expert-parallel share {EP8}")
        result["ep8_shard"] = ep8_measure(args.steps, args.warmup)
    if not args.no_stress:
        log(f"[bench] skewed-load workload {STRESS}")
        result["stress"] = stress_measure()
    log("[bench] the tiny fp32 and the 2024-layout workloads")
    result["other_configs"] = [forward_measure(n, args.steps, args.warmup)
                               for n in ("tiny_f32", "dsmoe2024_bf16")]
    log("[bench] measured peaks (MFMA / FMA loops, streaming read and copy)")
    peaks = measured_peaks()
    result["measured_peaks"] = peaks
    attach_measured_fractions(result, peaks)
    # matrix-core busy share of the GEMM launches, from the committed counter
    # run (null when the kernels changed since it was taken)
    util = measured_mfma_util()
    result["roofline"]["mfma_busy_pct"] = util.get("v3_gate_up")
    result["mfma_busy_pct_counters"] = util or None
    # the clock the part ran the GEMMs at (power-limited below the 2.4 GHz of
    # the published peak), from the committed counter run
    clock = measured_clock()
    result["roofline"]["clock_ghz"] = clock.get("v3_gate_up", {}).get("ghz")
    result["clock_counters"] = clock or None
    print(json.dumps(result), flush=True)
    if not result.get("parity_sample", {"pass": True})["pass"]:
        print("bench.py: the layer output does not match the oracle (parity_sample)", file=sys.stderr)
        sys.exit(1)


if __name__ == "__main__":
    main()
