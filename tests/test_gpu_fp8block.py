"""Fine-grained fp8 experts ("DeepSeekMoE架构解析" section 4.3) against the
oracle: moe_quantize_act bit-exact (codes and scales are decided in fp32 on
both sides), and the layer through moe_quantize_act + moe_experts_fp8 with
routing bit-exact up to near-ties and outputs within 2e-2 * RMS of the
oracle's fp64 evaluation on the same quantised tokens and block-scaled
weights. The intermediate h is quantised from each side's own value (fp32
on the GPU, fp64 rounded to fp32 in the oracle), so an h code may differ by
one step where the value sits near a rounding boundary. Such a code is an
integer decided by floating point, checked like a routing near-tie: every
differing code must be one the GPU can reach within the error bound of its
fp8 MFMA accumulation (measured, see EPS_MFMA), and the outputs are
compared with the oracle's down projection of the GPU's (validated) h
codes."""

import numpy as np
import pytest
import torch

import mixture_experts_layer_40_amd as moe
import oracle
import synth
from gpu_parity import (STORE_REL, check_permutation, check_route, host, oracle_route, rel_err,
                        run_steps, say, slot_storage_allowance)

pytestmark = pytest.mark.gpu

TOL = 2e-2


def _cfg(**kw):
    name = "fp8b_" + "_".join(f"{k}{v}" for k, v in sorted(kw.items()))
    return synth.scaled_config("v3_prefill_fp8b", name=name, **kw)


def _bank(inp, spec):
    def fetch(e):
        return (host(inp["w1"][e]), host(inp["w3"][e]), host(inp["w2"][e]),
                inp["s1"][e].cpu().numpy(), inp["s3"][e].cpu().numpy(), inp["s2"][e].cpu().numpy())
    shared = None
    if spec.S > 0:
        shared = tuple(host(inp[n]) for n in ("w1s", "w3s", "w2s")) + tuple(
            inp[n].cpu().numpy() for n in ("s1s", "s3s", "s2s"))
    return oracle.BlockExpertBank(fetch=fetch, shared=shared, S=spec.S)


@pytest.mark.parametrize("T,d", [(1, 128), (300, 256), (1000, 7168), (4097, 512)])
def test_quantize_act_matches_oracle(T, d):
    spec = _cfg(T=T, d=d, E=8, K=2, I=128, Is=128)
    x = synth.make_x(spec, "cuda")
    if T >= 300:
        x[3, :128] = 0                            # an all-zero tile
        x[5, 128:256] = torch.tensor(1e-30)       # a scale near the fp32 normal limit
        x[7, :128] = -x[7, :128].abs() * 1e-7
        x[7, 0] = -1.0                            # negative values below half a step -> -0 codes
    cfg = moe.config_of(spec, T=T, weight_layout="tiled")
    xq = torch.empty((T, d), dtype=torch.uint8, device="cuda")
    xs = torch.empty((T, d // 128), dtype=torch.float32, device="cuda")
    moe.moe_quantize_act(cfg, x, xq, xs)
    torch.cuda.synchronize()
    cq, cs = oracle.quantize_x(host(x))
    got_q, got_s = xq.cpu().numpy(), xs.cpu().numpy()
    assert np.array_equal(got_s, cs), f"{int((got_s != cs).sum())} scales differ"
    assert np.array_equal(got_q, cq), f"{int((got_q != cq).sum())} of {cq.size} codes differ"


CASES = {
    # ragged: 300 tokens over 64 experts (K = 6), two tiles of d and I
    "small": _cfg(T=300, d=256, E=64, K=6, I=256, Is=256),
    # fused router (T >= 4096), 256 experts, up to 4 token fragments per tile
    "many_experts": _cfg(T=4100, d=128, E=256, K=8, I=128, Is=128),
    # decode-like: one token fragment per expert, wider hidden
    "decode_like": _cfg(T=64, d=1024, E=64, K=8, I=384, Is=256),
    # no shared expert; two shared experts concatenated
    "no_shared": _cfg(T=257, d=256, E=32, K=4, I=256, S=0, Is=256),
    "two_shared": _cfg(T=200, d=384, E=16, K=4, I=128, S=2, Is=256),
}

# The fp8 MFMA of gfx950 (v_mfma_scale_f32_32x32x64_f8f6f4) aligns its 64
# products and its C input to the largest before summing: measured on the
# GPU, |error| <= 2^-12 (sum |a b| + |C|) per instruction (in-bounds probe,
# random E4M3 codes of every binade; exact when the products share a
# binade). The kernel sums each 128-wide block in two chained MFMAs from
# zero and adds it to fp32 accumulators, so per block |error| <= 2 EPS
# sum_block |x w|, EPS = 2^-11 leaving a factor 2 of margin.
EPS_MFMA = 2.0 ** -11
_POS = oracle.E4M3_TABLE[:0x7F]


def _h_bound(xd, w1, w3):
    """Bound on |h_GPU - h_oracle| per element for dequantised tokens xd and
    expert weights w1, w3 (float64): the MFMA bound on g and u, carried
    through h = SiLU(g) u (|SiLU'| <= 1.1), plus the GPU's own fp32
    rounding of g, u and h."""
    ax = np.abs(xd)
    g, u = xd @ w1.T, xd @ w3.T
    dg = 2 * EPS_MFMA * (ax @ np.abs(w1).T) + 2.0 ** -22 * np.abs(g)
    du = 2 * EPS_MFMA * (ax @ np.abs(w3).T) + 2.0 ** -22 * np.abs(u)
    sg = np.abs(oracle.silu(g))
    return 1.1 * dg * (np.abs(u) + du) + sg * du + 2.0 ** -22 * sg * np.abs(u)


def _code_interval(c):
    """The interval of scaled values that round to E4M3 code c."""
    m = c.astype(np.int64) & 0x7F
    lo = np.where(m > 0, (_POS[np.maximum(m - 1, 0)] + _POS[m]) / 2, 0.0)
    hi = np.where(m < 0x7E, (_POS[m] + _POS[np.minimum(m + 1, 0x7E)]) / 2, 464.0)
    neg = (c >> 7) == 1
    lo = np.where(m == 0, -_POS[1] / 2, lo)
    return np.where(neg, -hi, lo), np.where(neg, -lo, hi)


def _check_h(gq, gs, h32, dh, counts):
    """The GPU's quantised h rows against the oracle's h (fp32 values before
    quantisation) and the bound dh on their difference: each tile scale
    within the bound the max-abs can move (dh max / 448); codes equal,
    except where the oracle's scaled value q lies within the bound of the
    GPU code's rounding interval. Returns the oracle's codes and scales."""
    oq, os_ = oracle.quantize_tiles(h32)
    n, C = h32.shape
    ds = dh.reshape(n, C // 128, 128).max(axis=2) / 448.0 + 2.0 ** -23 * os_
    assert np.all(np.abs(gs.astype(np.float64) - os_) <= ds), "an h tile scale is outside its bound"
    diff = gq != oq
    counts[0] += int(diff.sum())
    counts[1] += diff.size
    if diff.any():
        sf = np.repeat(os_.astype(np.float64), 128, axis=1)
        dsf = np.repeat(ds, 128, axis=1)
        q = h32.astype(np.float64) / sf
        dq = (dh + np.abs(q) * dsf) / (sf - dsf)
        lo, hi = _code_interval(gq[diff])
        dist = np.maximum(0.0, np.maximum(lo - q[diff], q[diff] - hi))
        worst = int(np.argmax(dist / dq[diff]))
        assert np.all(dist <= dq[diff]), (
            f"an h code is outside the accumulation bound: GPU {int(gq[diff][worst])}, "
            f"oracle {int(oq[diff][worst])}, q {q[diff][worst]:.6g}, bound {dq[diff][worst]:.3g}")
    return oq, os_


def _split_calls(layer, spec):
    """The two launches with the quantised h held here; asserts they equal
    the layer's fused call bit for bit."""
    T, K, I, SI = spec.T, spec.K, spec.I, spec.S * spec.Is
    cfg, w = layer._cfg(T), layer.w
    hq = torch.empty((T * K, I), dtype=torch.uint8, device="cuda")
    hs = torch.empty((T * K, I // 128), dtype=torch.float32, device="cuda")
    hsq = torch.empty((T, SI), dtype=torch.uint8, device="cuda") if SI else None
    hss = torch.empty((T, SI // 128), dtype=torch.float32, device="cuda") if SI else None
    moe.moe_experts_fp8_gate_up(cfg, layer.xq[:T], layer.xs[:T], layer.expert_offsets,
                                layer.perm_slot[:T * K], w["w1"], w["s1"], w["s3"], w.get("w1s"),
                                w.get("s1s"), w.get("s3s"), hq, hs, hsq, hss)
    out2 = torch.empty_like(layer.out_slots[:T * K])
    ysh2 = torch.empty_like(layer.y_shared[:T]) if SI else None
    moe.moe_experts_fp8_down(cfg, hq, hs, hsq, hss, layer.expert_offsets, layer.perm_slot[:T * K],
                             layer.topk_gate[:T], w["w2"], w["s2"], w.get("w2s"), w.get("s2s"),
                             out2, ysh2)
    torch.cuda.synchronize()
    assert torch.equal(out2, layer.out_slots[:T * K]), "split calls differ from the fused call"
    if SI:
        assert torch.equal(ysh2, layer.y_shared[:T])
    return (hq.cpu().numpy(), hs.cpu().numpy(),
            None if hsq is None else hsq.cpu().numpy(), None if hss is None else hss.cpu().numpy())


def _layer_check(spec, inp, rows=None):
    """Routing bit-exact up to near-ties; the quantised tokens bit-exact; h
    codes validated (_check_h); the outputs against the oracle's down
    projection of the GPU's validated h codes, within 2e-2 x RMS."""
    layer, res = run_steps(spec, inp, bias=inp.get("bias"))
    r, _ = oracle_route(spec, inp["x"], inp["wr"], inp.get("bias"))
    n_near = check_route(spec, r, res["idx"], res["gate"], res["load"])
    check_permutation(spec, res["idx"], res["offsets"], res["perm"])
    T, K, d = spec.T, spec.K, spec.d
    rows = np.arange(T) if rows is None else np.asarray(rows)
    xq, xs = oracle.quantize_x(host(inp["x"][torch.as_tensor(rows, device="cuda")]))
    assert np.array_equal(layer.xq[:T].cpu().numpy()[rows], xq)
    assert np.array_equal(layer.xs[:T].cpu().numpy()[rows], xs)
    hq, hs, hsq, hss = _split_calls(layer, spec)
    bank = _bank(inp, spec)
    gpu_idx = res["idx"][rows]           # equal to the oracle's sets up to validated near-ties
    gate = oracle.gate_values(r["scores"][rows], gpu_idx, spec.norm)   # GPU slot order
    pos = np.empty(T * K, dtype=np.int64)
    pos[res["perm"]] = np.arange(T * K)                 # slot -> row of hq
    counts = [0, 0]
    routed = np.zeros((len(rows), K, d))
    pure = np.zeros((len(rows), K, d))                  # the oracle with its own h codes
    for e in np.unique(gpu_idx):
        ri, ks = np.nonzero(gpu_idx == e)
        w1, w3, w2 = bank.expert(int(e))
        h32 = oracle.expert_h_fp8(xq[ri], xs[ri], w1, w3)
        p = pos[rows[ri] * K + ks]
        dh = _h_bound(oracle.dequantize_tiles(xq[ri], xs[ri]), w1, w3)
        oq, os_ = _check_h(hq[p], hs[p], h32, dh, counts)
        routed[ri, ks] = gate[ri, ks][:, None] * (oracle.dequantize_tiles(hq[p], hs[p]) @ w2.T)
        pure[ri, ks] = gate[ri, ks][:, None] * (oracle.dequantize_tiles(oq, os_) @ w2.T)
    y_sh = np.zeros((len(rows), d))
    y_sh_pure = np.zeros((len(rows), d))
    if spec.S > 0:
        SI = spec.S * spec.Is
        W1, W3, W2 = (np.concatenate(m, axis=a) for m, a in
                      zip(zip(*bank.shared_experts()), (0, 0, 1)))
        h32 = oracle.expert_h_fp8(xq, xs, W1, W3)
        dh = _h_bound(oracle.dequantize_tiles(xq, xs), W1, W3)
        oq, os_ = _check_h(hsq[rows], hss[rows], h32, dh, counts)
        y_sh = oracle.dequantize_tiles(hsq[rows], hss[rows]) @ W2.T
        y_sh_pure = oracle.dequantize_tiles(oq, os_) @ W2.T
        assert SI % 128 == 0
        e_s, _ = rel_err(layer.y_shared[torch.as_tensor(rows, device="cuda")].double().cpu().numpy(), y_sh)
        assert e_s <= TOL, f"y_shared: {e_s:.3e}"
    trow = torch.as_tensor(rows, device="cuda")
    y_or = y_sh + routed.sum(axis=1)
    y = res["y"][trow].double().cpu().numpy()
    e_y, rms = rel_err(y, y_or, slot_storage_allowance("bf16", routed))
    assert e_y <= TOL, f"y: max err / RMS = {e_y:.3e}"
    slot_rows = (trow[:, None] * K + torch.arange(K, device="cuda")[None, :]).reshape(-1)
    osl = layer.out_slots[slot_rows].double().cpu().numpy().reshape(len(rows), K, d)
    rms_row = np.sqrt(np.mean(routed ** 2, axis=2, keepdims=True))
    excess = np.abs(osl - routed) - STORE_REL["bf16"] * np.abs(routed)
    e_o = float((excess / np.maximum(rms_row, 1e-300)).max())
    assert e_o <= TOL, f"out_slots: {e_o:.3e}"
    e_pure, _ = rel_err(y, y_sh_pure + pure.sum(axis=1))
    say(f"[fp8b] h codes within the accumulation bound of a boundary: {counts[0]} of {counts[1]}; "
        f"y err / RMS {e_y:.2e} (against the oracle's own h codes: {e_pure:.2e})")
    return n_near, e_y


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_block_layer_matches_oracle(name):
    spec = CASES[name]
    say(f"[fp8b] {name}")
    inp = synth.make_inputs(spec, "cuda")
    n_near, e_y = _layer_check(spec, inp)
    say(f"[fp8b] {name}: near-ties={n_near} y_err/rms={e_y:.3e}")


@pytest.mark.timeout(600)
def test_fullsize_v3_fp8_block():
    spec = synth.get_config("v3_prefill_fp8b")
    inp = synth.make_inputs(spec, "cuda")
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(spec.T, 10, replace=False))
    n_near, e_y = _layer_check(spec, inp, rows=rows)
    say(f"[fp8b] full V3: near-ties={n_near} y_err/rms={e_y:.3e}")
