"""Fine-grained fp8 experts ("DeepSeekMoE架构解析" section 4.3) against the
oracle: moe_quantize_act bit-exact (codes and scales are decided in fp32 on
both sides), and the layer through moe_quantize_act + moe_experts_fp8 with
routing bit-exact up to near-ties.

The intermediate h is quantised from each side's own value (fp32 on the GPU
from fp8 MFMA partial sums; float64 rounded to fp32 in the oracle), so an h
code may differ by a step where the value sits near a rounding boundary: an
integer decided by floating point, treated like a routing near-tie. The
window for that comes from the page alone: fp8 GEMM accumulation inside the
matrix unit keeps about 14 bits (section 4.3), read as g and u within
2^-14 sum |x w| of their exact values, plus the fp32 promotion of each
128-wide block and the fp32 SiLU and product, carried through h from the
oracle's own operands. Three comparisons:
  * validity: every GPU h code the oracle does not produce lies within that
    window of its rounding interval, and every tile scale within the
    window's effect;
  * the outputs against the oracle's down projection of the GPU's
    (validated) h codes, within 2e-2 x RMS (the down GEMM's arithmetic);
  * the outputs against the oracle's own evaluation (its own h codes; no GPU
    value on the expected side), within 2e-2 x RMS plus B: what the h codes
    inside the window can move each output, the reachable code range times
    the scale, |W2| and the gate (an oracle-side quantity). The plain
    2e-2 x RMS does not hold here at any width: one code flipped at the top
    of a tile moves h by 32/448 of the tile's max, and the shared expert's
    output carries it unweighted (3.9e-2 x RMS measured at the full V3
    shape over the tokens of every tile edge).
The accuracy of a single fp8 MFMA instruction on this part is measured by
test_fp8_mfma_accumulation_bound; it is what makes the per-block fp32
promotion necessary, and none of the three comparisons uses it.
"""

import numpy as np
import pytest
import torch

import mixture_experts_layer_40_amd as moe
import oracle
import synth
from gpu_parity import (check_permutation, check_route, check_slot_rows, coverage_rows, host,
                        oracle_route, rel_err, run_steps, say)

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

# Accuracy of one fp8 MFMA instruction, measured on codes of every binade
# by test_fp8_mfma_accumulation_bound: gfx950's
# v_mfma_scale_f32_32x32x64_f8f6f4 aligns its products and C input to the
# largest before summing, within
#   |D - (A B^T + C)| <= MFMA_EPS (sum_k |a_k b_k| + |C|).
# The parity checks below do not use it.
MFMA_EPS = 2.0 ** -11
U32 = 2.0 ** -24                      # fp32 unit roundoff
_POS = oracle.E4M3_TABLE[:0x7F]

# In-unit accumulation precision the page states for fp8 GEMMs: about 14
# bits ("DeepSeekMoE架构解析" section 4.3). Read as: each 128-wide block sum
# the matrix unit forms is within 2^-14 of the magnitudes it accumulates.
PAGE_BITS = 14


def _g_page(xd, w):
    """|g_GPU - g| for g = xd @ w.T (float64 from the dequantised operands)
    under the page's precision: each 128-wide block within 2^-14 of its
    sum |x w|, then promoted by one fp32 product of the two scales and one
    fp32 FMA into the accumulator (within 2^-24 of the scaled block and of
    the running sum): (2^-14 + 2 nb 2^-24) sum |x w| over the nb blocks."""
    S = np.abs(xd) @ np.abs(w).T
    nb = xd.shape[1] // 128
    return (2.0 ** -PAGE_BITS + 2 * nb * U32) * S


def _h_page(xd, w1, w3):
    """|h_GPU - h| per element for h = SiLU(g) u, g = xd w1^T, u = xd w3^T:
    the bounds on g and u carried through SiLU (|SiLU'| <= 1.1) and the
    product, plus the GPU's own evaluation of SiLU (fp32 exp and division)
    and of the product, within 2^-20 of the value."""
    g, u = xd @ w1.T, xd @ w3.T
    dg, du = _g_page(xd, w1), _g_page(xd, w3)
    sg, au = np.abs(oracle.silu(g)), np.abs(u)
    return 1.1 * dg * (au + du) + sg * du + 2.0 ** -20 * (sg + 1.1 * dg) * (au + du)


def _code_interval(c):
    """The interval of scaled values that round to E4M3 code c."""
    m = c.astype(np.int64) & 0x7F
    lo = np.where(m > 0, (_POS[np.maximum(m - 1, 0)] + _POS[m]) / 2, 0.0)
    hi = np.where(m < 0x7E, (_POS[m] + _POS[np.minimum(m + 1, 0x7E)]) / 2, 464.0)
    neg = (c >> 7) == 1
    lo = np.where(m == 0, -_POS[1] / 2, lo)
    return np.where(neg, -hi, lo), np.where(neg, -lo, hi)


def _window(h32, dh):
    """The oracle's quantisation of h (fp32 [n, C]) and what the GPU's may
    differ by, from dh (bound on |h_GPU - h|, float64): returns (codes,
    scales, dq, ds, delta) with dq the bound on the scaled value the code is
    decided from, ds the bound on each tile scale, and delta the bound on
    |h_GPU dequantised - h_oracle dequantised| per element: the codes
    reachable within dq of the oracle's scaled value (rounding is monotone)
    times the scale, plus the scale's own bound times the code."""
    oq, os_ = oracle.quantize_tiles(h32)
    n, C = h32.shape
    h64 = h32.astype(np.float64)
    dh = dh + U32 * np.abs(h64)                      # the oracle's own rounding to fp32
    ds = dh.reshape(n, C // 128, 128).max(axis=2) / 448.0 * (1 + U32) + 2 * U32 * os_
    sf = np.repeat(os_.astype(np.float64), 128, axis=1)
    dsf = np.repeat(ds, 128, axis=1)
    q = (h64 / sf).astype(np.float32).astype(np.float64)      # the oracle's decision input
    dq = (dh + np.abs(q) * dsf) / (sf - dsf) * (1 + 4 * U32) + 4 * U32 * np.abs(q)
    val = oracle.E4M3_TABLE
    c_lo = oracle.e4m3_encode(np.clip(q - dq, -448.0, 448.0))
    c_hi = oracle.e4m3_encode(np.clip(q + dq, -448.0, 448.0))
    v0 = val[oq]
    dval = np.maximum(np.abs(val[c_lo] - v0), np.abs(val[c_hi] - v0))
    vmax = np.maximum(np.abs(val[c_lo]), np.abs(val[c_hi]))
    delta = dval * (sf + dsf) + vmax * dsf
    return oq, os_, dq, ds, delta, c_lo != c_hi


def _check_h(gq, gs, h32, dh, counts):
    """The GPU's quantised h rows against the oracle's window (_window) for
    dh, the bound on |h_GPU - h| the page's accumulation precision gives:
    each tile scale within its bound; codes equal, except where the oracle's
    scaled value lies within dq of the GPU code's rounding interval. Returns
    the oracle's codes and scales and the per-element bound on what the
    GPU's dequantised h may differ by."""
    oq, os_, dq, ds, delta, cand = _window(h32, dh)
    assert np.all(np.abs(gs.astype(np.float64) - os_) <= ds), "an h tile scale is outside its bound"
    diff = gq != oq
    counts[0] += int(diff.sum())
    counts[1] += diff.size
    counts[2] += int(cand.sum())
    if diff.any():
        q = (h32.astype(np.float64) / np.repeat(os_.astype(np.float64), 128, axis=1))
        lo, hi = _code_interval(gq[diff])
        dist = np.maximum(0.0, np.maximum(lo - q[diff], q[diff] - hi))
        worst = int(np.argmax(dist / dq[diff]))
        assert np.all(dist <= dq[diff]), (
            f"an h code is outside the page's accumulation window: GPU {int(gq[diff][worst])}, "
            f"oracle {int(oq[diff][worst])}, q {q[diff][worst]:.6g}, bound {dq[diff][worst]:.3g}")
    return oq, os_, delta


def _codes(rng, shape, lo_exp=0, hi_exp=15):
    """Random finite E4M3 codes with exponent fields in [lo_exp, hi_exp]
    (0 = zero and subnormals, 15 = up to 448), random signs and mantissas."""
    e = rng.integers(lo_exp, hi_exp + 1, size=shape)
    m = rng.integers(0, 8, size=shape)
    m = np.where(e == 15, np.minimum(m, 6), m)          # 0x7F / 0xFF are NaN
    sgn = rng.integers(0, 2, size=shape)
    return ((sgn << 7) | (e << 3) | m).astype(np.uint8)


def test_fp8_mfma_accumulation_bound():
    """The accuracy MFMA_EPS states of v_mfma_scale_f32_32x32x64_f8f6f4
    (one instruction per problem through moe_probe_fp8_mfma): |D - (A B^T +
    C)| <= MFMA_EPS (sum |a b| + |C|) against the exact sums (every product
    of two E4M3 values, and every sum here, is exact in float64: products
    are multiples of 2^-18 below 2^18, C a float32 of magnitude >= 2^-4 or
    zero). Cases: codes of every binade with C = 0 (the first MFMA of a
    block) and with C the size of such a sum (the second), codes of a few
    neighbouring binades (the tile-scaled data of the GEMMs), and products
    of one binade."""
    from mixture_experts_layer_40_amd import peaks as pk
    rng = np.random.default_rng(20260211)
    n = 512
    cases = {
        "every binade, C = 0": (_codes(rng, (n, 32, 64)), _codes(rng, (n, 32, 64)), 0.0),
        "every binade, C ~ sum": (_codes(rng, (n, 32, 64)), _codes(rng, (n, 32, 64)), 1.0),
        "binades 10..15, C ~ sum": (_codes(rng, (n, 32, 64), 10), _codes(rng, (n, 32, 64), 10), 1.0),
        "one binade, C = 0": (_codes(rng, (n, 32, 64), 7, 7), _codes(rng, (n, 32, 64), 7, 7), 0.0),
    }
    worst = 0.0
    for name, (a, b, cmag) in cases.items():
        av, bv = oracle.E4M3_TABLE[a], oracle.E4M3_TABLE[b]
        prod = av @ np.swapaxes(bv, 1, 2)                            # [n, 32, 32], exact
        mag = np.abs(av) @ np.swapaxes(np.abs(bv), 1, 2)
        c = np.zeros((n, 32, 32), dtype=np.float32)
        if cmag:
            c = (rng.standard_normal((n, 32, 32)) * mag.mean()).astype(np.float32)
            c = np.where(np.abs(c) < 2.0 ** -4, np.float32(2.0 ** -4), c).astype(np.float32)
        d = torch.empty((n, 32, 32), dtype=torch.float32, device="cuda")
        pk.moe_probe_fp8_mfma(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(),
                              torch.from_numpy(c).cuda(), d)
        torch.cuda.synchronize()
        exact = prod + c.astype(np.float64)
        err = np.abs(d.cpu().numpy().astype(np.float64) - exact)
        denom = mag + np.abs(c)
        assert np.all(err[denom == 0] == 0)
        ratio = err / np.maximum(denom, 1e-300)
        worst = max(worst, float(ratio.max()))
        say(f"[fp8 mfma] {name}: max |err| / (sum |a b| + |C|) = 2^{np.log2(max(ratio.max(), 1e-300)):.2f}")
        assert np.all(ratio <= MFMA_EPS), f"{name}: 2^{np.log2(ratio.max()):.2f} > MFMA_EPS"
    say(f"[fp8 mfma] worst 2^{np.log2(max(worst, 1e-300)):.2f}, stated 2^{np.log2(MFMA_EPS):.0f}")


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
    projection of the GPU's validated h codes within 2e-2 x RMS, and against
    the oracle's own evaluation within 2e-2 x RMS + B. rows: the tokens whose outputs are checked (all by
    default), or a function of the GPU's routing results that picks them."""
    layer, res = run_steps(spec, inp, bias=inp.get("bias"))
    r, _ = oracle_route(spec, inp["x"], inp["wr"], inp.get("bias"))
    n_near = check_route(spec, r, res["idx"], res["gate"], res["load"])
    check_permutation(spec, res["idx"], res["offsets"], res["perm"])
    T, K, d = spec.T, spec.K, spec.d
    if callable(rows):
        rows = rows(res, r)
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
    counts = [0, 0, 0]
    routed = np.zeros((len(rows), K, d))
    pure = np.zeros((len(rows), K, d))                  # the oracle with its own h codes
    bound = np.zeros((len(rows), d))                    # B: what the window can move y by
    for e in np.unique(gpu_idx):
        ri, ks = np.nonzero(gpu_idx == e)
        w1, w3, w2 = bank.expert(int(e))
        h32 = oracle.expert_h_fp8(xq[ri], xs[ri], w1, w3)
        p = pos[rows[ri] * K + ks]
        xd = oracle.dequantize_tiles(xq[ri], xs[ri])
        oq, os_, delta = _check_h(hq[p], hs[p], h32, _h_page(xd, w1, w3), counts)
        g = gate[ri, ks][:, None]
        routed[ri, ks] = g * (oracle.dequantize_tiles(hq[p], hs[p]) @ w2.T)
        pure[ri, ks] = g * (oracle.dequantize_tiles(oq, os_) @ w2.T)
        np.add.at(bound, ri, np.abs(g) * (delta @ np.abs(w2).T))
    y_sh = np.zeros((len(rows), d))
    y_sh_pure = np.zeros((len(rows), d))
    if spec.S > 0:
        SI = spec.S * spec.Is
        W1, W3, W2 = (np.concatenate(m, axis=a) for m, a in
                      zip(zip(*bank.shared_experts()), (0, 0, 1)))
        h32 = oracle.expert_h_fp8(xq, xs, W1, W3)
        xd = oracle.dequantize_tiles(xq, xs)
        oq, os_, delta = _check_h(hsq[rows], hss[rows], h32, _h_page(xd, W1, W3), counts)
        y_sh = oracle.dequantize_tiles(hsq[rows], hss[rows]) @ W2.T
        y_sh_pure = oracle.dequantize_tiles(oq, os_) @ W2.T
        bound += delta @ np.abs(W2).T
        assert SI % 128 == 0
        e_s, _ = rel_err(layer.y_shared[torch.as_tensor(rows, device="cuda")].double().cpu().numpy(), y_sh)
        assert e_s <= TOL, f"y_shared: {e_s:.3e}"
    trow = torch.as_tensor(rows, device="cuda")
    y_or = y_sh + routed.sum(axis=1)
    y = res["y"][trow].double().cpu().numpy()
    e_y, rms = rel_err(y, y_or)
    assert e_y <= TOL, f"y against the down projection of the GPU's h codes: {e_y:.3e}"
    slot_rows = (trow[:, None] * K + torch.arange(K, device="cuda")[None, :]).reshape(-1)
    osl = layer.out_slots[slot_rows].double().cpu().numpy().reshape(len(rows), K, d)
    check_slot_rows(osl, routed, layer.slot_dtype, TOL)
    # the oracle's own evaluation: no GPU value on the expected side
    y_pure = y_sh_pure + pure.sum(axis=1)
    e_pure, rms_pure = rel_err(y, y_pure)
    excess = float(((np.abs(y - y_pure) - bound) / rms_pure).max())
    b_rel = float(bound.max() / rms_pure)
    say(f"[fp8b] h codes: {counts[0]} of {counts[1]} differ from the oracle's, {counts[2]} lie "
        f"within the page's accumulation precision of a rounding boundary; y err / RMS {e_y:.2e} "
        f"(GPU codes), {e_pure:.2e} (oracle's own codes; B <= {b_rel:.2e} x RMS, excess over B "
        f"{excess:.2e}) over {len(rows)} tokens")
    assert excess <= TOL, f"y against the oracle's own evaluation: {excess:.3e} x RMS beyond B"
    return n_near, e_y, e_pure


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_block_layer_matches_oracle(name):
    spec = CASES[name]
    say(f"[fp8b] {name}")
    inp = synth.make_inputs(spec, "cuda")
    n_near, e_y, e_pure = _layer_check(spec, inp)
    say(f"[fp8b] {name}: near-ties={n_near} y_err/rms={e_y:.3e} (oracle's own codes {e_pure:.3e})")


@pytest.mark.timeout(600)
def test_fullsize_v3_fp8_block():
    spec = synth.get_config("v3_prefill_fp8b")
    inp = synth.make_inputs(spec, "cuda")
    # the tokens owning the first and last row of every token tile (128-row
    # tiles in these kernels) of every expert, a few random ones, near-ties
    def rows(res, r):
        return coverage_rows(res["offsets"], res["perm"], spec, r["near_tie"], max_bm=128)
    n_near, e_y, e_pure = _layer_check(spec, inp, rows=rows)
    say(f"[fp8b] full V3: near-ties={n_near} y_err/rms={e_y:.3e} (oracle's own codes {e_pure:.3e})")
