"""Pins of the fp64 oracle to things other than itself.

Each test checks one oracle function against what the method's definition
fixes independently of the oracle's code: a hand-worked example, brute force
on tiny inputs, a library routine that is not the one the oracle calls,
closed forms and invariants. Chosen so that a plausible slip (a dropped term,
a wrong sign or index, a transposed operand, the bias leaking into the gates,
softmax instead of eq. (13), a dropped token) fails at least one of them.
"""

import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import moe as om


def _ev(s):
    """Evaluate a fixture expression: numbers, + - * / **, and log()."""
    return float(eval(str(s), {"__builtins__": {}}, {"log": math.log}))


def _arr(rows):
    return np.array([[_ev(v) for v in r] for r in rows], dtype=np.float64)


@pytest.fixture(scope="module")
def hand(golden_dir):
    with open(os.path.join(golden_dir, "hand_layer_e4k2.json")) as f:
        return json.load(f)


# --------------------------------------------------------------------------
# Hand-worked layer (eqs. 13-16, shared + routed experts)
# --------------------------------------------------------------------------

def _hand_bank(hand):
    exps = [(_arr(e["w1"]), _arr(e["w3"]), _arr(e["w2"])) for e in hand["experts"]]
    sh = hand["shared"]
    shared = (_arr(sh["w1"]), _arr(sh["w3"]), _arr(sh["w2"]), None, None, None)
    return oracle.ExpertBank(fetch=lambda e: exps[e] + (None, None, None), shared=shared, S=1)


def test_hand_worked_routing(hand):
    x, wr = _arr(hand["x"]), _arr(hand["wr"])
    bias = np.array([_ev(b) for b in hand["bias"]])
    r = oracle.route(x, wr, bias, hand["K"], "sigmoid", "selected")
    exp = hand["expected"]
    np.testing.assert_allclose(r["scores"], _arr(exp["scores"]), rtol=0, atol=1e-15)
    assert r["sel"].tolist() == exp["sel"]
    np.testing.assert_allclose(r["gate"], _arr(exp["gate"]), rtol=0, atol=1e-15)
    assert r["load"].tolist() == exp["load"]
    assert r["near_tie"].tolist() == exp["near_tie"]


def test_hand_worked_without_bias(hand):
    x, wr = _arr(hand["x"]), _arr(hand["wr"])
    r = oracle.route(x, wr, None, hand["K"], "sigmoid", "selected")
    exp = hand["expected"]
    assert r["sel"].tolist() == exp["sel_without_bias"]
    np.testing.assert_allclose(r["gate"][0], [_ev(v) for v in exp["gate_without_bias_token0"]], atol=1e-15)


def test_hand_worked_layer_output(hand):
    x, wr = _arr(hand["x"]), _arr(hand["wr"])
    bias = np.array([_ev(b) for b in hand["bias"]])
    r = oracle.route(x, wr, bias, hand["K"], "sigmoid", "selected")
    y, _, _ = oracle.layer_rows(x, r["sel"], r["gate"], _hand_bank(hand))
    np.testing.assert_allclose(y, _arr(hand["expected"]["y"]), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# Top-K selection (eqs. 14 and 16)
# --------------------------------------------------------------------------

def _brute_topk(keys_row, K):
    """All C(E, K) subsets: maximal exact key sum, lexicographically smallest
    index tuple among equal sums (= lower index wins ties)."""
    E = len(keys_row)
    best = None
    for sub in itertools.combinations(range(E), K):
        s = sum(Fraction(keys_row[i]) for i in sub)
        if best is None or s > best[0] or (s == best[0] and sub < best[1]):
            best = (s, sub)
    return set(best[1])


@pytest.mark.parametrize("E,K", [(16, 2), (8, 3), (6, 6), (7, 1)])
def test_topk_matches_brute_force(E, K):
    rng = np.random.default_rng(1234 + E * 10 + K)
    # dyadic keys from a small set: many exact ties, exact sums
    keys = rng.integers(-4, 5, size=(60, E)).astype(np.float64) / 8.0
    sel, gap = oracle.select_topk(keys, K)
    for t in range(keys.shape[0]):
        assert set(sel[t].tolist()) == _brute_topk(keys[t].tolist(), K)
        assert len(set(sel[t].tolist())) == K
        # key-descending order, lower index first among equal keys
        ks = keys[t, sel[t]]
        for a in range(K - 1):
            assert ks[a] > ks[a + 1] or (ks[a] == ks[a + 1] and sel[t, a] < sel[t, a + 1])
        if K < E:
            rest = np.setdiff1d(np.arange(E), sel[t])
            assert gap[t] == ks[-1] - keys[t, rest].max()
        else:
            assert gap[t] == np.inf


def test_topk_matches_lexsort_with_ties():
    rng = np.random.default_rng(7)
    T, E, K = 300, 64, 8
    keys = rng.random((T, E))
    keys[::3, 5] = keys[::3, 9]          # injected exact ties
    keys[::7, :] = 0.25                  # fully tied rows
    sel, _ = oracle.select_topk(keys, K)
    for t in range(T):
        order = np.lexsort((np.arange(E), -keys[t]))
        assert sel[t].tolist() == order[:K].tolist()


def test_topk_matches_torch_topk_distinct():
    rng = np.random.default_rng(8)
    keys = rng.standard_normal((500, 256))
    sel, _ = oracle.select_topk(keys, 8)
    tv, ti = torch.topk(torch.from_numpy(keys), 8, dim=1, largest=True, sorted=True)
    assert np.array_equal(sel, ti.numpy())


# --------------------------------------------------------------------------
# Scores and gates (eqs. 13, 15; 2024 softmax layout)
# --------------------------------------------------------------------------

def test_scores_match_scipy():
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((50, 64)) * 5.0
    np.testing.assert_allclose(oracle.scores(lg, "sigmoid"), scipy.special.expit(lg), rtol=1e-15, atol=0)
    np.testing.assert_allclose(oracle.scores(lg, "softmax"), scipy.special.softmax(lg, axis=1), rtol=1e-13, atol=0)


def test_router_logits_orientation():
    # x [T=2, d=3], wr [E=4, d=3]: logits[t, i] = <x_t, e_i>
    x = np.array([[1.0, 2.0, 3.0], [0.0, -1.0, 0.5]])
    wr = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 0.0], [0.0, 0.0, 1.0], [1.0, 1.0, 1.0]])
    np.testing.assert_array_equal(oracle.router_logits(x, wr), [[1, 2, 3, 6], [0, -1, 0.5, -0.5]])


def test_zero_router_sigmoid():
    T, d, E, K = 10, 16, 12, 4
    x = np.random.default_rng(0).standard_normal((T, d))
    r = oracle.route(x, np.zeros((E, d)), None, K, "sigmoid", "selected")
    assert np.all(r["scores"] == 0.5)
    assert r["sel"].tolist() == [list(range(K))] * T
    np.testing.assert_array_equal(r["gate"], np.full((T, K), 1.0 / K))


def test_zero_router_softmax_unnormalised():
    T, d, E, K = 10, 16, 64, 6
    x = np.random.default_rng(1).standard_normal((T, d))
    r = oracle.route(x, np.zeros((E, d)), None, K, "softmax", "none")
    np.testing.assert_allclose(r["gate"], np.full((T, K), 1.0 / E), rtol=1e-15)
    np.testing.assert_allclose(r["gate"].sum(1), K / E, rtol=1e-14)


def test_gates_sum_to_one_v3():
    rng = np.random.default_rng(4)
    x, wr = rng.standard_normal((200, 64)), rng.standard_normal((32, 64)) * 0.2
    r = oracle.route(x, wr, rng.uniform(-0.05, 0.05, 32), 8, "sigmoid", "selected")
    np.testing.assert_allclose(r["gate"].sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.all(r["gate"] > 0)


def test_gates_2024_unnormalised():
    rng = np.random.default_rng(5)
    x, wr = rng.standard_normal((200, 64)), rng.standard_normal((64, 64)) * 0.3
    r = oracle.route(x, wr, None, 6, "softmax", "none")
    tot = r["gate"].sum(1)
    assert np.all(tot < 1.0) and np.all(tot > 0.0)
    rest = r["scores"].sum(1) - tot
    np.testing.assert_allclose(tot, 1.0 - rest, atol=1e-14)
    # the gates are the selected softmax scores themselves
    np.testing.assert_array_equal(r["gate"], np.take_along_axis(r["scores"], r["sel"], 1))


def test_bias_changes_selection_not_gate_values():
    rng = np.random.default_rng(6)
    x, wr = rng.standard_normal((400, 32)), rng.standard_normal((32, 32)) * 0.3
    b = rng.uniform(-0.05, 0.05, 32)
    r0 = oracle.route(x, wr, None, 4, "sigmoid", "selected")
    r1 = oracle.route(x, wr, b, 4, "sigmoid", "selected")
    same = np.all(np.sort(r0["sel"], 1) == np.sort(r1["sel"], 1), axis=1)
    assert same.any() and (~same).any()
    for t in np.flatnonzero(same):
        g0 = dict(zip(r0["sel"][t].tolist(), r0["gate"][t].tolist()))
        g1 = dict(zip(r1["sel"][t].tolist(), r1["gate"][t].tolist()))
        # same gate per expert; only the order of the K-term sum may differ
        assert g0.keys() == g1.keys()
        for e in g0:
            assert g0[e] == pytest.approx(g1[e], rel=1e-15)


def test_forcing_bias_selects_set_and_keeps_gates():
    rng = np.random.default_rng(9)
    E, K = 16, 3
    x, wr = rng.standard_normal((50, 8)), rng.standard_normal((E, 8)) * 0.5
    forced = [2, 11, 7]
    b = np.zeros(E)
    b[forced] = 10.0
    r = oracle.route(x, wr, b, K, "sigmoid", "selected")
    assert all(set(s) == set(forced) for s in r["sel"].tolist())
    s = r["scores"][:, forced]
    want = s / s.sum(1, keepdims=True)
    got = np.stack([[dict(zip(r["sel"][t], r["gate"][t]))[e] for e in forced] for t in range(50)])
    np.testing.assert_allclose(got, want, rtol=1e-15)
    b2 = b * 2
    r2 = oracle.route(x, wr, b2, K, "sigmoid", "selected")
    np.testing.assert_array_equal(r2["gate"], r["gate"])


def test_k_equals_e_bias_independent():
    rng = np.random.default_rng(10)
    E, d = 6, 8
    x, wr = rng.standard_normal((20, d)), rng.standard_normal((E, d))
    bank, _ = _random_bank(rng, E, d, 4, S=1, Is=4)
    ra = oracle.route(x, wr, None, E, "sigmoid", "selected")
    rb = oracle.route(x, wr, rng.uniform(-1, 1, E), E, "sigmoid", "selected")
    ya, _, _ = oracle.layer_rows(x, ra["sel"], ra["gate"], bank)
    yb, _, _ = oracle.layer_rows(x, rb["sel"], rb["gate"], bank)
    np.testing.assert_allclose(ya, yb, rtol=1e-13, atol=1e-15)
    assert np.all(ra["gap"] == np.inf)


# --------------------------------------------------------------------------
# Loads and permutation (no token dropping)
# --------------------------------------------------------------------------

def test_loads_and_permutation_vs_library():
    rng = np.random.default_rng(11)
    T, E, K = 333, 40, 5
    keys = rng.random((T, E))
    sel, _ = oracle.select_topk(keys, K)
    load = oracle.expert_loads(sel, E)
    assert np.array_equal(load, np.bincount(sel.ravel(), minlength=E))
    assert load.sum() == T * K
    assert all(len(set(r)) == K for r in sel.tolist())
    off, perm = oracle.permutation(sel, E)
    assert np.array_equal(perm, np.argsort(sel.ravel(), kind="stable"))
    assert np.array_equal(off[1:], np.cumsum(np.bincount(sel.ravel(), minlength=E)))
    assert off[0] == 0 and np.array_equal(np.sort(perm), np.arange(T * K))


# --------------------------------------------------------------------------
# SwiGLU expert and combine
# --------------------------------------------------------------------------

def test_swiglu_scalar_closed_form():
    # d = I = 1: E(x) = w2 * SiLU(w1 x) * (w3 x); at w1 x = log 3, sigmoid = 3/4
    y = oracle.swiglu_expert(np.array([[math.log(3)]]), np.array([[1.0]]), np.array([[2.0]]), np.array([[3.0]]))
    assert y[0, 0] == pytest.approx(4.5 * math.log(3) ** 2, rel=1e-15)
    assert oracle.silu(np.array([0.0]))[0] == 0.0


def test_swiglu_gate_vs_up_and_orientation():
    # I = 3, d = 2: W1, W3 are [I, d], W2 is [d, I]
    v = np.array([[1.0, 2.0]])
    w1 = np.array([[40.0, 0.0], [-40.0, 0.0], [0.0, 0.0]])
    w3 = np.array([[0.0, 1.0], [0.0, 1.0], [5.0, 5.0]])
    w2 = np.array([[1.0, 0.0, 0.0], [0.0, 1.0, 7.0]])
    y = oracle.swiglu_expert(v, w1, w3, w2)
    # h = [SiLU(40)*2, SiLU(-40)*2, SiLU(0)*15] ~ [80, ~0, 0]
    assert y[0, 0] == pytest.approx(80.0, rel=1e-15)
    assert abs(y[0, 1]) < 1e-14


def test_swiglu_linearity_and_zero_gate():
    rng = np.random.default_rng(12)
    v = rng.standard_normal((5, 8))
    w1, w3, w2 = rng.standard_normal((6, 8)), rng.standard_normal((6, 8)), rng.standard_normal((8, 6))
    y = oracle.swiglu_expert(v, w1, w3, w2)
    np.testing.assert_allclose(oracle.swiglu_expert(v, w1, w3, 2 * w2), 2 * y, rtol=1e-15)
    np.testing.assert_allclose(oracle.swiglu_expert(v, w1, 3 * w3, w2), 3 * y, rtol=1e-13, atol=1e-13 * np.abs(y).max())
    assert np.all(oracle.swiglu_expert(v, np.zeros_like(w1), w3, w2) == 0)
    assert np.all(oracle.swiglu_expert(v, w1, np.zeros_like(w3), w2) == 0)


def _random_bank(rng, E, d, I, S=0, Is=0, identical=False):
    ws = [(rng.standard_normal((I, d)) * 0.3, rng.standard_normal((I, d)) * 0.3, rng.standard_normal((d, I)) * 0.3)
          for _ in range(1 if identical else E)]
    fetch = (lambda e: ws[0] + (None, None, None)) if identical else (lambda e: ws[e] + (None, None, None))
    shared = None
    if S:
        shared = (rng.standard_normal((S * Is, d)) * 0.3, rng.standard_normal((S * Is, d)) * 0.3,
                  rng.standard_normal((d, S * Is)) * 0.3, None, None, None)
    return oracle.ExpertBank(fetch=fetch, shared=shared, S=S), ws


@pytest.mark.parametrize("score,norm", [("sigmoid", "selected"), ("softmax", "none")])
def test_identical_experts(score, norm):
    rng = np.random.default_rng(13)
    E, d, I, K = 10, 12, 7, 3
    bank, ws = _random_bank(rng, E, d, I, identical=True)
    x, wr = rng.standard_normal((30, d)), rng.standard_normal((E, d))
    r = oracle.route(x, wr, None, K, score, norm)
    y, ysh, _ = oracle.layer_rows(x, r["sel"], r["gate"], bank)
    assert np.all(ysh == 0)
    one = oracle.swiglu_expert(x, *ws[0])
    np.testing.assert_allclose(y, r["gate"].sum(1, keepdims=True) * one, rtol=1e-12, atol=1e-14)
    if norm == "selected":
        np.testing.assert_allclose(y, one, rtol=1e-12, atol=1e-14)


def test_shared_concat_identity():
    rng = np.random.default_rng(14)
    d, Is = 8, 5
    w1s, w3s, w2s = rng.standard_normal((2 * Is, d)), rng.standard_normal((2 * Is, d)), rng.standard_normal((d, 2 * Is))
    x = rng.standard_normal((9, d))
    sel, gate = np.zeros((9, 1), dtype=np.int64), np.zeros((9, 1))
    zero = oracle.ExpertBank(fetch=lambda e: (np.zeros((1, d)), np.zeros((1, d)), np.zeros((d, 1)), None, None, None),
                             shared=(w1s, w3s, w2s, None, None, None), S=2)
    two, ysh2, _ = oracle.layer_rows(x, sel, gate, zero)
    zero.S = 1
    one, ysh1, _ = oracle.layer_rows(x, sel, gate, zero)
    np.testing.assert_allclose(two, one, rtol=1e-13, atol=1e-14)
    # and the two halves are really two experts summed
    a = oracle.swiglu_expert(x, w1s[:Is], w3s[:Is], w2s[:, :Is])
    b = oracle.swiglu_expert(x, w1s[Is:], w3s[Is:], w2s[:, Is:])
    np.testing.assert_allclose(ysh2, a + b, rtol=1e-13, atol=1e-14)


def test_routed_linearity_in_down_projection():
    rng = np.random.default_rng(15)
    E, d, I, K = 6, 8, 4, 2
    bank, ws = _random_bank(rng, E, d, I, S=1, Is=3)
    bank2 = oracle.ExpertBank(fetch=lambda e: (ws[e][0], ws[e][1], 2 * ws[e][2], None, None, None),
                              shared=bank.shared, S=1)
    x, wr = rng.standard_normal((20, d)), rng.standard_normal((E, d))
    r = oracle.route(x, wr, None, K, "sigmoid", "selected")
    y1, s1, _ = oracle.layer_rows(x, r["sel"], r["gate"], bank)
    y2, s2, _ = oracle.layer_rows(x, r["sel"], r["gate"], bank2)
    np.testing.assert_allclose(y2 - s2, 2 * (y1 - s1), rtol=1e-13, atol=1e-14)


# --------------------------------------------------------------------------
# Stored formats
# --------------------------------------------------------------------------

def test_e4m3_table_vs_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.E4M3_TABLE
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours))
    assert np.array_equal(ref[~nan], ours[~nan])


def test_e4m3_spot_values(golden_dir):
    with open(os.path.join(golden_dir, "e4m3_spot_values.json")) as f:
        g = json.load(f)
    for code, expr in g["values"].items():
        want = -0.0 if expr == "-0" else _ev(expr)
        got = oracle.E4M3_TABLE[int(code)]
        assert got == want and math.copysign(1, got) == math.copysign(1, want), (code, got, want)
    for c in g["nan_codes"]:
        assert math.isnan(oracle.E4M3_TABLE[c])
    assert np.nanmax(np.abs(oracle.E4M3_TABLE)) == 448.0


def test_bf16_decode_vs_torch():
    bits = torch.arange(0, 65536, 37, dtype=torch.int32).to(torch.int16)
    ref = bits.view(torch.bfloat16).to(torch.float64).numpy()
    ours = oracle.bf16_to_f64(bits.numpy().view(np.uint16))
    fin = np.isfinite(ref)
    assert np.array_equal(ref[fin], ours[fin])


def test_fp8_row_scale_applied_per_output_row():
    codes = np.array([[56, 64], [56, 64]], dtype=np.uint8)        # [[1, 2], [1, 2]]
    got = oracle.decode_stored(codes, np.array([0.5, 3.0], dtype=np.float32))
    np.testing.assert_array_equal(got, [[0.5, 1.0], [3.0, 6.0]])


# --------------------------------------------------------------------------
# Bias update (section 2.2)
# --------------------------------------------------------------------------

def test_bias_update_signs():
    # E = 4, loads sum to 8, mean 2: over, at, under, under -> -g, 0, +g, +g
    b = np.zeros(4, dtype=np.float32)
    nb = oracle.bias_update(b, np.array([5, 2, 1, 0]))
    g = np.float32(1e-3)
    assert nb.dtype == np.float32
    assert nb.tolist() == [-g, 0.0, g, g]
    # mean is not an integer: 7/4 -> 2 is over, 1 is under
    nb = oracle.bias_update(b, np.array([2, 1, 4, 0]))
    assert nb.tolist() == [-g, g, -g, g]


def test_bias_update_trajectory_closed_form():
    # an expert overloaded in each of n batches ends near -n*gamma, with only
    # fp32 rounding of each exact step in between
    b = np.zeros(3, dtype=np.float32)
    n = 20
    for _ in range(n):
        b = oracle.bias_update(b, np.array([10, 1, 1]))
    g = float(np.float32(1e-3))
    assert abs(float(b[0]) + n * g) < n * 2e-10
    assert abs(float(b[1]) - n * g) < n * 2e-10
    assert b[1] == b[2] == -b[0]


def test_near_tie_flag_threshold():
    keys = np.array([[1.0, 0.5, 0.5 - 2e-5, 0.0], [1.0, 0.5, 0.5 - 5e-6, 0.0]])
    sel, gap = oracle.select_topk(keys, 2)
    assert (gap < oracle.NEAR_TIE_GAP).tolist() == [False, True]


def _route_keys(keys, K, groups=None):
    """A route() result whose scores are the given keys (no bias): logits =
    logit(keys), identity router."""
    keys = np.asarray(keys, dtype=np.float64)
    return oracle.route(np.log(keys / (1.0 - keys)), np.eye(keys.shape[1]), None, K, "sigmoid",
                        "selected", groups=groups)


def test_selection_valid_accepts_only_the_open_sets_of_a_near_tie():
    # token 0: a clear top-2 {0, 1}; token 1: 2nd and 3rd keys 5e-6 apart
    # (a near-tie: {0, 1} and {0, 2} are both correct, {0, 3} is not)
    r = _route_keys([[0.9, 0.7, 0.5, 0.3], [0.9, 0.7, 0.7 - 5e-6, 0.3]], 2)
    assert r["near_tie"].tolist() == [False, True]
    v = lambda idx: oracle.selection_valid(r, np.array(idx), 2).tolist()
    assert v([[0, 1], [0, 1]]) == [True, True]
    assert v([[1, 0], [2, 0]]) == [True, True]          # order is free; the tie's other set
    assert v([[0, 2], [0, 3]]) == [False, False]        # not near: must equal; 0.3 is not within 1e-5
    assert v([[0, 0], [0, 0]]) == [False, False]        # an expert twice
    assert v([[0, 4], [0, -1]]) == [False, False]       # out of range


def test_selection_valid_node_limited_near_tie():
    # groups of 2 with sums 1.0, 1.0 - 2e-6, 0.3 and M = 1: the kept group is
    # group 0 in the oracle, group 1 within the tolerance
    r = _route_keys([[0.5, 0.5, 0.25, 0.75 - 2e-6, 0.1, 0.2]], 2, groups=(3, 1))
    assert r["near_tie"][0]
    v = lambda idx: bool(oracle.selection_valid(r, np.array([idx]), 2, groups=(3, 1))[0])
    assert v([0, 1]) and v([2, 3])
    assert not v([1, 3])                                # two groups used with M = 1
    assert not v([4, 5])                                # group 2 is 0.7 below the kept one


# ---- node-limited (group-limited) routing ("DeepSeekMoE架构解析" section 2.3) ----

def _rand_route_inputs(rng, T, E, d=16):
    return rng.standard_normal((T, d)), rng.standard_normal((E, d)) * 0.5


def test_groups_all_kept_is_plain_topk():
    rng = np.random.default_rng(11)
    x, wr = _rand_route_inputs(rng, 50, 32)
    b = rng.uniform(-0.05, 0.05, 32)
    a = oracle.route(x, wr, b, 6, "sigmoid", "selected")
    for groups in ((8, 8), (1, 1)):
        g = oracle.route(x, wr, b, 6, "sigmoid", "selected", groups=groups)
        assert np.array_equal(a["sel"], g["sel"]) and np.array_equal(a["gate"], g["gate"])


def test_groups_containing_global_topk_change_nothing():
    """When the kept groups hold the plain top-K, the group limit is moot."""
    rng = np.random.default_rng(12)
    x, wr = _rand_route_inputs(rng, 400, 64)
    b = rng.uniform(-0.05, 0.05, 64)
    plain = oracle.route(x, wr, b, 8, "sigmoid", "selected")
    grp = oracle.route(x, wr, b, 8, "sigmoid", "selected", groups=(8, 4))
    inside = np.all(np.take_along_axis(grp["allowed"], plain["sel"], axis=1), axis=1)
    assert 0 < inside.sum() < len(inside)          # both kinds of token occur
    assert np.array_equal(plain["sel"][inside], grp["sel"][inside])
    assert not np.array_equal(plain["sel"][~inside], grp["sel"][~inside])
    # every selected expert lies in a kept group, at most M groups are used
    assert np.all(np.take_along_axis(grp["allowed"], grp["sel"], axis=1))
    assert max(len(set((grp["sel"][t] // 8).tolist())) for t in range(400)) <= 4


def test_groups_against_pairwise_count_definition():
    """Brute force with ties: a group is kept iff fewer than M groups beat it
    (larger sum, or equal sum and lower index); an expert is chosen iff it is
    allowed and fewer than K allowed experts beat it the same way."""
    rng = np.random.default_rng(13)
    E, G, M, K = 12, 4, 2, 3
    n = E // G
    for _ in range(300):
        s = rng.integers(0, 4, size=(1, E)) / 8.0          # coarse values: many ties
        keys = s + rng.integers(0, 3, size=(1, E)) / 16.0
        allowed, gs, _ = oracle.select_groups(s, G, M)
        kept = [g for g in range(G)
                if sum(gs[0, h] > gs[0, g] or (gs[0, h] == gs[0, g] and h < g) for h in range(G)) < M]
        want_allowed = np.array([e // n in kept for e in range(E)])
        assert np.array_equal(allowed[0], want_allowed)
        cand = np.where(allowed, keys, -np.inf)
        sel, _ = oracle.select_topk(cand, K)
        chosen = [e for e in range(E) if want_allowed[e] and sum(
            want_allowed[f] and (keys[0, f] > keys[0, e] or (keys[0, f] == keys[0, e] and f < e))
            for f in range(E)) < K]
        assert sorted(sel[0].tolist()) == chosen


def test_groups_hand_example_sum_not_max_and_bias_outside():
    """E = 8 in G = 4 groups of 2, M = 2, K = 2. Group sums 1.0, 0.95, 0.96,
    0.5: groups 0 and 2 are kept (by the sum; the maxima 0.9, 0.5, 0.48, 0.3
    would keep 0 and 1). Plain top-2 is {0, 2}; group-limited top-2 is {0, 4}
    (experts 4 and 5 tie at 0.48: the lower index wins). A bias on expert 2
    (group 1, not kept) cannot bring it back: the bias is not part of the
    group affinity."""
    s = np.array([[0.9, 0.1, 0.5, 0.45, 0.48, 0.48, 0.2, 0.3]])
    allowed, gs, ggap = oracle.select_groups(s, 4, 2)
    assert np.allclose(gs[0], [1.0, 0.95, 0.96, 0.5])
    assert allowed[0].tolist() == [True, True, False, False, True, True, False, False]
    assert abs(ggap[0] - 0.01) < 1e-12
    x1 = np.log(s / (1.0 - s))               # one token whose logits (x1 @ I) give s
    r = oracle.route(x1, np.eye(8), None, 2, "sigmoid", "selected", groups=(4, 2))
    assert sorted(r["sel"][0].tolist()) == [0, 4]
    assert np.allclose(r["gate"][0], np.array([0.9, 0.48]) / 1.38)
    plain = oracle.route(x1, np.eye(8), None, 2, "sigmoid", "selected")
    assert sorted(plain["sel"][0].tolist()) == [0, 2]
    bias = np.zeros(8)
    bias[2] = 5.0
    rb = oracle.route(x1, np.eye(8), bias, 2, "sigmoid", "selected", groups=(4, 2))
    assert sorted(rb["sel"][0].tolist()) == [0, 4]
    assert sorted(oracle.route(x1, np.eye(8), bias, 2, "sigmoid", "selected")["sel"][0].tolist()) == [0, 2]


def test_groups_near_tie_flag_and_capacity_check():
    s_eq = np.array([[0.5, 0.5, 0.25, 0.75, 0.1, 0.2]])      # groups of 2: sums 1.0, 1.0, 0.3
    _, _, ggap = oracle.select_groups(s_eq, 3, 1)
    assert ggap[0] == 0.0
    logits = np.log(s_eq / (1.0 - s_eq))
    r = oracle.route(logits, np.eye(6), None, 2, "sigmoid", "selected", groups=(3, 1))
    assert r["near_tie"][0]
    assert sorted(r["sel"][0].tolist()) == [0, 1]     # group 0 wins the tie (lower index)
    with pytest.raises(ValueError):
        oracle.route(logits, np.eye(6), None, 3, "sigmoid", "selected", groups=(3, 1))


# ---- "1 + sum" gate weighting and per-sequence loads ----

def test_one_plus_gates_closed_form():
    """Scores 1/2, 1/4, 1/4 selected: gates s / (1 + 1) = 1/4, 1/8, 1/8."""
    s = np.array([[0.5, 0.25, 0.25, 0.1]])
    sel = np.array([[0, 1, 2]])
    g = oracle.gate_values(s, sel, "one_plus")
    assert np.array_equal(g, np.array([[0.25, 0.125, 0.125]]))
    assert np.array_equal(oracle.gate_values(s, sel, "selected"), np.array([[0.5, 0.25, 0.25]]))


def test_one_plus_gates_relations():
    """g_one_plus = g_selected * S / (1 + S) with S the selected-score sum, so
    the gates sum to S / (1 + S) < 1; routing is unaffected by the weighting."""
    rng = np.random.default_rng(21)
    x, wr = rng.standard_normal((40, 16)), rng.standard_normal((32, 16))
    a = oracle.route(x, wr, None, 6, "sigmoid", "selected")
    b = oracle.route(x, wr, None, 6, "sigmoid", "one_plus")
    assert np.array_equal(a["sel"], b["sel"])
    S = np.take_along_axis(a["scores"], a["sel"], axis=1).sum(axis=1)
    assert np.allclose(b["gate"], a["gate"] * (S / (1 + S))[:, None], rtol=1e-14, atol=0)
    assert np.allclose(b["gate"].sum(axis=1), S / (1 + S), rtol=1e-14, atol=0)
    assert np.all(b["gate"].sum(axis=1) < 1)


def test_sequence_loads_against_bincount():
    rng = np.random.default_rng(22)
    sel = np.stack([rng.choice(20, 3, replace=False) for _ in range(53)])
    q = oracle.sequence_loads(sel, 20, 10)
    assert q.shape == (6, 20)
    for i in range(6):
        assert np.array_equal(q[i], np.bincount(sel[i * 10:(i + 1) * 10].ravel(), minlength=20))
    assert np.array_equal(q.sum(axis=0), oracle.expert_loads(sel, 20))
    assert q[5].sum() == 3 * 3                       # the short last sequence


# ---- pre-MoE RMSNorm ("DeepSeekMoE架构解析" section 4.1) and fp64 -> bf16 rounding ----

def test_rmsnorm_closed_forms():
    w = np.array([1.0, 2.0, 0.5, -1.0])
    u = oracle.rmsnorm(np.full((1, 4), 3.0), w)
    assert np.allclose(u, 3.0 / np.sqrt(9.0 + 1e-6) * w, rtol=1e-15, atol=0)
    u0 = oracle.rmsnorm(np.zeros((1, 4)), w)                    # eps keeps it finite
    assert np.all(u0 == 0.0)
    us = oracle.rmsnorm(np.full((1, 4), 1e-4), np.ones(4))       # eps dominates
    assert np.allclose(us, 1e-4 / np.sqrt(1e-8 + 1e-6), rtol=1e-15, atol=0)
    assert oracle.RMS_EPS == 1e-6


def test_rmsnorm_against_torch():
    rng = np.random.default_rng(31)
    x = rng.standard_normal((20, 96))
    w = rng.uniform(0.5, 1.5, 96)
    want = torch.nn.functional.rms_norm(torch.tensor(x), (96,), torch.tensor(w), eps=1e-6).numpy()
    assert np.allclose(oracle.rmsnorm(x, w), want, rtol=1e-14, atol=0)


def test_rmsnorm_sum_of_bf16_squares_is_exact():
    """The premise of computing the mean square in float64: for bf16 inputs of
    this magnitude the sum of squares has no rounding, whatever the order."""
    import math
    rng = np.random.default_rng(32)
    x = oracle.bf16_to_f64((rng.standard_normal((8, 7168)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    for row in x:
        sq = row * row
        assert float(np.sum(sq)) == math.fsum(sq.tolist()) == float(np.sum(sq[::-1]))


def test_f64_to_bf16_rounding():
    rng = np.random.default_rng(33)
    # fp32-representable inputs: the same as torch's fp32 -> bf16 conversion (round to nearest even)
    v32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    want = torch.tensor(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.f64_to_bf16_bits(v32.astype(np.float64)), want)
    # arbitrary doubles: the result is the nearer of the two neighbouring bf16 values
    v = rng.standard_normal(20000) * np.exp(rng.uniform(-5, 5, 20000))
    b = oracle.f64_to_bf16_bits(v)
    r = oracle.bf16_to_f64(b)
    lo = oracle.bf16_to_f64((b.astype(np.int32) - np.sign(r - v).astype(np.int32) * np.where(v < 0, -1, 1)).astype(np.uint16))
    assert np.all(np.abs(r - v) <= np.abs(lo - v))
    # exact midpoints go to the even neighbour (no double rounding through fp32)
    one = 1.0
    assert oracle.f64_to_bf16_bits(np.array([one + 2.0 ** -8]))[0] == 0x3F80        # tie -> even (1.0)
    assert oracle.f64_to_bf16_bits(np.array([one + 3 * 2.0 ** -8]))[0] == 0x3F82    # tie -> even (1 + 2^-6)
    assert oracle.f64_to_bf16_bits(np.array([one + 2.0 ** -8 + 2.0 ** -40]))[0] == 0x3F81
    assert oracle.f64_to_bf16_bits(np.array([-(one + 2.0 ** -8)]))[0] == 0xBF80


# ---- fine-grained FP8 ("DeepSeekMoE架构解析" section 4.3): 1x128 tiles, 128x128 blocks ----

def _e4m3_midpoints():
    pos = oracle.E4M3_TABLE[:0x7F]
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mid.astype(np.float64), (pos[:-1] + pos[1:]) / 2)   # exact in fp32
    return np.concatenate([mid, -mid])


def test_e4m3_encode_against_torch():
    """The nearest-value encoder against torch's own fp32 -> float8_e4m3fn
    cast (round to nearest even), on random values of every binade, on the
    subnormals and on every exact midpoint between neighbouring codes."""
    rng = np.random.default_rng(41)
    v = (rng.standard_normal(50000) * np.exp(rng.uniform(-14, 6, 50000))).astype(np.float32)
    v = np.clip(v, -448, 448)
    for arr in (v, _e4m3_midpoints(), np.float32([0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -9 * 1.5, 448.0, -448.0])):
        want = torch.tensor(arr).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        assert np.array_equal(oracle.e4m3_encode(arr), want)
    # decoding what was encoded gives the nearest representable value
    d = oracle.E4M3_TABLE[oracle.e4m3_encode(v)]
    pos = oracle.E4M3_TABLE[:0x7F]
    near = np.min(np.abs(np.abs(v.astype(np.float64))[:, None] - pos[None, :]), axis=1)
    assert np.array_equal(np.abs(d - v), near)


def test_quantize_tiles_closed_forms():
    rng = np.random.default_rng(42)
    x = rng.standard_normal((3, 512)).astype(np.float32)
    x[1, 128:256] = 0.0                                      # an all-zero tile
    codes, s = oracle.quantize_tiles(x)
    assert codes.shape == (3, 512) and s.shape == (3, 4) and s.dtype == np.float32
    t = np.abs(x.reshape(3, 4, 128))
    amax = t.max(axis=2)
    assert s[1, 1] == 1.0 and np.all(codes[1, 128:256] & 0x7F == 0)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    # the largest element of each tile maps to +-448 (code magnitude 0x7E)
    arg = t.argmax(axis=2)
    for r in range(3):
        for j in range(4):
            if nz[r, j]:
                assert codes[r, 128 * j + arg[r, j]] & 0x7F == 0x7E
    # orientation: tile j of row r has amax 448 * 2^(j - r) -> scale 2^(j - r) exactly
    y = np.ones((3, 512), np.float32)
    for r in range(3):
        for j in range(4):
            y[r, 128 * j] = np.float32(448.0 * 2.0 ** (j - r))
    cy, sy = oracle.quantize_tiles(y)
    assert np.array_equal(sy, np.float32([[2.0 ** (j - r) for j in range(4)] for r in range(3)]))
    # powers of two commute with the quantisation: same codes, scales times 2^p
    c8, s8 = oracle.quantize_tiles((x * np.float32(8.0)).astype(np.float32))
    assert np.array_equal(c8, codes)
    assert np.array_equal(s8, np.where(nz, s * np.float32(8.0), np.float32(1.0)))
    # values already on the grid (code value times a power-of-two scale) round-trip exactly
    g = oracle.E4M3_TABLE[rng.integers(0, 0x7F, (2, 256))] * (2.0 ** -5)
    g[:, 0] = 448.0 * 2.0 ** -5
    g[:, 128] = 448.0 * 2.0 ** -5
    cg, sg = oracle.quantize_tiles(g.astype(np.float32))
    assert np.array_equal(oracle.dequantize_tiles(cg, sg), g)


def test_quantize_tiles_error_bound():
    """|x - dequantised| <= 2^-4 |x| where x/s is in the normal E4M3 range (3
    mantissa bits: half a step), and <= s * 2^-10 below it (subnormal step
    2^-9 times the scale)."""
    rng = np.random.default_rng(43)
    x = (rng.standard_normal((16, 1024)) * np.exp(rng.uniform(-8, 3, (16, 1024)))).astype(np.float32)
    codes, s = oracle.quantize_tiles(x)
    err = np.abs(oracle.dequantize_tiles(codes, s) - x.astype(np.float64))
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    q = np.abs(x.astype(np.float64)) / sf
    normal = q >= 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(x[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= sf[~normal] * 2.0 ** -10 * (1 + 1e-6))


def test_dequantize_blocks_layout():
    """Block (i, j) of the scale matrix scales rows 128i.. and columns 128j..:
    brute force over every element, with a different scale per block."""
    rng = np.random.default_rng(44)
    codes = rng.integers(0, 0x7F, (256, 384)).astype(np.uint8)
    codes |= (rng.integers(0, 2, codes.shape) << 7).astype(np.uint8)
    sc = np.float32([[1 + i * 10 + j for j in range(3)] for i in range(2)])
    deq = oracle.dequantize_blocks(codes, sc)
    for r in range(0, 256, 37):
        for c in range(0, 384, 29):
            assert deq[r, c] == oracle.E4M3_TABLE[codes[r, c]] * float(sc[r // 128, c // 128])
    with pytest.raises(ValueError):
        oracle.dequantize_blocks(codes, sc.T)


def _fp8_weights(rng, rows, cols):
    codes = oracle.e4m3_encode(np.clip(rng.standard_normal((rows, cols)) * 100, -448, 448).astype(np.float32))
    sc = rng.uniform(1e-4, 3e-4, (rows // 128, cols // 128)).astype(np.float32)
    return codes, sc


def test_fp8_expert_within_the_h_quantisation_bound():
    """The fp8 expert against the plain SwiGLU expert on the dequantised x and
    weights: they differ only by the quantisation of h, so
    |difference| <= |W2| (2^-4 |h32| + 2^-10 s_h + |h - h32|) elementwise.
    A wrong tile or block scale, or a transposed operand, is far outside it."""
    rng = np.random.default_rng(45)
    n, d, I = 5, 256, 384
    x = rng.standard_normal((n, d)).astype(np.float32)
    xq, xs = oracle.quantize_tiles(x)
    (c1, s1), (c3, s3), (c2, s2) = _fp8_weights(rng, I, d), _fp8_weights(rng, I, d), _fp8_weights(rng, d, I)
    w1, w3, w2 = oracle.dequantize_blocks(c1, s1), oracle.dequantize_blocks(c3, s3), oracle.dequantize_blocks(c2, s2)
    out, hq, hs = oracle.swiglu_expert_fp8(xq, xs, w1, w3, w2)
    xd = oracle.dequantize_tiles(xq, xs)
    h = om.silu(xd @ w1.T) * (xd @ w3.T)
    plain = h @ w2.T
    assert np.allclose(plain, oracle.swiglu_expert(xd, w1, w3, w2), rtol=1e-12, atol=0)
    h32 = h.astype(np.float32).astype(np.float64)
    dh = 2.0 ** -4 * np.abs(h32) + 2.0 ** -10 * np.repeat(hs.astype(np.float64), 128, axis=1) + np.abs(h - h32)
    bound = dh @ np.abs(w2).T
    assert np.all(np.abs(out - plain) <= bound * (1 + 1e-9))
    assert np.max(np.abs(out - plain)) > 0                     # h really was quantised


def _e4m3_codes_torch(v):
    return torch.tensor(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_fp8_expert_exact_case():
    """A case where every quantisation is exact, so the fp8 expert must give
    the exact SwiGLU result of the real values it was built from: x tiles
    with amax 448 * 2^p (power-of-two scales), weights that are code values
    times power-of-two block scales (encoded by torch's own cast), gate
    pre-activations g = 56 or 112 (SiLU(g) == g in float64, and 1.75 * 2^m
    keeps h on the E4M3 grid of its tile), and up values +-2^k. The expected
    output is summed in exact rationals from the real values. A wrong tile,
    block or row/column orientation of any scale changes the result."""
    rng = np.random.default_rng(47)
    n, d, I = 2, 256, 256
    x = np.zeros((n, d))
    for t in range(n):
        x[t, 0], x[t, 1] = 448 * 2.0 ** -3, 2.0 ** -3 * (t + 1)
        x[t, 128], x[t, 129] = 448 * 2.0 ** -1, 2.0 ** -1
    W1 = np.zeros((I, d))
    W1[:128, 0], W1[:128, 128] = 2.0 ** -1, 2.0 ** -3      # g = 28 + 28 = 56
    W1[128:, 0], W1[128:, 128] = 1.0, 2.0 ** -2            # g = 56 + 56 = 112
    s1 = np.float32([[2.0 ** -4, 2.0 ** -5], [2.0 ** -6, 2.0 ** -7]])
    v = (2.0 ** rng.integers(-3, 2, I)) * rng.choice([-1.0, 1.0], I)
    W3 = np.zeros((I, d))
    W3[:, 1] = v * 2.0 ** 3                                  # u = (t + 1) v
    s3 = np.float32([[2.0 ** -2, 1.0], [2.0 ** -3, 1.0]])
    W2 = np.where(rng.random((d, I)) < 0.3, (2.0 ** rng.integers(-6, -2, (d, I))) * rng.choice([-1.0, 1.0], (d, I)), 0.0)
    s2 = np.float32([[2.0 ** -9, 2.0 ** -8], [2.0 ** -10, 2.0 ** -7]])

    def codes(w, sc):
        return _e4m3_codes_torch(w / np.repeat(np.repeat(sc.astype(np.float64), 128, 0), 128, 1))

    c1, c3, c2 = codes(W1, s1), codes(W3, s3), codes(W2, s2)
    for c, w, sc in ((c1, W1, s1), (c3, W3, s3), (c2, W2, s2)):
        assert np.array_equal(oracle.dequantize_blocks(c, sc), w)        # exact construction
    xq, xs = oracle.quantize_tiles(x.astype(np.float32))
    assert np.array_equal(xs, np.float32([[2.0 ** -3, 2.0 ** -1]] * n))
    out, hq, hs = oracle.swiglu_expert_fp8(xq, xs, oracle.dequantize_blocks(c1, s1),
                                           oracle.dequantize_blocks(c3, s3), oracle.dequantize_blocks(c2, s2))
    g = np.where(np.arange(I) < 128, 56, 112)
    for t in range(n):
        h = [Fraction(int(g[i])) * (t + 1) * Fraction(v[i]) for i in range(I)]
        for j in range(0, d, 7):
            want = sum(Fraction(W2[j, i]) * h[i] for i in range(I) if W2[j, i] != 0)
            assert Fraction(out[t, j]) == want


def test_fp8_layer_identical_experts_and_shared_concat():
    """With every routed expert identical the routed sum is (sum of gates) x
    one expert; two shared experts passed concatenated equal the sum of the
    two computed apart (the 1 x 128 tiles of h never straddle them)."""
    rng = np.random.default_rng(46)
    n, d, I, E, K = 6, 128, 256, 4, 2
    xb = (rng.standard_normal((n, d)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    c1, s1 = _fp8_weights(rng, I, d)
    c3, s3 = _fp8_weights(rng, I, d)
    c2, s2 = _fp8_weights(rng, d, I)
    sel = np.array([[0, 1], [2, 3], [1, 2], [3, 0], [0, 2], [1, 3]])
    gate = rng.uniform(0.1, 0.9, (n, K))
    bank = oracle.BlockExpertBank(fetch=lambda e: (c1, c3, c2, s1, s3, s2))
    y, y_sh, routed = oracle.layer_rows_fp8(xb, sel, gate, bank)
    xq, xs = oracle.quantize_x(xb)
    one = oracle.swiglu_expert_fp8(xq, xs, *bank.expert(0))[0]
    assert np.allclose(y, gate.sum(axis=1)[:, None] * one, rtol=1e-12, atol=1e-15)
    assert np.all(y_sh == 0)
    # shared: two experts of width I concatenated
    d1, e1 = _fp8_weights(rng, 2 * I, d)
    d3, e3 = _fp8_weights(rng, 2 * I, d)
    d2, e2 = _fp8_weights(rng, d, 2 * I)
    sh = oracle.BlockExpertBank(fetch=lambda e: (c1, c3, c2, s1, s3, s2),
                                shared=(d1, d3, d2, e1, e3, e2), S=2)
    _, ysh2, _ = oracle.layer_rows_fp8(xb, sel, gate, sh)
    W1, W3, W2 = (oracle.dequantize_blocks(d1, e1), oracle.dequantize_blocks(d3, e3),
                  oracle.dequantize_blocks(d2, e2))
    apart = sum(oracle.swiglu_expert_fp8(xq, xs, W1[m * I:(m + 1) * I], W3[m * I:(m + 1) * I],
                                         W2[:, m * I:(m + 1) * I])[0] for m in range(2))
    assert np.allclose(ysh2, apart, rtol=1e-12, atol=1e-15)
