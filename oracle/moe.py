"""The DeepSeekMoE layer forward pass, written out in float64.

Notation follows "DeepSeekMoE架构解析" section 2.1: u_t is the hidden vector of
token t, e_i the centroid (router row) of routed expert i, s_{i,t} the
affinity score, K_r the number of routed experts each token uses, b_i the
balance bias of section 2.2.

Readings of points the pages leave open (each also listed in the design notes):
  * SwiGLU expert (named, never written out): E(v) = W2 (SiLU(W1 v) * (W3 v)),
    SiLU(z) = z * sigmoid(z), no bias terms. W1 = gate, W3 = up, W2 = down.
  * Gate normalisation: eq. (13) (divide by the sum over the selected experts),
    not the softmax of the section 3.1 sketch nor the "1 + sum" of the aiqz.cc
    page; the 2024 variant keeps the selected softmax scores unnormalised
    (course notes, section 四).
  * 2024 softmax runs over all E routed logits; top-K is taken on the scores.
  * The bias is added to the score (eq. 16), after the sigmoid, and enters
    only the selection; the gate uses the unbiased score.
  * Top-K order and ties: key descending, and among equal keys the lower
    expert index wins.
  * No residual: the layer output is shared(x) + sum_k g_k E_k(x).
  * Expert load = number of (token, slot) pairs routed to the expert, so the
    loads sum to T*K (no token is dropped: section 1 and course notes 六).
  * Bias update (section 2.2): an expert whose load exceeds the batch mean
    loses gamma, one below it gains gamma, one exactly at the mean is left
    unchanged; the mean is sum(load)/E, compared exactly in integers.
"""

from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction
from typing import Callable, Optional, Sequence

import numpy as np

from .formats import decode_stored

#: gamma = 1e-3 ("DeepSeekMoE架构解析" section 2.2), held as an fp32 constant
#: because the bias it updates is an fp32 vector.
GAMMA_F32 = np.float32(1e-3)

#: Tokens whose K-th and (K+1)-th biased keys differ by less than this are
#: near-ties: their selected set is not decided beyond rounding.
NEAR_TIE_GAP = 1e-5


#: RMSNorm epsilon of the MoE layer's norms ("DeepSeekMoE架构解析" section 4.1).
RMS_EPS = 1e-6


def rmsnorm(x: np.ndarray, w: np.ndarray, eps: float = RMS_EPS) -> np.ndarray:
    """Pre-MoE RMSNorm ("DeepSeekMoE架构解析" section 4.1 places an RMSNorm
    before and after the MoE layer, eps 1e-6): u = x / sqrt(mean(x^2) + eps) * w
    per token, w the per-channel weight. In float64: for bf16 inputs every
    square is exact and, at the magnitudes used here, so is their sum in any
    order; the mean, the sum with eps, the square root, the division and the
    product are each one correctly rounded operation, in this order."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.sum(x * x, axis=-1, keepdims=True) / x.shape[-1]
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def router_logits(x: np.ndarray, wr: np.ndarray) -> np.ndarray:
    """Affinities u_t^T e_i for every token t and routed expert i (eq. 15's
    argument). x: [T, d], wr: [E, d] (one centroid per row) -> [T, E]."""
    x = np.asarray(x, dtype=np.float64)
    wr = np.asarray(wr, dtype=np.float64)
    return x @ wr.T


def scores(logits: np.ndarray, fn: str) -> np.ndarray:
    """s_{i,t}. "sigmoid": eq. (15), applied to each expert independently.
    "softmax": the 2024 layout, normalised over all E routed experts."""
    logits = np.asarray(logits, dtype=np.float64)
    if fn == "sigmoid":
        with np.errstate(over="ignore"):
            return 1.0 / (1.0 + np.exp(-logits))
    if fn == "softmax":
        m = logits.max(axis=-1, keepdims=True)
        ex = np.exp(logits - m)
        return ex / ex.sum(axis=-1, keepdims=True)
    raise ValueError(fn)


def select_topk(keys: np.ndarray, K: int):
    """Top-K selection of eqs. (14)/(16): the K experts with the largest key,
    in key-descending order, lower index first among equal keys.

    Returns (sel [T, K] int64, gap [T] float64) where gap is the K-th key minus
    the (K+1)-th key (+inf when K == E)."""
    keys = np.asarray(keys, dtype=np.float64)
    T, E = keys.shape
    if not (1 <= K <= E):
        raise ValueError("need 1 <= K <= E")
    # A stable sort of the negated keys keeps equal keys in index order.
    order = np.argsort(-keys, axis=1, kind="stable")
    sel = order[:, :K]
    if K < E:
        kth = np.take_along_axis(keys, order[:, K - 1:K], axis=1)[:, 0]
        nxt = np.take_along_axis(keys, order[:, K:K + 1], axis=1)[:, 0]
        gap = kth - nxt
    else:
        gap = np.full(T, np.inf)
    return sel.astype(np.int64), gap


def select_groups(s: np.ndarray, G: int, M: int):
    """Node-limited routing ("DeepSeekMoE架构解析" section 2.3): the E routed
    experts form G groups of E/G consecutive experts (group g holds experts
    g*E/G .. (g+1)*E/G - 1, the experts one node hosts); a group's affinity is
    the sum of its experts' affinity scores s; each token keeps the M groups
    of largest affinity (lower group index first among equal sums) and its
    top-K is then taken only among the experts of those groups.

    Returns (allowed [T, E] bool, group_scores [T, G], group_gap [T]) where
    group_gap is the M-th largest group affinity minus the (M+1)-th (+inf
    when M == G)."""
    s = np.asarray(s, dtype=np.float64)
    T, E = s.shape
    if G < 1 or E % G != 0 or not (1 <= M <= G):
        raise ValueError("need E % G == 0 and 1 <= M <= G")
    n = E // G
    gs = s.reshape(T, G, n).sum(axis=2)
    order = np.argsort(-gs, axis=1, kind="stable")
    keep = np.zeros((T, G), dtype=bool)
    np.put_along_axis(keep, order[:, :M], True, axis=1)
    if M < G:
        mth = np.take_along_axis(gs, order[:, M - 1:M], axis=1)[:, 0]
        nxt = np.take_along_axis(gs, order[:, M:M + 1], axis=1)[:, 0]
        ggap = mth - nxt
    else:
        ggap = np.full(T, np.inf)
    return np.repeat(keep, n, axis=1), gs, ggap


def gate_values(s: np.ndarray, sel: np.ndarray, norm: str) -> np.ndarray:
    """g_{i,t} for the selected experts. "selected": eq. (13), each selected
    score divided by the sum of the selected scores (so the K gates sum to 1).
    "none": the 2024 layout, the selected scores themselves. "one_plus": the
    weighting of "DeepSeek-V3：MoE大模型架构" (section 路由机制 and its Python
    demo), each selected score divided by 1 + the sum of the selected scores,
    the 1 standing for the always-on shared expert (so the gates sum to
    sum/(1 + sum) < 1)."""
    s_sel = np.take_along_axis(np.asarray(s, dtype=np.float64), sel, axis=1)
    if norm == "selected":
        return s_sel / s_sel.sum(axis=1, keepdims=True)
    if norm == "none":
        return s_sel
    if norm == "one_plus":
        return s_sel / (1.0 + s_sel.sum(axis=1, keepdims=True))
    raise ValueError(norm)


def sequence_loads(sel: np.ndarray, E: int, seq_len: int) -> np.ndarray:
    """Per-sequence expert loads: the batch's tokens taken as consecutive
    sequences of seq_len tokens (the last one may be shorter); entry [q, e]
    counts the (token, slot) pairs of sequence q routed to expert e (the
    per-sequence counterpart of the batch load, for sequence-wise balance
    statistics: course notes "省钱第一招", section 五)."""
    sel = np.asarray(sel)
    T = sel.shape[0]
    nq = -(-T // seq_len)
    out = np.zeros((nq, E), dtype=np.int64)
    for q in range(nq):
        out[q] = expert_loads(sel[q * seq_len:(q + 1) * seq_len], E)
    return out


def expert_loads(sel: np.ndarray, E: int) -> np.ndarray:
    """Load of each routed expert in the batch: how many (token, slot) pairs
    chose it (section 2.2's per-batch selection count)."""
    sel = np.asarray(sel)
    return np.array([int(np.count_nonzero(sel == e)) for e in range(E)], dtype=np.int64)


def permutation(sel: np.ndarray, E: int):
    """Grouping of the T*K (token, slot) pairs by expert, in token order within
    each expert. Slot f = t*K + k. Returns (offsets [E+1], perm_slot [T*K]):
    rows offsets[e] .. offsets[e+1]-1 of the grouped order belong to expert e
    and perm_slot[p] is the slot placed at row p."""
    flat = np.asarray(sel).reshape(-1)
    groups = [np.flatnonzero(flat == e) for e in range(E)]
    counts = np.array([len(g) for g in groups], dtype=np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    perm = np.concatenate(groups) if groups else np.zeros(0, dtype=np.int64)
    return offsets, perm.astype(np.int64)


def silu(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_expert(v: np.ndarray, w1: np.ndarray, w3: np.ndarray, w2: np.ndarray) -> np.ndarray:
    """One SwiGLU expert on rows v [n, d]: W2 (SiLU(W1 v) * (W3 v)).
    w1, w3: [I, d]; w2: [d, I]. Returns [n, d]."""
    v = np.asarray(v, dtype=np.float64)
    h = silu(v @ np.asarray(w1, np.float64).T) * (v @ np.asarray(w3, np.float64).T)
    return h @ np.asarray(w2, np.float64).T


def route(x: np.ndarray, wr: np.ndarray, bias: Optional[np.ndarray], K: int,
          score_fn: str, norm: str, groups: Optional[tuple] = None) -> dict:
    """Gating of section 2.1/2.2 for every token: scores, biased top-K,
    gates from the unbiased scores, loads and the near-tie gap.

    groups = (G, M): node-limited routing of section 2.3 (select_groups) before
    the top-K; the group choice uses the affinity scores themselves (the bias
    of section 2.2 enters the expert choice only). A token is a near-tie when
    either its K-th and (K+1)-th allowed keys or its M-th and (M+1)-th group
    affinities differ by less than NEAR_TIE_GAP."""
    s = scores(router_logits(x, wr), score_fn)
    keys = s if bias is None else s + np.asarray(bias, dtype=np.float64)[None, :]
    out = {}
    near = np.zeros(s.shape[0], dtype=bool)
    cand = keys
    if groups is not None and groups[0] > 1:
        G, M = groups
        allowed, gs, ggap = select_groups(s, G, M)
        if M * (s.shape[1] // G) < K:
            raise ValueError("the kept groups hold fewer than K experts")
        cand = np.where(allowed, keys, -np.inf)
        near |= ggap < NEAR_TIE_GAP
        out.update({"allowed": allowed, "group_scores": gs, "group_gap": ggap})
    sel, gap = select_topk(cand, K)
    near |= gap < NEAR_TIE_GAP
    g = gate_values(s, sel, norm)
    out.update({"scores": s, "keys": keys, "sel": sel, "gate": g,
                "load": expert_loads(sel, s.shape[1]), "gap": gap, "near_tie": near})
    return out


def selection_valid(r: dict, idx: np.ndarray, K: int, groups: Optional[tuple] = None) -> np.ndarray:
    """Which rows of another implementation's selection idx [T, K] the
    routing r (from route(), same tokens) accepts. A set is accepted when it
    holds K distinct experts and either equals the oracle's set, or the token
    is a near-tie (r["near_tie"]) and the set is one the tie leaves open:
    every chosen key within NEAR_TIE_GAP of the oracle's K-th key; with
    node-limited routing (groups = (G, M)), at most M groups used, each with
    an affinity within NEAR_TIE_GAP of the M-th largest, and every chosen key
    within NEAR_TIE_GAP of the K-th largest key among the used groups'
    experts. Returns a boolean vector [T]."""
    idx = np.asarray(idx, dtype=np.int64)
    keys, sel, near = r["keys"], r["sel"], r["near_tie"]
    T, E = keys.shape
    inside = np.all((idx >= 0) & (idx < E), axis=1)
    srt = np.sort(np.clip(idx, 0, E - 1), axis=1)
    distinct = np.all(np.diff(srt, axis=1) > 0, axis=1) if K > 1 else np.ones(T, dtype=bool)
    same = np.all(srt == np.sort(sel, axis=1), axis=1)
    ok = inside & distinct & same
    chosen = np.take_along_axis(keys, np.clip(idx, 0, E - 1), axis=1)
    if groups is None or groups[0] <= 1:
        kth = np.take_along_axis(keys, sel[:, K - 1:K], axis=1)[:, 0]
        tie_ok = np.all(chosen >= kth[:, None] - NEAR_TIE_GAP, axis=1)
    else:
        G, M = groups
        n = E // G
        gs = r["group_scores"]
        mth = -np.sort(-gs, axis=1)[:, M - 1]
        tie_ok = np.zeros(T, dtype=bool)
        for t in np.flatnonzero(near & inside & distinct):
            used = np.unique(idx[t] // n)
            if len(used) > M or np.any(gs[t, used] < mth[t] - NEAR_TIE_GAP):
                continue
            pool = keys[t, (used[:, None] * n + np.arange(n)[None, :]).ravel()]
            kth_pool = np.sort(pool)[::-1][K - 1]
            tie_ok[t] = bool(np.all(keys[t, idx[t]] >= kth_pool - NEAR_TIE_GAP))
    return ok | (near & inside & distinct & tie_ok)


@dataclass
class ExpertBank:
    """Stored expert weights, decoded to float64 one expert at a time.

    `fetch(e)` returns the stored (w1, w3, w2, s1, s3, s2) of routed expert e
    (scales None unless fp8); `shared` holds the stored concatenated shared
    weights (w1s [S*Is, d], w3s, w2s [d, S*Is], s1s, s3s, s2s) and S."""
    fetch: Callable[[int], tuple]
    shared: Optional[tuple] = None
    S: int = 0

    def expert(self, e: int):
        w1, w3, w2, s1, s3, s2 = self.fetch(e)
        return decode_stored(w1, s1), decode_stored(w3, s3), decode_stored(w2, s2)

    def shared_experts(self):
        """The S shared experts as separate (w1, w3, w2) float64 triples."""
        if self.S == 0 or self.shared is None:
            return []
        w1s, w3s, w2s, s1s, s3s, s2s = self.shared
        W1, W3, W2 = decode_stored(w1s, s1s), decode_stored(w3s, s3s), decode_stored(w2s, s2s)
        Is = W1.shape[0] // self.S
        return [(W1[m * Is:(m + 1) * Is], W3[m * Is:(m + 1) * Is], W2[:, m * Is:(m + 1) * Is])
                for m in range(self.S)]


def layer_rows(x_rows: np.ndarray, sel: np.ndarray, gate: np.ndarray, bank: ExpertBank,
               experts: Optional[Sequence[int]] = None):
    """Layer output for the given token rows: y = sum_m Shared_m(x)
    + sum_k g_k E_{sel_k}(x) (section 1: shared experts always on, routed
    experts weighted by their gates; no residual). Returns (y, y_shared,
    routed [n, K, d]) where routed[:, k] = g_k E_{sel_k}(x)."""
    x_rows = np.asarray(x_rows, dtype=np.float64)
    n, d = x_rows.shape
    K = sel.shape[1]
    y_sh = np.zeros((n, d))
    for (w1, w3, w2) in bank.shared_experts():
        y_sh += swiglu_expert(x_rows, w1, w3, w2)
    routed = np.zeros((n, K, d))
    used = sorted(set(int(e) for e in np.unique(sel))) if experts is None else list(experts)
    for e in used:
        rows, ks = np.nonzero(sel == e)
        if len(rows) == 0:
            continue
        w1, w3, w2 = bank.expert(e)
        out = swiglu_expert(x_rows[rows], w1, w3, w2)
        routed[rows, ks] = gate[rows, ks][:, None] * out
    y = y_sh.copy()
    for k in range(K):
        y += routed[:, k]
    return y, y_sh, routed


def bias_update(bias: np.ndarray, load: np.ndarray, gamma: np.float32 = GAMMA_F32) -> np.ndarray:
    """Auxiliary-loss-free bias step ("DeepSeekMoE架构解析" section 2.2):
    b_i <- b_i - gamma * sign(load_i - mean_load), with mean_load = sum/E.
    The sign is decided in integers as sign(load_i * E - sum(load)); the fp32
    result is the exact difference rounded once to fp32."""
    bias = np.asarray(bias, dtype=np.float32)
    load = np.asarray(load, dtype=np.int64)
    E = bias.shape[0]
    if load.shape != (E,):
        raise ValueError("load must have one entry per expert")
    total = int(load.sum())
    sgn = np.sign(load * E - total).astype(np.float64)
    b64 = bias.astype(np.float64)
    step = float(np.float32(gamma)) * sgn
    new64 = b64 - step
    # The difference of two fp32 values is exact in fp64 when their exponents
    # are within 29 of each other; check it with exact rationals so the single
    # rounding below is the correctly rounded fp32 result.
    for b, st, nv in zip(b64.tolist(), step.tolist(), new64.tolist()):
        if Fraction(nv) != Fraction(b) - Fraction(st):
            raise ArithmeticError("fp64 difference not exact; bias too small relative to gamma")
    return new64.astype(np.float32)
