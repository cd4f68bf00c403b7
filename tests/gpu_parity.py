"""Shared helpers of the GPU parity tests: run the HIP path step by step on
seeded inputs and compare every result with the fp64 oracle.

The bar (the tolerances of the layer's specification):
  * expert indices and load counts bit-exact, except tokens whose K-th and
    (K+1)-th biased keys differ by less than 1e-5 in the oracle (near-ties):
    those are counted and their GPU set must be valid within 1e-5;
  * permutation and offsets bit-exact (they are defined by the indices);
  * outputs: max |GPU - oracle| <= 2e-2 * RMS(oracle) for bf16/fp8 paths and
    <= 1e-4 * RMS(oracle) for the fp32 path, elementwise over the layer
    output y and the shared-expert output, with nothing added to the bar;
    near-tie tokens are compared with the oracle evaluated on the GPU's
    selected set.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import mixture_experts_layer_40_amd as moe
import oracle
import synth

OUT_TOL = {"f32": 1e-4, "bf16": 2e-2}
GATE_ATOL = 2e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t):
    return synth.to_numpy_stored(t)


def f64(t):
    return oracle.decode_stored(host(t))


def bank_of(inp, spec):
    def fetch(e):
        sc = lambda n: None if inp.get(n) is None else inp[n][e].cpu().numpy()
        return (host(inp["w1"][e]), host(inp["w3"][e]), host(inp["w2"][e]), sc("s1"), sc("s3"), sc("s2"))
    shared = None
    if spec.S > 0:
        sc = lambda n: None if inp.get(n) is None else inp[n].cpu().numpy()
        shared = (host(inp["w1s"]), host(inp["w3s"]), host(inp["w2s"]), sc("s1s"), sc("s3s"), sc("s2s"))
    return oracle.ExpertBank(fetch=fetch, shared=shared, S=spec.S)


def run_steps(spec, inp, bias=None, x=None, layer=None, side_stream=False, fused=None):
    """One layer call through the C ABI, step by step; returns host copies."""
    x = inp["x"] if x is None else x
    if layer is None:
        layer = moe.MoELayer(spec, inp, max_tokens=x.shape[0], shared_stream=side_stream,
                             fused=fused)
    y = layer.forward(x, bias)
    torch.cuda.synchronize()
    T, K = x.shape[0], spec.K
    return layer, {
        "idx": layer.topk_idx[:T].cpu().numpy().astype(np.int64),
        "gate": layer.topk_gate[:T].cpu().numpy().astype(np.float64),
        "load": layer.load.cpu().numpy().astype(np.int64),
        "offsets": layer.expert_offsets.cpu().numpy().astype(np.int64),
        "perm": layer.perm_slot[:T * K].cpu().numpy().astype(np.int64),
        "y": y,
    }


def groups_of(spec):
    G = getattr(spec, "n_groups", 0)
    return (G, spec.topk_groups) if G > 1 else None


def oracle_route(spec, x, wr, bias, rows=None):
    x64 = f64(x) if rows is None else f64(x[rows])
    b64 = None if bias is None else bias.detach().cpu().numpy().astype(np.float64)
    return oracle.route(x64, f64(wr), b64, spec.K, spec.score, spec.norm,
                        groups=groups_of(spec)), x64


def check_route(spec, r, idx, gate, load=None, rows=None):
    """Routing parity on the tokens `rows` (all when None). Returns the number
    of near-tie tokens."""
    K, E = spec.K, spec.E
    idx_r = idx if rows is None else idx[rows]
    gate_r = gate if rows is None else gate[rows]
    assert idx_r.min() >= 0 and idx_r.max() < E
    srt = np.sort(idx_r, axis=1)
    assert np.all(np.diff(srt, axis=1) > 0), "a token selected an expert twice"
    if load is not None:
        assert np.array_equal(load, np.bincount(idx.ravel(), minlength=E)), "load != histogram of indices"
        assert int(load.sum()) == idx.shape[0] * K, "a token was dropped"
    near = r["near_tie"]
    ok = ~near
    # sets equal to the oracle's outside near-ties; inside them, one of the
    # sets the tie leaves open (oracle.selection_valid)
    valid = oracle.selection_valid(r, idx_r, K, groups_of(spec))
    bad = np.flatnonzero(~valid)
    assert bad.size == 0, (f"{bad.size} tokens have a selection the oracle does not accept, "
                           f"e.g. {bad[:5]} (near-tie: {near[bad[:5]].tolist()})")
    assert np.array_equal(np.bincount(idx_r[ok].ravel(), minlength=E),
                          np.bincount(r["sel"][ok].ravel(), minlength=E))
    g_or = oracle.gate_values(r["scores"], idx_r, spec.norm)
    err = np.abs(gate_r - g_or).max()
    assert err <= GATE_ATOL, f"gate error {err}"
    return int(near.sum())


def check_permutation(spec, idx, offsets, perm):
    off_or, perm_or = oracle.permutation(idx, spec.E)
    assert np.array_equal(offsets, off_or), "expert offsets differ"
    assert np.array_equal(perm, perm_or), "permutation differs"


def rel_err(got, want):
    """max |got - want| / RMS(want), and RMS(want)."""
    rms = float(np.sqrt(np.mean(want ** 2)))
    return float(np.abs(got - want).max()) / max(rms, 1e-300), rms


# Relative rounding of one value stored in a dtype: bf16 keeps 8 significant
# bits (round to nearest: at most 2^-8 of the value), fp32 24.
STORE_REL = {"bf16": 2.0 ** -8, "f32": 2.0 ** -24}


def check_slot_rows(osl, want, slot_dtype, tol):
    """The routed slot rows [n, K, d] (an intermediate of the layer, held in
    the slot dtype) against the oracle's gate-weighted expert outputs: each
    (token, slot) row's error, beyond the element's own storage rounding in
    the slot dtype, within tol of that row's RMS. Returns the worst ratio."""
    rms_row = np.sqrt(np.mean(want ** 2, axis=2, keepdims=True))
    excess = np.abs(osl - want) - STORE_REL[slot_dtype] * np.abs(want)
    e_o = float((excess / np.maximum(rms_row, 1e-300)).max())
    assert e_o <= tol, f"out_slots: {e_o:.3e}"
    return e_o


def check_outputs(spec, layer, inp, res, r, x=None, rows=None, residual=None):
    """Layer output (and its shared and routed parts) on `rows` against the
    oracle. `r` is the oracle routing of all tokens of the batch. The oracle
    uses its own selected set, except on near-tie tokens, where any set
    within 1e-5 is correct: there it evaluates the (validated) GPU set."""
    x = inp["x"] if x is None else x
    T, K, d = x.shape[0], spec.K, spec.d
    rows = np.arange(T) if rows is None else np.asarray(rows)
    trow = torch.as_tensor(rows, device=x.device)
    x64 = f64(x[trow])
    gpu_idx = res["idx"][rows]
    sel = r["sel"][rows].copy()
    near = r["near_tie"][rows]
    sel[near] = gpu_idx[near]
    g_or = oracle.gate_values(r["scores"][rows], sel, spec.norm)
    y_or, ysh_or, routed_or = oracle.layer_rows(x64, sel, g_or, bank_of(inp, spec))
    tol = OUT_TOL[spec.act_dtype]
    y = oracle.decode_stored(host(res["y"][trow].contiguous()))
    if residual is not None:
        # y = residual + expert sum: the error is measured against the
        # expert sum's own RMS (the residual itself enters exactly)
        y = y - residual[rows]
    e_y, rms = rel_err(y, y_or)
    assert e_y <= tol, f"y: max err / RMS = {e_y:.3e} > {tol}"
    if spec.S > 0:
        ysh = oracle.decode_stored(host(layer.y_shared[trow].contiguous()))
        e_s, _ = rel_err(ysh, ysh_or)
        assert e_s <= tol, f"y_shared: {e_s:.3e}"
    # routed slot rows: GPU slot (t, k) holds expert gpu_idx[t, k]; line the
    # oracle's terms up by expert id (the sets are equal, checked above)
    aligned = np.empty_like(routed_or)
    og, oo = np.argsort(gpu_idx, axis=1), np.argsort(sel, axis=1)
    for i in range(len(rows)):
        aligned[i, og[i]] = routed_or[i, oo[i]]
    slot_rows = (trow[:, None] * K + torch.arange(K, device=x.device)[None, :]).reshape(-1)
    osl = oracle.decode_stored(host(layer.out_slots[slot_rows].contiguous())).reshape(len(rows), K, d)
    e_o = check_slot_rows(osl, aligned, layer.slot_dtype, tol)
    return {"y_err": e_y, "y_rms": rms, "slot_err": e_o}


def sample_rows(T, n, near, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, min(n, T), replace=False).tolist())
    rows.update(np.flatnonzero(near)[:4].tolist())
    return np.array(sorted(rows))


def tile_bm(rows_per_expert):
    """Token-tile height the grouped GEMMs pick for this many expected rows
    per expert (32 / 64 / 128 / 256; the fine-grained fp8 kernels stop at
    128)."""
    for bm in (32, 64, 128):
        if rows_per_expert <= bm:
            return bm
    return 256


def tile_edge_tokens(offsets, perm, K, E, T, max_bm=256):
    """Tokens owning the first and the last row of every token tile of every
    expert: an expert's m rows are split into ceil(m / bm) tiles of equal
    height (a multiple of 32 rows), the last one ragged."""
    bm = min(tile_bm(-(-T * K // E)), max_bm)
    toks = set()
    for e in range(E):
        m = int(offsets[e + 1] - offsets[e])
        if m == 0:
            continue
        mt = -(-m // bm)
        per = ((-(-m // mt)) + 31) & ~31
        for j in range(mt):
            for p in (j * per, min(m, (j + 1) * per) - 1):
                toks.add(int(perm[offsets[e] + p]) // K)
    return toks


def coverage_rows(offsets, perm, spec, near_tie, n_random=12, max_bm=256):
    """The tokens owning every token tile's first and last row, a few random
    tokens and the first near-ties, sorted."""
    toks = tile_edge_tokens(offsets, perm, spec.K, spec.E, spec.T, max_bm)
    toks.update(sample_rows(spec.T, n_random, near_tie).tolist())
    return np.array(sorted(toks))
