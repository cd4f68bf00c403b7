"""Fine-grained FP8 expert path, written out in float64 -- TEST INFRASTRUCTURE.

"DeepSeekMoE架构解析" section 4.3 names the scheme: activations are quantised
to fp8 in tiles of 1 x 128 (one scale per token per 128 consecutive
channels) and weights in blocks of 128 x 128, both with scales derived from
the tile's / block's max-abs, and the products are accumulated at full
precision with each 128-wide block of the reduction multiplied by its two
scales. The fp8 format is OCP E4M3FN (largest finite magnitude 448).

Readings of points the page leaves open (also listed in the design notes):
  * scale = amax / 448 of the tile, computed in fp32 (the precision of the
    scale the kernel keeps); an all-zero tile gets scale 1 (all codes 0).
  * code = the E4M3 value nearest to x / scale (fp32 division), ties to the
    even code; |x / scale| never exceeds 448 by more than rounding, which
    rounds back to 448.
  * The expert input x (bf16) is quantised in 1 x 128 tiles; the
    intermediate h = SiLU(W1 x) * (W3 x) is quantised the same way before the
    down projection (the kernel holds h in fp32, so the oracle rounds its
    float64 h to fp32 first: the quantisation decision is taken in the same
    precision on both sides).
  * Everything else -- the dequantised products, their sums, SiLU, the gate
    weighting -- is float64.
The router stays in bf16 / float64 (section 4.3 concerns the GEMMs).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np

from .formats import E4M3_TABLE, bf16_to_f64, e4m3_to_f64
from .moe import silu

E4M3_MAX = 448.0
TILE = 128

# non-negative finite E4M3 values by code 0x00 .. 0x7E (increasing)
_POS = E4M3_TABLE[:0x7F]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3FN code to each finite value (ties to the even code),
    |v| <= 448 after rounding. Sign-magnitude: a negative value that rounds
    to zero gets the negative-zero code 0x80."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("finite values only")
    a = np.abs(v)
    if np.any(a > E4M3_MAX + 16.0):
        raise ValueError("value beyond the E4M3 range")
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, 0x7E)   # first value >= a
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - _POS[lo], _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(a >= _POS[0x7E], 0x7E, np.where(pick_hi, hi, lo)).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x80), code).astype(np.uint8)


def quantize_tiles(x: np.ndarray, tile: int = TILE):
    """1 x `tile` quantisation of an fp32 matrix [n, C] (C % tile == 0):
    returns (codes uint8 [n, C], scales float32 [n, C / tile])."""
    x = np.asarray(x)
    if x.dtype != np.float32:
        raise TypeError("tile quantisation takes fp32 values")
    n, C = x.shape
    if C % tile:
        raise ValueError("columns must be a multiple of the tile")
    t = x.reshape(n, C // tile, tile)
    amax = np.max(np.abs(t), axis=2)                                    # exact in fp32
    s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (t / s[:, :, None]).astype(np.float32)                          # fp32 division
    return e4m3_encode(q).reshape(n, C), s


def dequantize_tiles(codes: np.ndarray, scales: np.ndarray, tile: int = TILE) -> np.ndarray:
    codes = np.asarray(codes)
    n, C = codes.shape
    return (e4m3_to_f64(codes).reshape(n, C // tile, tile)
            * np.asarray(scales, np.float64)[:, :, None]).reshape(n, C)


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray, block: int = TILE) -> np.ndarray:
    """Weights [R, C] stored as E4M3 codes with one fp32 scale per
    `block` x `block` block: scales [R / block, C / block]."""
    codes = np.asarray(codes)
    R, C = codes.shape
    s = np.asarray(scales, np.float64)
    if s.shape != (R // block, C // block) or R % block or C % block:
        raise ValueError("block scales do not match the weight shape")
    full = np.repeat(np.repeat(s, block, axis=0), block, axis=1)
    return e4m3_to_f64(codes) * full


def expert_h_fp8(xq: np.ndarray, xs: np.ndarray, w1, w3) -> np.ndarray:
    """The intermediate of one SwiGLU expert on quantised rows, h = SiLU(W1 x)
    * (W3 x) in float64 from the dequantised tokens (xq codes [n, d], tile
    scales xs [n, d/128]) and weights (w1, w3 [I, d] float64), rounded to the
    fp32 value that the 1 x 128 quantisation of h starts from."""
    x = dequantize_tiles(xq, xs)
    return (silu(x @ w1.T) * (x @ w3.T)).astype(np.float32)


def swiglu_expert_fp8(xq: np.ndarray, xs: np.ndarray, w1, w3, w2) -> np.ndarray:
    """One SwiGLU expert on quantised rows (w2 [d, I] float64): h from
    expert_h_fp8, quantised in 1 x 128 tiles, then W2 h.
    Returns (out [n, d] float64, hq, hs)."""
    hq, hs = quantize_tiles(expert_h_fp8(xq, xs, w1, w3))
    return dequantize_tiles(hq, hs) @ w2.T, hq, hs


@dataclass
class BlockExpertBank:
    """Stored fp8 expert weights with 128 x 128 block scales, decoded to
    float64 one expert at a time. `fetch(e)` returns (w1, w3, w2, s1, s3, s2):
    codes w1, w3 [I, d], w2 [d, I]; scales s1, s3 [I/128, d/128],
    s2 [d/128, I/128]. `shared` = (w1s [S*Is, d], w3s, w2s [d, S*Is], s1s,
    s3s, s2s) for the S shared experts concatenated (Is % 128 == 0)."""
    fetch: Callable[[int], tuple]
    shared: Optional[tuple] = None
    S: int = 0

    def expert(self, e: int):
        w1, w3, w2, s1, s3, s2 = self.fetch(e)
        return dequantize_blocks(w1, s1), dequantize_blocks(w3, s3), dequantize_blocks(w2, s2)

    def shared_experts(self):
        if self.S == 0 or self.shared is None:
            return []
        w1s, w3s, w2s, s1s, s3s, s2s = self.shared
        W1, W3, W2 = dequantize_blocks(w1s, s1s), dequantize_blocks(w3s, s3s), dequantize_blocks(w2s, s2s)
        Is = W1.shape[0] // self.S
        return [(W1[m * Is:(m + 1) * Is], W3[m * Is:(m + 1) * Is], W2[:, m * Is:(m + 1) * Is])
                for m in range(self.S)]


def quantize_x(x_bf16: np.ndarray):
    """The layer input (bf16 bit patterns [n, d]) in 1 x 128 tiles."""
    return quantize_tiles(bf16_to_f64(x_bf16).astype(np.float32))


def layer_rows_fp8(x_bf16: np.ndarray, sel: np.ndarray, gate: np.ndarray, bank: BlockExpertBank,
                   experts: Optional[Sequence[int]] = None):
    """Layer output for the given token rows with the fine-grained fp8
    experts: y = sum_m Shared_m(x) + sum_k g_k E_{sel_k}(x), every expert on
    the tile-quantised x. Returns (y, y_shared, routed [n, K, d])."""
    xq, xs = quantize_x(x_bf16)
    n, d = xq.shape
    K = sel.shape[1]
    y_sh = np.zeros((n, d))
    for (w1, w3, w2) in bank.shared_experts():
        y_sh += swiglu_expert_fp8(xq, xs, w1, w3, w2)[0]
    routed = np.zeros((n, K, d))
    used = sorted(set(int(e) for e in np.unique(sel))) if experts is None else list(experts)
    for e in used:
        rows, ks = np.nonzero(sel == e)
        if len(rows) == 0:
            continue
        w1, w3, w2 = bank.expert(e)
        out = swiglu_expert_fp8(xq[rows], xs[rows], w1, w3, w2)[0]
        routed[rows, ks] = gate[rows, ks][:, None] * out
    y = y_sh.copy()
    for k in range(K):
        y += routed[:, k]
    return y, y_sh, routed
