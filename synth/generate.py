"""Seeded tensor generation in the stored formats the layer consumes.

Every tensor is drawn from its own torch.Generator, seeded from
(config seed, tensor tag, index), on the device the caller names. Values are
drawn in fp32 and rounded once to the storage type (bf16 round-to-nearest-even,
or fp8-e4m3 codes with one fp32 scale per output row). The same stored tensors
are then handed to the HIP path and, copied to host, to the oracle.

Draws on "cuda" and on "cpu" differ (different generator streams); each run
generates once and both sides read the same values.

Layouts (row-major, contiguous):
  x   [T, d]            act dtype
  wr  [E, d]            act dtype (router rows = expert centroids)
  bias[E]               fp32 (or None)
  w1, w3 [E, I, d]      weight dtype (gate / up projections)
  w2     [E, d, I]      weight dtype (down projection)
  s1, s3 [E, I], s2 [E, d]      fp32 per-output-row scales (fp8 only), or with
                                fp8_scaling "block": s1, s3 [E, I/128, d/128],
                                s2 [E, d/128, I/128], one per 128 x 128 block
  w1s, w3s [S*Is, d], w2s [d, S*Is]  shared experts concatenated
  s1s, s3s [S*Is], s2s [d]           fp32 scales (fp8 only; block: [S*Is/128, d/128], [d/128, S*Is/128])
  norm_w [d]                          fp32 RMSNorm weight for the optional pre-norm
"""

from __future__ import annotations

import hashlib
from typing import Dict, Optional

import numpy as np
import torch

from .configs import MoEConfig

E4M3_MAX = 448.0

_TAGS = {"x": 1, "wr": 2, "bias": 3, "w1": 4, "w3": 5, "w2": 6,
         "w1s": 7, "w3s": 8, "w2s": 9, "perm": 10, "norm_w": 11}


def _seed(base: int, tag: str, idx: int = 0) -> int:
    h = hashlib.sha256(f"{base}:{_TAGS[tag]}:{idx}".encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, base, tag, idx=0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(base, tag, idx))
    return g


def _normal(shape, std, device, base, tag, idx=0) -> torch.Tensor:
    g = _gen(device, base, tag, idx)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _store_act(v: torch.Tensor, dtype: str) -> torch.Tensor:
    if dtype == "f32":
        return v.contiguous()
    if dtype == "bf16":
        return v.to(torch.bfloat16).contiguous()
    raise ValueError(dtype)


def _quant_fp8_rows(w: torch.Tensor):
    """Per-output-row fp8-e4m3 quantisation: scale = amax/448, code = RNE(w/scale)."""
    amax = w.abs().amax(dim=-1, keepdim=True)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (w / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), scale.squeeze(-1).to(torch.float32).contiguous()


def _quant_fp8_blocks(w: torch.Tensor, block: int = 128):
    """128 x 128 block fp8-e4m3 quantisation of a [R, C] matrix: one scale
    amax/448 per block (1 for an all-zero block), code = RNE(w/scale)."""
    R, C = w.shape
    t = w.reshape(R // block, block, C // block, block)
    amax = t.abs().amax(dim=(1, 3), keepdim=True)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax))
    q = (t / scale).clamp_(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn).reshape(R, C)
    return q.view(torch.uint8), scale.reshape(R // block, C // block).to(torch.float32).contiguous()


def _store_weight(v: torch.Tensor, dtype: str, scaling: str = "row"):
    if dtype == "fp8":
        return _quant_fp8_blocks(v) if scaling == "block" else _quant_fp8_rows(v)
    return _store_act(v, dtype), None


def make_x(cfg: MoEConfig, device="cpu", batch: int = 0, T: Optional[int] = None) -> torch.Tensor:
    """Token activations [T, d] for batch `batch` of the workload."""
    T = cfg.T if T is None else T
    v = _normal((T, cfg.d), cfg.x_std, device, cfg.seed, "x", batch)
    if cfg.zipf_s is not None:
        v[:, 0] = 1.0   # constant coordinate that carries the popularity offsets
    return _store_act(v, cfg.act_dtype)


def zipf_offsets(cfg: MoEConfig, device="cpu") -> torch.Tensor:
    """Router logit offsets o_e = A * rank(e)^(-s) over a seeded expert ranking."""
    g = _gen("cpu", cfg.seed, "perm")
    order = torch.randperm(cfg.E, generator=g)          # order[r-1] = expert of rank r
    rank = torch.empty(cfg.E, dtype=torch.float64)
    rank[order] = torch.arange(1, cfg.E + 1, dtype=torch.float64)
    off = cfg.zipf_A * rank.pow(-cfg.zipf_s)
    return off.to(torch.float32).to(device)


def make_inputs(cfg: MoEConfig, device="cpu", batch: int = 0,
                with_experts: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    dev = torch.device(device)
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = make_x(cfg, dev, batch)

    wr = _normal((cfg.E, cfg.d), cfg.w_std, dev, cfg.seed, "wr")
    if cfg.zipf_s is not None:
        wr[:, 0] = zipf_offsets(cfg, dev)
    out["wr"] = _store_act(wr, cfg.act_dtype)

    # RMSNorm weight of the optional pre-norm: 1 + N(0, 0.1^2) per channel, fp32
    out["norm_w"] = (1.0 + _normal((cfg.d,), 0.1, dev, cfg.seed, "norm_w")).float().contiguous()

    if cfg.bias_range is not None:
        g = _gen(dev, cfg.seed, "bias")
        b = (torch.rand((cfg.E,), generator=g, device=dev, dtype=torch.float32) * 2.0 - 1.0) * cfg.bias_range
        out["bias"] = b.contiguous()
    else:
        out["bias"] = None

    if not with_experts:
        return out

    wdt = cfg.weight_dtype
    stored_dt = {"f32": torch.float32, "bf16": torch.bfloat16, "fp8": torch.uint8}[wdt]
    E, I, d = cfg.E, cfg.I, cfg.d
    block = wdt == "fp8" and cfg.fp8_scaling == "block"
    for name, shape in (("w1", (I, d)), ("w3", (I, d)), ("w2", (d, I))):
        buf = torch.empty((E,) + shape, dtype=stored_dt, device=dev)
        sshape = (E, shape[0] // 128, shape[1] // 128) if block else (E, shape[0])
        sc = torch.empty(sshape, dtype=torch.float32, device=dev) if wdt == "fp8" else None
        for e in range(E):
            v = _normal(shape, cfg.w_std, dev, cfg.seed, name, e)
            q, s = _store_weight(v, wdt, cfg.fp8_scaling)
            buf[e].copy_(q)
            if sc is not None:
                sc[e].copy_(s)
            del v, q
        out[name] = buf
        out["s" + name[1]] = sc

    if cfg.S > 0:
        SI = cfg.S * cfg.Is
        for name, shape in (("w1s", (SI, d)), ("w3s", (SI, d)), ("w2s", (d, SI))):
            v = _normal(shape, cfg.w_std, dev, cfg.seed, name)
            q, s = _store_weight(v, wdt, cfg.fp8_scaling)
            out[name] = q
            out["s" + name[1] + "s"] = s
    else:
        for name in ("w1s", "w3s", "w2s", "s1s", "s3s", "s2s"):
            out[name] = None
    return out


def to_numpy_stored(t: Optional[torch.Tensor]):
    """Host copy of a stored tensor as numpy: bf16 -> uint16 bits, fp8 -> uint8
    codes, fp32 -> float32. The oracle decodes these itself."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype == torch.uint8:
        return t.cpu().numpy()
    if t.dtype == torch.float32:
        return t.cpu().numpy()
    if t.dtype == torch.int32:
        return t.cpu().numpy()
    raise TypeError(t.dtype)
