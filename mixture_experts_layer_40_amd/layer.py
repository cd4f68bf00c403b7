"""One DeepSeekMoE layer call through the C ABI, with its buffers held in HBM.

MoELayer keeps the weights the caller hands it (torch tensors on the GPU, in
their stored formats) and allocates every intermediate buffer once, sized
for `max_tokens`. With layout="tiled" (the default for bf16 / fp8 weights)
it relocates the expert weights once into the tiled layout of
moe_pack_weights and keeps only that copy's references for the calls.
forward() enqueues, on the current stream,

    fused (default with bf16 activations):
        moe_shared_ffn (second stream, from the start of the call)
        ||  moe_route -> moe_permute (no row gather) -> moe_experts (routed
            experts only) -> join -> moe_combine
        (with shared_stream=False: moe_route -> moe_permute -> moe_experts,
        shared and routed experts in one launch each -> moe_combine)
    fine-grained fp8 (weights with 128 x 128 block scales):
        moe_route -> moe_permute (no row gather) -> moe_quantize_act
        -> moe_experts_fp8 -> moe_combine
    otherwise:
        moe_shared_ffn (second stream)  ||  moe_route -> moe_permute -> moe_expert_ffn
        -> join -> moe_combine

and returns y (plus the routing results it kept). The per-batch bias step is
`bias_update()`; `capture()` records a call into a HIP graph for replay.
Nothing here computes: every step is a libmoe kernel.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import torch

from . import _lib as L

_TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


class MoELayer:
    def __init__(self, spec, weights: dict, max_tokens: Optional[int] = None,
                 shared_stream: bool = True, device=None, layout: Optional[str] = None,
                 fused: Optional[bool] = None, pre_norm: bool = False, residual: bool = False,
                 slot_dtype: Optional[str] = None):
        self.spec = spec
        self.device = torch.device(device) if device is not None else weights["wr"].device
        self.max_tokens = spec.T if max_tokens is None else max_tokens
        self.act = _TORCH_DT[spec.act_dtype]
        if layout is None:
            layout = "rows" if spec.weight_dtype == "f32" else "tiled"
        self.layout = layout
        self.fused = spec.act_dtype == "bf16" if fused is None else fused
        self.fp8_block = getattr(spec, "fp8_scaling", "row") == "block"
        if self.fp8_block and (layout != "tiled" or not self.fused):
            raise ValueError("block-scaled fp8 experts run fused on the tiled layout")
        self.pre_norm, self.residual = pre_norm, residual
        # out_slots: fp32 unless the workload (or the caller) asks for bf16
        self.slot_dtype = slot_dtype or getattr(spec, "slot_dtype", "f32")
        self.w = dict(weights)
        if layout == "tiled":
            wd = spec.weight_dtype
            self.w["w1"] = L.pack_gate_up(weights["w1"], weights["w3"], wd)
            self.w["w3"] = None
            self.w["w2"] = L.pack_down(weights["w2"], wd)
            if spec.S > 0:
                self.w["w1s"] = L.pack_gate_up(weights["w1s"], weights["w3s"], wd)
                self.w["w3s"] = None
                self.w["w2s"] = L.pack_down(weights["w2s"], wd)
        self.cfg_max = L.config_of(spec, T=self.max_tokens, weight_layout=layout,
                                   slot_dtype=self.slot_dtype)
        st = L.moe_validate(self.cfg_max)
        if st != L.MOE_OK:
            raise L.MoEError("MoELayer", st, L.moe_status_string(st))
        T, K, d, E = self.max_tokens, spec.K, spec.d, spec.E
        dev = self.device
        self.topk_idx = torch.empty((T, K), dtype=torch.int32, device=dev)
        self.topk_gate = torch.empty((T, K), dtype=torch.float32, device=dev)
        self.load = torch.empty((E,), dtype=torch.int32, device=dev)
        self.expert_offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
        self.perm_slot = torch.empty((T * K,), dtype=torch.int32, device=dev)
        self.x_perm = torch.empty((T * K, d), dtype=self.act, device=dev)
        self.out_slots = torch.empty((T * K, d), dtype=_TORCH_DT[self.slot_dtype], device=dev)
        self.y_shared = torch.empty((T, d), dtype=torch.float32, device=dev) if spec.S > 0 else None
        self.y = torch.empty((T, d), dtype=_TORCH_DT[getattr(spec, "out_dtype", "f32")], device=dev)
        self.u = torch.empty((T, d), dtype=self.act, device=dev) if pre_norm else None

        def ws(which):
            n = L.moe_workspace_size(self.cfg_max, which)
            return torch.empty(max(n, 256), dtype=torch.uint8, device=dev)
        self.ws_route = ws(L.MOE_WS_ROUTE)
        self.ws_perm = ws(L.MOE_WS_PERMUTE)
        self.ws_ffn = ws(L.MOE_WS_FFN)
        self.ws_shared = ws(L.MOE_WS_SHARED)
        self.ws_experts = ws(L.MOE_WS_EXPERTS) if self.fused and not self.fp8_block else None
        if self.fp8_block:
            self.xq = torch.empty((T, d), dtype=torch.uint8, device=dev)
            self.xs = torch.empty((T, d // 128), dtype=torch.float32, device=dev)
            self.ws_experts = ws(L.MOE_WS_EXPERTS_FP8)
        # The shared experts do not depend on the routing: on a second stream
        # they run while the router and the sort leave most of the part idle
        # (measured on one box, alternated, identical outputs: the 2024
        # layout 0.758 -> 0.723 ms, the V3 prefill layer 7.47 -> 7.37 ms,
        # decode unchanged). The routed experts then run as moe_experts with
        # no shared set (spec_routed).
        self.side = (torch.cuda.Stream(device=dev)
                     if (shared_stream and spec.S > 0 and not self.fp8_block) else None)
        self.spec_routed = dataclasses.replace(spec, S=0, Is=0) if spec.S > 0 else spec

    def _cfg(self, T):
        if T > self.max_tokens:
            raise ValueError(f"{T} tokens exceed the layer's buffers ({self.max_tokens})")
        return L.config_of(self.spec, T=T, weight_layout=self.layout, slot_dtype=self.slot_dtype)

    def route(self, x, bias=None):
        T = x.shape[0]
        cfg = self._cfg(T)
        L.moe_route(cfg, x, self.w["wr"], bias, self.topk_idx[:T], self.topk_gate[:T], self.load,
                    ws=self.ws_route)
        return cfg

    def permute(self, cfg, x, gather=True):
        T = cfg.num_tokens
        L.moe_permute(cfg, self.topk_idx[:T], x if gather else None, self.expert_offsets,
                      self.perm_slot[:T * cfg.top_k],
                      self.x_perm[:T * cfg.top_k] if gather else None, ws=self.ws_perm)

    def routed_cfg(self, T):
        """The configuration of the routed experts alone (no shared set)."""
        return L.config_of(self.spec_routed, T=T, weight_layout=self.layout,
                           slot_dtype=self.slot_dtype)

    def experts_fused(self, cfg, x, with_shared=True):
        """moe_experts over the routed experts, and the shared ones too
        unless with_shared is False (they then run through shared())."""
        T, w = cfg.num_tokens, self.w
        if not with_shared and self.y_shared is not None:
            L.moe_experts(self.routed_cfg(T), x, self.expert_offsets,
                          self.perm_slot[:T * cfg.top_k], self.topk_gate[:T], w["w1"], w["w3"],
                          w["w2"], w.get("s1"), w.get("s3"), w.get("s2"), None, None, None, None,
                          None, None, self.out_slots[:T * cfg.top_k], None, ws=self.ws_experts)
            return
        L.moe_experts(cfg, x, self.expert_offsets, self.perm_slot[:T * cfg.top_k],
                      self.topk_gate[:T], w["w1"], w["w3"], w["w2"], w.get("s1"), w.get("s3"),
                      w.get("s2"), w.get("w1s"), w.get("w3s"), w.get("w2s"), w.get("s1s"),
                      w.get("s3s"), w.get("s2s"), self.out_slots[:T * cfg.top_k],
                      None if self.y_shared is None else self.y_shared[:T], ws=self.ws_experts)

    def experts_fp8(self, cfg, x):
        T, w = cfg.num_tokens, self.w
        L.moe_quantize_act(cfg, x, self.xq[:T], self.xs[:T])
        L.moe_experts_fp8(cfg, self.xq[:T], self.xs[:T], self.expert_offsets,
                          self.perm_slot[:T * cfg.top_k], self.topk_gate[:T], w["w1"], w["w2"],
                          w["s1"], w["s3"], w["s2"], w.get("w1s"), w.get("w2s"), w.get("s1s"),
                          w.get("s3s"), w.get("s2s"), self.out_slots[:T * cfg.top_k],
                          None if self.y_shared is None else self.y_shared[:T], ws=self.ws_experts)

    def experts(self, cfg):
        T, w = cfg.num_tokens, self.w
        L.moe_expert_ffn(cfg, self.x_perm[:T * cfg.top_k], self.expert_offsets,
                         self.perm_slot[:T * cfg.top_k], self.topk_gate[:T], w["w1"], w["w3"],
                         w["w2"], w.get("s1"), w.get("s3"), w.get("s2"),
                         self.out_slots[:T * cfg.top_k], ws=self.ws_ffn)

    def shared(self, cfg, x, stream=None):
        T, w = cfg.num_tokens, self.w
        L.moe_shared_ffn(cfg, x, w["w1s"], w["w3s"], w["w2s"], w.get("s1s"), w.get("s3s"),
                         w.get("s2s"), self.y_shared[:T], ws=self.ws_shared, stream=stream)

    def combine(self, cfg, residual=None):
        T = cfg.num_tokens
        ysh = None if self.y_shared is None else self.y_shared[:T]
        if residual is None:
            L.moe_combine(cfg, self.out_slots[:T * cfg.top_k], ysh, self.y[:T])
        else:
            L.moe_combine_residual(cfg, self.out_slots[:T * cfg.top_k], ysh, residual, self.y[:T])

    def forward(self, x, bias=None):
        """Enqueue one layer call on the current stream; returns y [T, d].
        With pre_norm the experts and the router see u = RMSNorm(x) (weight
        weights["norm_w"], eps 1e-6); with residual, y = x + the expert sum."""
        cfg = self._cfg(x.shape[0])
        if cfg.num_tokens == 0:
            L.moe_route(cfg, x, self.w["wr"], bias, None, None, self.load, ws=self.ws_route)
            return self.y[:0]
        res = x if self.residual else None
        if self.pre_norm:
            L.moe_rmsnorm(cfg, x, self.w["norm_w"], self.u[:cfg.num_tokens])
            x = self.u[:cfg.num_tokens]
        cur = torch.cuda.current_stream(self.device)
        if self.fused:
            if self.side is not None:
                self.side.wait_stream(cur)
                with torch.cuda.stream(self.side):
                    self.shared(cfg, x, stream=self.side)
            self.route(x, bias)
            self.permute(cfg, x, gather=False)
            if self.fp8_block:
                self.experts_fp8(cfg, x)
            else:
                self.experts_fused(cfg, x, with_shared=self.side is None)
            if self.side is not None:
                cur.wait_stream(self.side)
            self.combine(cfg, res)
            return self.y[:cfg.num_tokens]
        if self.side is not None:
            self.side.wait_stream(cur)
            with torch.cuda.stream(self.side):
                self.shared(cfg, x, stream=self.side)
        elif self.y_shared is not None:
            self.shared(cfg, x)
        self.route(x, bias)
        self.permute(cfg, x)
        self.experts(cfg)
        if self.side is not None:
            cur.wait_stream(self.side)
        self.combine(cfg, res)
        return self.y[:cfg.num_tokens]

    def capture(self, x, bias=None):
        """Record one forward(x, bias) into a HIP graph and return it
        (torch.cuda.CUDAGraph): a launch-bound caller -- few tokens, the fp32
        layer -- then reruns the whole call sequence with graph.replay(). x,
        bias and the layer's outputs keep their addresses, so new inputs are
        written into x before a replay. Every node is a libmoe kernel (no
        memset nodes), so each replay recomputes everything."""
        cur = torch.cuda.current_stream(self.device)
        warm = torch.cuda.Stream(device=self.device)
        warm.wait_stream(cur)
        with torch.cuda.stream(warm):
            self.forward(x, bias)
        cur.wait_stream(warm)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            self.forward(x, bias)
        return graph

    def bias_update(self, bias, gamma=None):
        L.moe_bias_update(self.spec.E, self.load, self.spec.gamma if gamma is None else gamma, bias)
