// Host-side launchers of the libmoe kernels (internal to the library).
// The C ABI in abi.hip validates arguments, then calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "libmoe.h"

namespace moe {

// ---- route ------------------------------------------------------------------
// Router path chosen from the shape alone: a fused GEMM + score + top-K kernel
// for bf16 with many tokens; otherwise a split-K logits kernel (bf16 MFMA or
// fp32) into the workspace followed by a score + top-K kernel.
bool route_uses_fused(const moe_config& c);
int route_k_splits(const moe_config& c);
size_t route_ws_bytes(const moe_config& c);
hipError_t launch_route(const moe_config& c, const void* x, const void* wr, const float* bias,
                        int32_t* topk_idx, float* topk_gate, int32_t* load, void* ws,
                        hipStream_t s);

// ---- permute ----------------------------------------------------------------
size_t permute_ws_bytes(const moe_config& c);
hipError_t launch_permute(const moe_config& c, const int32_t* topk_idx, const void* x,
                          int32_t* expert_offsets, int32_t* perm_slot, void* x_perm, void* ws,
                          hipStream_t s);

// ---- expert FFN (routed and shared) ------------------------------------------
size_t ffn_ws_bytes(const moe_config& c);
size_t sched_ws_bytes(const moe_config& c);
// Largest grid (tile count) of any grouped GEMM launch of this configuration.
int64_t grouped_tiles_bound(const moe_config& c);
size_t shared_ws_bytes(const moe_config& c);
hipError_t launch_gate_up(const moe_config& c, const void* x_perm, const int32_t* expert_offsets,
                          const void* w1, const void* w3, const float* s1, const float* s3,
                          void* h, void* ws, hipStream_t s);
hipError_t launch_down(const moe_config& c, const void* h, const int32_t* expert_offsets,
                       const int32_t* perm_slot, const float* topk_gate, const void* w2,
                       const float* s2, void* out_slots, void* ws, hipStream_t s);
hipError_t launch_expert_ffn(const moe_config& c, const void* x_perm,
                             const int32_t* expert_offsets, const int32_t* perm_slot,
                             const float* topk_gate, const void* w1, const void* w3,
                             const void* w2, const float* s1, const float* s3, const float* s2,
                             void* out_slots, void* ws, hipStream_t s);
size_t experts_ws_bytes(const moe_config& c);
// With `scheduled`, ws already holds the launch's tile table (moe_experts
// computes both launches' tables in one pass).
hipError_t launch_experts_gate_up(const moe_config& c, const void* x,
                                  const int32_t* expert_offsets, const int32_t* perm_slot,
                                  const void* w1, const void* w3, const float* s1,
                                  const float* s3, const void* w1s, const void* w3s,
                                  const float* s1s, const float* s3s, void* h, void* hs,
                                  void* ws, hipStream_t s, bool scheduled = false);
hipError_t launch_experts_down(const moe_config& c, const void* h, const void* hs,
                               const int32_t* expert_offsets, const int32_t* perm_slot,
                               const float* topk_gate, const void* w2, const float* s2,
                               const void* w2s, const float* s2s, void* out_slots,
                               void* y_shared, void* ws, hipStream_t s, bool scheduled = false);
hipError_t launch_experts(const moe_config& c, const void* x, const int32_t* expert_offsets,
                          const int32_t* perm_slot, const float* topk_gate, const void* w1,
                          const void* w3, const void* w2, const float* s1, const float* s3,
                          const float* s2, const void* w1s, const void* w3s, const void* w2s,
                          const float* s1s, const float* s3s, const float* s2s, void* out_slots,
                          void* y_shared, void* ws, hipStream_t s);
hipError_t launch_shared_ffn(const moe_config& c, const void* x, const void* w1s,
                             const void* w3s, const void* w2s, const float* s1s,
                             const float* s3s, const float* s2s, void* y_shared, void* ws,
                             hipStream_t s);

// ---- fine-grained fp8 experts (128 x 128 weight blocks, 1 x 128 token tiles) --
hipError_t launch_quantize_act(const moe_config& c, const void* x, void* xq, float* xs,
                               hipStream_t s);
size_t experts_fp8_ws_bytes(const moe_config& c);
hipError_t launch_experts_fp8_gate_up(const moe_config& c, const void* xq, const float* xs,
                                      const int32_t* expert_offsets, const int32_t* perm_slot,
                                      const void* w13, const float* s1, const float* s3,
                                      const void* w13s, const float* s1s, const float* s3s,
                                      void* hq, float* hs, void* hsq, float* hss, void* ws,
                                      hipStream_t s);
hipError_t launch_experts_fp8_down(const moe_config& c, const void* hq, const float* hs,
                                   const void* hsq, const float* hss,
                                   const int32_t* expert_offsets, const int32_t* perm_slot,
                                   const float* topk_gate, const void* w2, const float* s2,
                                   const void* w2s, const float* s2s, void* out_slots,
                                   void* y_shared, void* ws, hipStream_t s);
hipError_t launch_experts_fp8(const moe_config& c, const void* xq, const float* xs,
                              const int32_t* expert_offsets, const int32_t* perm_slot,
                              const float* topk_gate, const void* w13, const void* w2,
                              const float* s1, const float* s3, const float* s2,
                              const void* w13s, const void* w2s, const float* s1s,
                              const float* s3s, const float* s2s, void* out_slots,
                              void* y_shared, void* ws, hipStream_t s);

hipError_t launch_sequence_loads(const moe_config& c, const int32_t* topk_idx, int seq_len,
                                 int32_t* seq_load, hipStream_t s);

// Rows -> tiled layout of expert weights. which: 0 = gate/up (a = W1, b = W3,
// each [groups, rows, cols]), 1 = down (a = W2 [groups, rows, cols], b unused).
hipError_t launch_pack(int which, int64_t groups, int rows, int cols, int wbytes,
                       const void* a, const void* b, void* dst, hipStream_t s);

// ---- combine / bias ----------------------------------------------------------
hipError_t launch_combine(const moe_config& c, const void* out_slots, const void* y_shared,
                          const void* residual, void* y, hipStream_t s);
hipError_t launch_rmsnorm(const moe_config& c, const void* x, const float* weight, double eps,
                          void* u, hipStream_t s);
hipError_t launch_bias_update(int32_t E, const int32_t* load, float gamma, float* bias,
                              hipStream_t s);
hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s);

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

}  // namespace moe
