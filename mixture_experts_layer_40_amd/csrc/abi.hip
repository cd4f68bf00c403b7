// The C ABI of libmoe: host-side argument validation, workspace sizes and
// status strings, then the kernel launchers. Nothing here touches the GPU
// before every argument has been checked, so invalid calls return an error
// without a device present.
#include <math.h>

#include "launch.hpp"
#include "libmoe.h"

using namespace moe;

namespace {

constexpr int64_t kInt32Max = 2147483647LL;

bool aligned256(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 255u) == 0; }

// Every device pointer the kernels read or write in 16-byte pieces must be
// 16-byte aligned; NULL (an absent optional argument) passes.
template <class... P>
bool aligned16(P... p) {
  return ((((reinterpret_cast<uintptr_t>(static_cast<const void*>(p)) & 15u) == 0)) && ...);
}

int check_ws(size_t need, const void* ws, size_t ws_bytes) {
  if (need == 0) return MOE_OK;
  if (!ws || ws_bytes < need || !aligned256(ws)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

int from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool is_fp8(const moe_config* c) { return c->weight_dtype == MOE_DTYPE_FP8_E4M3; }

bool is_tiled(const moe_config* c) { return c->weight_layout == MOE_LAYOUT_TILED; }

// The second gate/up weight pointer: required in the rows layout, NULL in the
// tiled one (its rows live in the tiled gate/up tensor).
int check_w3(const moe_config* c, const void* w3) {
  if (is_tiled(c)) return w3 ? MOE_ERR_SHAPE : MOE_OK;
  return w3 ? MOE_OK : MOE_ERR_NULL;
}

// fp8 weights need all three scale arrays; other weight types take none.
int check_scales(const moe_config* c, const float* a, const float* b, const float* d) {
  if (is_fp8(c)) return (a && b && d) ? MOE_OK : MOE_ERR_NULL;
  return (!a && !b && !d) ? MOE_OK : MOE_ERR_DTYPE;
}

// The fine-grained fp8 experts: bf16 activations quantised in 1 x 128 tiles,
// fp8 weights in the tiled layout with 128 x 128 block scales; every
// reduction length and weight-row count a multiple of 128, at most 8192.
int check_fp8_block(const moe_config* c) {
  if (c->act_dtype != MOE_DTYPE_BF16 || c->weight_dtype != MOE_DTYPE_FP8_E4M3) return MOE_ERR_DTYPE;
  if (c->weight_layout != MOE_LAYOUT_TILED) return MOE_ERR_SHAPE;
  const int64_t si = static_cast<int64_t>(c->num_shared) * c->shared_inter;
  if (c->hidden % 128 != 0 || c->inter % 128 != 0 || (c->num_shared > 0 && si % 128 != 0))
    return MOE_ERR_SHAPE;
  if (c->hidden > 8192 || c->inter > 8192 || si > 8192) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

}  // namespace

extern "C" {

int moe_validate(const moe_config* c) {
  if (!c) return MOE_ERR_NULL;
  if (c->act_dtype != MOE_DTYPE_F32 && c->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (c->act_dtype == MOE_DTYPE_F32 && c->weight_dtype != MOE_DTYPE_F32) return MOE_ERR_DTYPE;
  if (c->act_dtype == MOE_DTYPE_BF16 && c->weight_dtype != MOE_DTYPE_BF16 &&
      c->weight_dtype != MOE_DTYPE_FP8_E4M3)
    return MOE_ERR_DTYPE;
  if (c->out_dtype != MOE_DTYPE_F32 && c->out_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (c->act_dtype == MOE_DTYPE_F32 && c->out_dtype != MOE_DTYPE_F32) return MOE_ERR_DTYPE;
  if (c->slot_dtype != MOE_DTYPE_F32 && c->slot_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (c->act_dtype == MOE_DTYPE_F32 && c->slot_dtype != MOE_DTYPE_F32) return MOE_ERR_DTYPE;
  if (c->weight_layout != MOE_LAYOUT_ROWS && c->weight_layout != MOE_LAYOUT_TILED)
    return MOE_ERR_SHAPE;
  if (c->weight_layout == MOE_LAYOUT_TILED && c->weight_dtype == MOE_DTYPE_F32)
    return MOE_ERR_DTYPE;
  if (c->score_fn != MOE_SCORE_SIGMOID && c->score_fn != MOE_SCORE_SOFTMAX) return MOE_ERR_SHAPE;
  if (c->norm != MOE_NORM_SELECTED && c->norm != MOE_NORM_NONE &&
      c->norm != MOE_NORM_ONE_PLUS_SELECTED)
    return MOE_ERR_SHAPE;
  if (c->num_tokens < 0) return MOE_ERR_SHAPE;
  if (c->num_experts < 1 || c->num_experts > 256) return MOE_ERR_SHAPE;
  if (c->top_k < 1 || c->top_k > c->num_experts) return MOE_ERR_SHAPE;
  if (c->hidden <= 0 || c->hidden % 64 != 0) return MOE_ERR_SHAPE;
  if (c->inter <= 0 || c->inter % 64 != 0) return MOE_ERR_SHAPE;
  if (c->num_shared < 0) return MOE_ERR_SHAPE;
  if (c->num_shared > 0) {
    const int64_t si = static_cast<int64_t>(c->num_shared) * c->shared_inter;
    if (c->shared_inter <= 0 || si % 64 != 0 || si > kInt32Max) return MOE_ERR_SHAPE;
  }
  const int64_t tk = static_cast<int64_t>(c->num_tokens) * c->top_k;
  if (tk >= (1LL << 30)) return MOE_ERR_SHAPE;
  // grouped GEMM tiles are indexed in int and launched as one grid
  if (grouped_tiles_bound(*c) > (1LL << 30)) return MOE_ERR_UNSUPPORTED;
  if (c->num_groups < 0) return MOE_ERR_SHAPE;
  if (c->num_groups > 1) {
    const int G = c->num_groups, M = c->topk_groups;
    if (G > 64 || c->num_experts % G != 0) return MOE_ERR_SHAPE;
    if (M < 1 || M > G || static_cast<int64_t>(M) * (c->num_experts / G) < c->top_k)
      return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

size_t moe_workspace_size(const moe_config* c, int which) {
  if (moe_validate(c) != MOE_OK) return 0;
  switch (which) {
    case MOE_WS_ROUTE: return route_ws_bytes(*c);
    case MOE_WS_PERMUTE: return c->num_tokens == 0 ? 0 : permute_ws_bytes(*c);
    case MOE_WS_FFN: return c->num_tokens == 0 ? 0 : ffn_ws_bytes(*c);
    case MOE_WS_SHARED: return (c->num_tokens == 0 || c->num_shared == 0) ? 0 : shared_ws_bytes(*c);
    case MOE_WS_GEMM: return c->num_tokens == 0 ? 0 : sched_ws_bytes(*c);
    case MOE_WS_EXPERTS: return c->num_tokens == 0 ? 0 : experts_ws_bytes(*c);
    case MOE_WS_EXPERTS_FP8:
      return (c->num_tokens == 0 || check_fp8_block(c) != MOE_OK) ? 0 : experts_fp8_ws_bytes(*c);
    default: return 0;
  }
}

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: sizes out of range or not supported";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE: invalid dtype or dtype combination";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: not implemented";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, too small or misaligned";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: the HIP runtime reported an error";
    case MOE_ERR_SCRATCH:
      return "MOE_ERR_SCRATCH: the request needs more than the 1 MiB scratch array of "
             "moe_permute_noalloc";
    default: return "unknown libmoe status";
  }
}

int moe_pack_weights(int which, int32_t groups, int32_t rows, int32_t cols, int32_t weight_dtype,
                     const void* src_a, const void* src_b, void* dst, void* stream) {
  if (which != MOE_PACK_GATE_UP && which != MOE_PACK_DOWN) return MOE_ERR_SHAPE;
  if (weight_dtype != MOE_DTYPE_BF16 && weight_dtype != MOE_DTYPE_FP8_E4M3) return MOE_ERR_DTYPE;
  if (groups < 1 || rows < 1 || cols < 1 || cols % 64 != 0) return MOE_ERR_SHAPE;
  if (rows % (which == MOE_PACK_GATE_UP ? 16 : 32) != 0) return MOE_ERR_SHAPE;
  if (!src_a || !dst) return MOE_ERR_NULL;
  if (which == MOE_PACK_GATE_UP ? !src_b : src_b != nullptr)
    return which == MOE_PACK_GATE_UP ? MOE_ERR_NULL : MOE_ERR_SHAPE;
  if (!aligned16(src_a, src_b, dst)) return MOE_ERR_SHAPE;
  const int wbytes = weight_dtype == MOE_DTYPE_BF16 ? 2 : 1;
  (void)hipGetLastError();
  return from_hip(launch_pack(which == MOE_PACK_GATE_UP ? 0 : 1, groups, rows, cols, wbytes, src_a,
                              src_b, dst, as_stream(stream)));
}

int moe_route(const moe_config* c, const void* x, const void* w_router, const float* bias,
              int32_t* topk_idx, float* topk_gate, int32_t* load, void* ws, size_t ws_bytes,
              void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (!load) return MOE_ERR_NULL;
  if (c->num_tokens > 0 && (!x || !w_router || !topk_idx || !topk_gate)) return MOE_ERR_NULL;
  if (!aligned16(x, w_router, bias, topk_idx, topk_gate, load)) return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_ROUTE), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_route(*c, x, w_router, bias, topk_idx, topk_gate, load, ws,
                               as_stream(stream)));
}

int moe_permute(const moe_config* c, const int32_t* topk_idx, const void* x,
                int32_t* expert_offsets, int32_t* perm_slot, void* x_perm, void* ws,
                size_t ws_bytes, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (!expert_offsets) return MOE_ERR_NULL;
  if (c->num_tokens > 0 && (!topk_idx || !perm_slot || (x_perm && !x))) return MOE_ERR_NULL;
  if (!aligned16(topk_idx, x, expert_offsets, perm_slot, x_perm)) return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_PERMUTE), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_permute(*c, topk_idx, x, expert_offsets, perm_slot, x_perm, ws,
                                 as_stream(stream)));
}

int moe_expert_ffn(const moe_config* c, const void* x_perm, const int32_t* expert_offsets,
                   const int32_t* perm_slot, const float* topk_gate, const void* w1,
                   const void* w3, const void* w2, const float* s1, const float* s3,
                   const float* s2, void* out_slots, void* ws, size_t ws_bytes, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if ((st = check_scales(c, s1, s3, s2)) != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  if ((st = check_w3(c, w3)) != MOE_OK) return st;
  if (!x_perm || !expert_offsets || !perm_slot || !topk_gate || !w1 || !w2 || !out_slots)
    return MOE_ERR_NULL;
  if (!aligned16(x_perm, expert_offsets, perm_slot, topk_gate, w1, w3, w2, s1, s3, s2, out_slots))
    return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_FFN), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_expert_ffn(*c, x_perm, expert_offsets, perm_slot, topk_gate, w1, w3, w2,
                                    s1, s3, s2, out_slots, ws, as_stream(stream)));
}

int moe_expert_gate_up(const moe_config* c, const void* x_perm, const int32_t* expert_offsets,
                       const void* w1, const void* w3, const float* s1, const float* s3, void* h,
                       void* ws, size_t ws_bytes, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if ((st = check_scales(c, s1, s3, s3)) != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  if ((st = check_w3(c, w3)) != MOE_OK) return st;
  if (!x_perm || !expert_offsets || !w1 || !h) return MOE_ERR_NULL;
  if (!aligned16(x_perm, expert_offsets, w1, w3, s1, s3, h)) return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_GEMM), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_gate_up(*c, x_perm, expert_offsets, w1, w3, s1, s3, h, ws,
                                 as_stream(stream)));
}

int moe_expert_down(const moe_config* c, const void* h, const int32_t* expert_offsets,
                    const int32_t* perm_slot, const float* topk_gate, const void* w2,
                    const float* s2, void* out_slots, void* ws, size_t ws_bytes, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if ((st = check_scales(c, s2, s2, s2)) != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  if (!h || !expert_offsets || !perm_slot || !topk_gate || !w2 || !out_slots) return MOE_ERR_NULL;
  if (!aligned16(h, expert_offsets, perm_slot, topk_gate, w2, s2, out_slots)) return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_GEMM), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_down(*c, h, expert_offsets, perm_slot, topk_gate, w2, s2, out_slots, ws,
                              as_stream(stream)));
}

int moe_shared_ffn(const moe_config* c, const void* x, const void* w1s, const void* w3s,
                   const void* w2s, const float* s1s, const float* s3s, const float* s2s,
                   void* y_shared, void* ws, size_t ws_bytes, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (c->num_shared == 0) return MOE_ERR_SHAPE;
  if ((st = check_scales(c, s1s, s3s, s2s)) != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  if ((st = check_w3(c, w3s)) != MOE_OK) return st;
  if (!x || !w1s || !w2s || !y_shared) return MOE_ERR_NULL;
  if (!aligned16(x, w1s, w3s, w2s, s1s, s3s, s2s, y_shared)) return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_SHARED), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_shared_ffn(*c, x, w1s, w3s, w2s, s1s, s3s, s2s, y_shared, ws,
                                    as_stream(stream)));
}

int moe_experts(const moe_config* c, const void* x, const int32_t* expert_offsets,
                const int32_t* perm_slot, const float* topk_gate, const void* w1, const void* w3,
                const void* w2, const float* s1, const float* s3, const float* s2,
                const void* w1s, const void* w3s, const void* w2s, const float* s1s,
                const float* s3s, const float* s2s, void* out_slots, void* y_shared, void* ws,
                size_t ws_bytes, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (c->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if ((st = check_scales(c, s1, s3, s2)) != MOE_OK) return st;
  if (c->num_shared > 0) {
    if ((st = check_scales(c, s1s, s3s, s2s)) != MOE_OK) return st;
  } else if (w1s || w3s || w2s || s1s || s3s || s2s || y_shared) {
    return MOE_ERR_SHAPE;
  }
  if (c->num_tokens == 0) return MOE_OK;
  if ((st = check_w3(c, w3)) != MOE_OK) return st;
  if (!x || !expert_offsets || !perm_slot || !topk_gate || !w1 || !w2 || !out_slots)
    return MOE_ERR_NULL;
  if (c->num_shared > 0) {
    if ((st = check_w3(c, w3s)) != MOE_OK) return st;
    if (!w1s || !w2s || !y_shared) return MOE_ERR_NULL;
  }
  if (!aligned16(x, expert_offsets, perm_slot, topk_gate, w1, w3, w2, s1, s3, s2, w1s, w3s, w2s,
                 s1s, s3s, s2s, out_slots, y_shared))
    return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_EXPERTS), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_experts(*c, x, expert_offsets, perm_slot, topk_gate, w1, w3, w2, s1, s3,
                                 s2, w1s, w3s, w2s, s1s, s3s, s2s, out_slots, y_shared, ws,
                                 as_stream(stream)));
}

int moe_experts_gate_up(const moe_config* c, const void* x, const int32_t* expert_offsets,
                        const int32_t* perm_slot, const void* w1, const void* w3,
                        const float* s1, const float* s3, const void* w1s, const void* w3s,
                        const float* s1s, const float* s3s, void* h, void* hs, void* ws,
                        size_t ws_bytes, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (c->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if ((st = check_scales(c, s1, s3, s3)) != MOE_OK) return st;
  if (c->num_shared > 0) {
    if ((st = check_scales(c, s1s, s3s, s3s)) != MOE_OK) return st;
  } else if (w1s || w3s || s1s || s3s || hs) {
    return MOE_ERR_SHAPE;
  }
  if (c->num_tokens == 0) return MOE_OK;
  if ((st = check_w3(c, w3)) != MOE_OK) return st;
  if (!x || !expert_offsets || !perm_slot || !w1 || !h) return MOE_ERR_NULL;
  if (c->num_shared > 0) {
    if ((st = check_w3(c, w3s)) != MOE_OK) return st;
    if (!w1s || !hs) return MOE_ERR_NULL;
  }
  if (!aligned16(x, expert_offsets, perm_slot, w1, w3, s1, s3, w1s, w3s, s1s, s3s, h, hs))
    return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_GEMM), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_experts_gate_up(*c, x, expert_offsets, perm_slot, w1, w3, s1, s3, w1s,
                                         w3s, s1s, s3s, h, hs, ws, as_stream(stream)));
}

int moe_experts_down(const moe_config* c, const void* h, const void* hs,
                     const int32_t* expert_offsets, const int32_t* perm_slot,
                     const float* topk_gate, const void* w2, const float* s2, const void* w2s,
                     const float* s2s, void* out_slots, void* y_shared, void* ws,
                     size_t ws_bytes, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (c->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if ((st = check_scales(c, s2, s2, s2)) != MOE_OK) return st;
  if (c->num_shared > 0) {
    if ((st = check_scales(c, s2s, s2s, s2s)) != MOE_OK) return st;
  } else if (hs || w2s || s2s || y_shared) {
    return MOE_ERR_SHAPE;
  }
  if (c->num_tokens == 0) return MOE_OK;
  if (!h || !expert_offsets || !perm_slot || !topk_gate || !w2 || !out_slots) return MOE_ERR_NULL;
  if (c->num_shared > 0 && (!hs || !w2s || !y_shared)) return MOE_ERR_NULL;
  if (!aligned16(h, hs, expert_offsets, perm_slot, topk_gate, w2, s2, w2s, s2s, out_slots,
                 y_shared))
    return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_GEMM), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_experts_down(*c, h, hs, expert_offsets, perm_slot, topk_gate, w2, s2,
                                      w2s, s2s, out_slots, y_shared, ws, as_stream(stream)));
}

int moe_quantize_act(const moe_config* c, const void* x, void* xq, float* xs, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (c->act_dtype != MOE_DTYPE_BF16) return MOE_ERR_DTYPE;
  if (c->hidden % 128 != 0) return MOE_ERR_SHAPE;
  if (c->num_tokens == 0) return MOE_OK;
  if (!x || !xq || !xs) return MOE_ERR_NULL;
  if (!aligned16(x, xq, xs)) return MOE_ERR_SHAPE;
  (void)hipGetLastError();
  return from_hip(launch_quantize_act(*c, x, xq, xs, as_stream(stream)));
}

int moe_experts_fp8(const moe_config* c, const void* xq, const float* xs,
                    const int32_t* expert_offsets, const int32_t* perm_slot,
                    const float* topk_gate, const void* w13, const void* w2, const float* s1,
                    const float* s3, const float* s2, const void* w13s, const void* w2s,
                    const float* s1s, const float* s3s, const float* s2s, void* out_slots,
                    void* y_shared, void* ws, size_t ws_bytes, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if ((st = check_fp8_block(c)) != MOE_OK) return st;
  if (c->num_shared == 0 && (w13s || w2s || s1s || s3s || s2s || y_shared)) return MOE_ERR_SHAPE;
  if (c->num_tokens == 0) return MOE_OK;
  if (!xq || !xs || !expert_offsets || !perm_slot || !topk_gate || !w13 || !w2 || !s1 || !s3 ||
      !s2 || !out_slots)
    return MOE_ERR_NULL;
  if (c->num_shared > 0 && (!w13s || !w2s || !s1s || !s3s || !s2s || !y_shared)) return MOE_ERR_NULL;
  if (!aligned16(xq, xs, expert_offsets, perm_slot, topk_gate, w13, w2, s1, s3, s2, w13s, w2s, s1s,
                 s3s, s2s, out_slots, y_shared))
    return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_EXPERTS_FP8), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_experts_fp8(*c, xq, xs, expert_offsets, perm_slot, topk_gate, w13, w2, s1,
                                     s3, s2, w13s, w2s, s1s, s3s, s2s, out_slots, y_shared, ws,
                                     as_stream(stream)));
}

int moe_experts_fp8_gate_up(const moe_config* c, const void* xq, const float* xs,
                            const int32_t* expert_offsets, const int32_t* perm_slot,
                            const void* w13, const float* s1, const float* s3, const void* w13s,
                            const float* s1s, const float* s3s, void* hq, float* hs, void* hsq,
                            float* hss, void* ws, size_t ws_bytes, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if ((st = check_fp8_block(c)) != MOE_OK) return st;
  if (c->num_shared == 0 && (w13s || s1s || s3s || hsq || hss)) return MOE_ERR_SHAPE;
  if (c->num_tokens == 0) return MOE_OK;
  if (!xq || !xs || !expert_offsets || !perm_slot || !w13 || !s1 || !s3 || !hq || !hs)
    return MOE_ERR_NULL;
  if (c->num_shared > 0 && (!w13s || !s1s || !s3s || !hsq || !hss)) return MOE_ERR_NULL;
  if (!aligned16(xq, xs, expert_offsets, perm_slot, w13, s1, s3, w13s, s1s, s3s, hq, hs, hsq, hss))
    return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_GEMM), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_experts_fp8_gate_up(*c, xq, xs, expert_offsets, perm_slot, w13, s1, s3,
                                             w13s, s1s, s3s, hq, hs, hsq, hss, ws,
                                             as_stream(stream)));
}

int moe_experts_fp8_down(const moe_config* c, const void* hq, const float* hs, const void* hsq,
                         const float* hss, const int32_t* expert_offsets,
                         const int32_t* perm_slot, const float* topk_gate, const void* w2,
                         const float* s2, const void* w2s, const float* s2s, void* out_slots,
                         void* y_shared, void* ws, size_t ws_bytes, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if ((st = check_fp8_block(c)) != MOE_OK) return st;
  if (c->num_shared == 0 && (hsq || hss || w2s || s2s || y_shared)) return MOE_ERR_SHAPE;
  if (c->num_tokens == 0) return MOE_OK;
  if (!hq || !hs || !expert_offsets || !perm_slot || !topk_gate || !w2 || !s2 || !out_slots)
    return MOE_ERR_NULL;
  if (c->num_shared > 0 && (!hsq || !hss || !w2s || !s2s || !y_shared)) return MOE_ERR_NULL;
  if (!aligned16(hq, hs, hsq, hss, expert_offsets, perm_slot, topk_gate, w2, s2, w2s, s2s,
                 out_slots, y_shared))
    return MOE_ERR_SHAPE;
  if ((st = check_ws(moe_workspace_size(c, MOE_WS_GEMM), ws, ws_bytes)) != MOE_OK) return st;
  (void)hipGetLastError();
  return from_hip(launch_experts_fp8_down(*c, hq, hs, hsq, hss, expert_offsets, perm_slot,
                                          topk_gate, w2, s2, w2s, s2s, out_slots, y_shared, ws,
                                          as_stream(stream)));
}

int moe_combine(const moe_config* c, const void* out_slots, const void* y_shared, void* y,
                void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  if (!out_slots || !y) return MOE_ERR_NULL;
  if (!aligned16(out_slots, y_shared, y)) return MOE_ERR_SHAPE;
  (void)hipGetLastError();
  return from_hip(launch_combine(*c, out_slots, y_shared, nullptr, y, as_stream(stream)));
}

int moe_combine_residual(const moe_config* c, const void* out_slots, const void* y_shared,
                         const void* residual, void* y, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (c->num_tokens == 0) return MOE_OK;
  if (!out_slots || !residual || !y) return MOE_ERR_NULL;
  if (!aligned16(out_slots, y_shared, residual, y)) return MOE_ERR_SHAPE;
  (void)hipGetLastError();
  return from_hip(launch_combine(*c, out_slots, y_shared, residual, y, as_stream(stream)));
}

int moe_rmsnorm(const moe_config* c, const void* x, const float* weight, double eps, void* u,
                void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (!(eps > 0.0) || isinf(eps)) return MOE_ERR_SHAPE;
  // one block per token keeps its row in registers: at most 16384 elements
  if (c->hidden > (c->act_dtype == MOE_DTYPE_BF16 ? 16384 : 8192)) return MOE_ERR_UNSUPPORTED;
  if (c->num_tokens == 0) return MOE_OK;
  if (!x || !weight || !u) return MOE_ERR_NULL;
  if (!aligned16(x, weight, u)) return MOE_ERR_SHAPE;
  (void)hipGetLastError();
  return from_hip(launch_rmsnorm(*c, x, weight, eps, u, as_stream(stream)));
}

int moe_sequence_loads(const moe_config* c, const int32_t* topk_idx, int32_t seq_len,
                       int32_t* seq_load, void* stream) {
  int st = moe_validate(c);
  if (st != MOE_OK) return st;
  if (seq_len < 1) return MOE_ERR_SHAPE;
  if (c->num_tokens == 0) return MOE_OK;
  if (!topk_idx || !seq_load) return MOE_ERR_NULL;
  if (!aligned16(topk_idx, seq_load)) return MOE_ERR_SHAPE;
  (void)hipGetLastError();
  return from_hip(launch_sequence_loads(*c, topk_idx, seq_len, seq_load, as_stream(stream)));
}

int moe_bias_update(int32_t num_experts, const int32_t* load, float gamma, float* bias,
                    void* stream) {
  if (num_experts < 1 || num_experts > 256) return MOE_ERR_SHAPE;
  if (!load || !bias) return MOE_ERR_NULL;
  if (!aligned16(load, bias)) return MOE_ERR_SHAPE;
  if (!(gamma >= 0.0f) || isinf(gamma)) return MOE_ERR_SHAPE;
  (void)hipGetLastError();
  return from_hip(launch_bias_update(num_experts, load, gamma, bias, as_stream(stream)));
}

}  // extern "C"
