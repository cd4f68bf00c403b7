// Router of the DeepSeekMoE layer: affinity GEMM, score, bias-adjusted top-K,
// gate normalisation and per-expert load counts.
//
// Method: "DeepSeekMoE架构解析" section 2.1 (eq. 15: s = sigmoid(u^T e_i);
// eq. 14: keep the K largest; eq. 13: divide by the sum of the kept scores)
// and section 2.2 (eq. 16: the balance bias b_i is added to the score only
// for the choice of experts, never to the gate value). The 2024 layout
// (course notes "省钱第一招", sections 三-四) uses a softmax over all routed
// experts and keeps the selected scores unnormalised.
//
// Top-K on CDNA4: one wave per token. Lane l holds the keys of experts
// l, l+64, l+128, l+192 (E <= 256) in registers; each of the K rounds takes a
// lane-local best, then a 6-step xor butterfly over (key, index) pairs with
// the total order "larger key first, then lower index", so every lane ends
// with the same winner and the result is deterministic.
#include <math.h>

#include "common.hpp"
#include "gemm_core.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kFusedTokens = 32;     // tokens per block of the fused router
constexpr int kFusedMinTokens = 4096;

__device__ __forceinline__ bool key_better(float ka, int ia, float kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ float pick4(const float (&v)[4], int j) {
  return j == 0 ? v[0] : (j == 1 ? v[1] : (j == 2 ? v[2] : v[3]));
}

// Scores, top-K, gates for one token on one wave. lg[j] is the logit of
// expert (lane + 64 j); entries with expert >= E are ignored. G > 1: only the
// experts of the M groups with the largest score sums take part
// ("DeepSeekMoE架构解析" section 2.3, node-limited routing).
__device__ void topk_token(const float (&lg)[4], int t, int E, int K, int G, int M, int score_fn,
                           int norm, const float* __restrict__ bias,
                           int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
                           int* hist) {
  const int l = lane_id();
  float s[4], key[4];
  if (score_fn == MOE_SCORE_SIGMOID) {
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = sigmoid(lg[j]);
  } else {
    float m = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (l + 64 * j < E) m = fmaxf(m, lg[j]);
    m = wave_max(m);
    float ex[4], part = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ex[j] = (l + 64 * j < E) ? expf(lg[j] - m) : 0.f;
      part += ex[j];
    }
    const float sum = wave_sum(part);
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] = ex[j] / sum;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = l + 64 * j;
    key[j] = e < E ? (bias ? s[j] + bias[e] : s[j]) : -INFINITY;
  }
  if (G > 1) {
    // group affinity = sum of its experts' scores; lane g ends with group g's
    const int n = E / G;
    int grp[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) grp[j] = (l + 64 * j) < E ? (l + 64 * j) / n : -1;
    float gsum = -INFINITY;
    for (int gi = 0; gi < G; ++gi) {
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) part += grp[j] == gi ? s[j] : 0.f;
      const float tot = wave_sum(part);
      if (l == gi) gsum = tot;
    }
    // keep the M largest (ties: lower group index)
    uint64_t keep = 0;
    for (int r = 0; r < M; ++r) {
      float bv = gsum;
      int bi = l;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ov = __shfl_xor(bv, o, kWave);
        const int oi = __shfl_xor(bi, o, kWave);
        if (key_better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
      }
      keep |= 1ull << bi;
      if (l == bi) gsum = -INFINITY;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (grp[j] >= 0 && !((keep >> grp[j]) & 1ull)) key[j] = -INFINITY;
  }

  int rec_idx[4] = {0, 0, 0, 0};
  float rec_s[4] = {0.f, 0.f, 0.f, 0.f};
  float ssum = 0.f;
  for (int k = 0; k < K; ++k) {
    float bk = key[0];
    int bi = l;
#pragma unroll
    for (int j = 1; j < 4; ++j)
      if (key_better(key[j], l + 64 * j, bk, bi)) { bk = key[j]; bi = l + 64 * j; }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ok = __shfl_xor(bk, o, kWave);
      const int oi = __shfl_xor(bi, o, kWave);
      if (key_better(ok, oi, bk, bi)) { bk = ok; bi = oi; }
    }
    const int owner = bi & 63, slot = bi >> 6;
    const float sv = __shfl(pick4(s, slot), owner, kWave);
    if (l == owner) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == slot) key[j] = -INFINITY;
    }
    ssum += sv;
    if (l == (k & 63)) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j == (k >> 6)) { rec_idx[j] = bi; rec_s[j] = sv; }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int k = l + 64 * j;
    if (k < K) {
      const size_t o = static_cast<size_t>(t) * K + k;
      topk_idx[o] = rec_idx[j];
      topk_gate[o] = norm == MOE_NORM_SELECTED ? rec_s[j] / ssum
                   : norm == MOE_NORM_ONE_PLUS_SELECTED ? rec_s[j] / (1.0f + ssum)
                   : rec_s[j];
      atomicAdd(&hist[rec_idx[j]], 1);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused path (bf16, many tokens): one block = 32 tokens x all E (<= 256)
// experts, in the shape of the expert GEMMs' K loop: 8 waves, wave w streams
// router rows 32w .. 32w+31 into MFMA operands, the 32-token tile is shared
// through LDS. The logits stay in LDS; each wave then runs the top-K of 4
// tokens. Rows past E (E < 256) are computed on a repeated row and dropped.
// wr_tiled: the router rows in the tiled layout of the expert weights (see
// pack_tiles; E a multiple of 32), so that each weight load instruction
// reads one contiguous 1 KB stripe instead of 16 bytes from each of 64 row
// pieces; else row-major.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void route_fused_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int wr_tiled,
    const float* __restrict__ bias, int T, int d, int E, int K, int G, int M, int score_fn,
    int norm, int32_t* __restrict__ topk_idx, float* __restrict__ topk_gate,
    int32_t* __restrict__ load) {
  constexpr int BT = kFusedTokens;
  __shared__ __attribute__((aligned(16))) uint16_t bs0[BT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t bs1[BT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t bs2[BT * 64];
  __shared__ __attribute__((aligned(16))) uint16_t bs3[MOE_TOKEN_STAGES > 3 ? BT * 64 : 8];
  __shared__ float lgs[BT][257];
  __shared__ int hist[256];

  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 5, r32 = l & 31;
  const int t0 = blockIdx.x * BT;
  const int mvalid = min(BT, T - t0);
  if (tid < 256) hist[tid] = 0;

  const uint8_t* aptr[1];
  if (wr_tiled) {
    const int rb = 32 * w < E ? w : 0;   // fragments past E compute fragment 0 (dropped)
    aptr[0] = reinterpret_cast<const uint8_t*>(wr) + static_cast<size_t>(rb) * (d / 64) * 4096 + 16 * l;
  } else {
    const int row = min(32 * w + r32, E - 1);
    aptr[0] = reinterpret_cast<const uint8_t*>(wr + static_cast<size_t>(row) * d + 32 * g);
  }
  f32x16 acc[1] = {f32x16{}};
  MainLoop<false, 3, BT>::template run<1>(aptr, x, t0, nullptr, 1, mvalid, d,
                                          wr_tiled ? 4096 : 64 * 2, wr_tiled ? 1024 : 16, bs0,
                                          bs1, bs2, bs3, acc);
  // acc[0][4i + j] = logit of expert 32w + 8i + 4g + j for token t0 + r32
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = 32 * w + 8 * i + 4 * g + j;
      if (e < E) lgs[r32][e] = acc[0][4 * i + j];
    }
  __syncthreads();

  for (int tt = w; tt < BT; tt += kThreads / kWave) {
    const int t = t0 + tt;
    if (t >= T) break;
    float lg[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = l + 64 * j;
      lg[j] = e < E ? lgs[tt][e] : 0.f;
    }
    topk_token(lg, t, E, K, G, M, score_fn, norm, bias, topk_idx, topk_gate, hist);
  }
  __syncthreads();
  if (tid < E && hist[tid] > 0) atomicAdd(&load[tid], hist[tid]);
}

// ---------------------------------------------------------------------------
// Split path, step 1 (bf16): partial logits over a slice of the hidden axis.
// Block = 16 tokens x 64 experts (one 16-expert fragment per wave); grid.z
// splits the 64-wide K stages evenly. Writes part[z][t][e] in fp32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void route_logits_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ wr, int T, int d, int E,
    int stages_per_split, float* __restrict__ part, int32_t* __restrict__ load) {
  const int l = lane_id(), w = wave_id(), g = l >> 4, r16 = l & 15;
  // the load counts the top-K kernel accumulates start from zero
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x < E) load[threadIdx.x] = 0;
  const int ef = blockIdx.y * 4 + w;
  if (16 * ef >= E) return;
  const int nk = d / 64;
  const int ks0 = blockIdx.z * stages_per_split;
  const int ks1 = min(nk, ks0 + stages_per_split);
  int er = 16 * ef + r16;
  er = er < E ? er : E - 1;
  int tr = blockIdx.x * 16 + r16;
  tr = tr < T ? tr : T - 1;
  const uint16_t* pa = wr + static_cast<size_t>(er) * d + 16 * g;
  const uint16_t* pb = x + static_cast<size_t>(tr) * d + 16 * g;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int ks = ks0; ks < ks1; ++ks) {
    const u32x4* qa = reinterpret_cast<const u32x4*>(pa + ks * 64);
    const u32x4* qb = reinterpret_cast<const u32x4*>(pb + ks * 64);
    const u32x4 a0 = qa[0], a1 = qa[1], b0 = qb[0], b1 = qb[1];
    acc = mfma_16x16x32(a0, b0, acc);
    acc = mfma_16x16x32(a1, b1, acc);
  }
  const int t = blockIdx.x * 16 + r16;
  if (t < T) {
    float* dst = part + (static_cast<size_t>(blockIdx.z) * T + t) * E;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 16 * ef + 4 * g + q;
      if (e < E) dst[e] = acc[q];
    }
  }
}

// Split path, step 1 (fp32): one thread per (token, expert), sequential fp32
// dot product over the hidden axis.
__global__ __launch_bounds__(256) void route_logits_f32(const float* __restrict__ x,
                                                        const float* __restrict__ wr, int T,
                                                        int d, int E, float* __restrict__ part,
                                                        int32_t* __restrict__ load) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  // the load counts the top-K kernel accumulates start from zero
  if (blockIdx.x == 0 && threadIdx.x < E) load[threadIdx.x] = 0;
  if (i >= static_cast<int64_t>(T) * E) return;
  const int t = static_cast<int>(i / E), e = static_cast<int>(i % E);
  const float* a = x + static_cast<size_t>(t) * d;
  const float* b = wr + static_cast<size_t>(e) * d;
  float acc = 0.f;
  for (int j = 0; j < d; ++j) acc = fmaf(a[j], b[j], acc);
  part[i] = acc;
}

// Split path, step 2: sum the K-splits in order, then score + top-K + gates
// (one wave per token) and the block's load histogram.
__global__ __launch_bounds__(256) void route_topk(const float* __restrict__ part, int splits,
                                                  const float* __restrict__ bias, int T, int E,
                                                  int K, int G, int M, int score_fn, int norm,
                                                  int32_t* __restrict__ topk_idx,
                                                  float* __restrict__ topk_gate,
                                                  int32_t* __restrict__ load) {
  __shared__ int hist[256];
  const int tid = threadIdx.x, l = lane_id();
  hist[tid] = 0;
  __syncthreads();
  const int t = blockIdx.x * 4 + wave_id();
  if (t < T) {
    // the splits are summed in order; the loads of 8 splits are issued
    // together (a split-serial loop would wait one memory latency per split)
    float lg[4] = {0.f, 0.f, 0.f, 0.f};
    const size_t zs = static_cast<size_t>(T) * E;
    const float* base = part + static_cast<size_t>(t) * E;
    for (int z0 = 0; z0 < splits; z0 += 8) {
      float v[8][4];
#pragma unroll
      for (int z = 0; z < 8; ++z)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = l + 64 * j;
          v[z][j] = (z0 + z < splits && e < E) ? base[(z0 + z) * zs + e] : 0.f;
        }
#pragma unroll
      for (int z = 0; z < 8; ++z)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (z0 + z < splits) lg[j] += v[z][j];
    }
    topk_token(lg, t, E, K, G, M, score_fn, norm, bias, topk_idx, topk_gate, hist);
  }
  __syncthreads();
  if (tid < E && hist[tid] > 0) atomicAdd(&load[tid], hist[tid]);
}

}  // namespace

bool route_uses_fused(const moe_config& c) {
  return c.act_dtype == MOE_DTYPE_BF16 && c.num_tokens >= kFusedMinTokens;
}

int route_k_splits(const moe_config& c) {
  if (route_uses_fused(c) || c.act_dtype == MOE_DTYPE_F32 || c.num_tokens == 0) return 1;
  const int nk = c.hidden / 64;
  const int64_t base = static_cast<int64_t>((c.num_tokens + 15) / 16) * ((c.num_experts + 63) / 64);
  int64_t want = (512 + base - 1) / base;
  if (want < 1) want = 1;
  if (want > nk) want = nk;
  // even split of the stages
  const int sps = static_cast<int>((nk + want - 1) / want);
  return (nk + sps - 1) / sps;
}

// The fused router reads a tiled copy of the router rows that it writes to
// the workspace on each call (E * d act elements, a pure relocation).
bool route_tiles_router(const moe_config& c) {
  return route_uses_fused(c) && c.num_experts % 32 == 0;
}

// Workspace of one call with exactly c.num_tokens tokens.
size_t route_ws_bytes_at(const moe_config& c) {
  if (route_tiles_router(c)) return align_up(static_cast<size_t>(c.num_experts) * c.hidden * 2, 256);
  if (route_uses_fused(c)) return 0;
  return align_up(static_cast<size_t>(route_k_splits(c)) * c.num_tokens * c.num_experts * 4, 256);
}

// The largest of route_ws_bytes_at over 1 .. c.num_tokens tokens, so that a
// workspace sized for a batch also serves every smaller one (the split-K
// partials do not grow monotonically with T, and the fused path below them
// needs a different amount).
size_t route_ws_bytes(const moe_config& c) {
  size_t m = route_ws_bytes_at(c);
  moe_config t = c;
  const int top = c.num_tokens < kFusedMinTokens ? c.num_tokens : kFusedMinTokens - 1;
  for (int n = 1; n <= top; ++n) {
    t.num_tokens = n;
    const size_t b = route_ws_bytes_at(t);
    if (b > m) m = b;
  }
  return m;
}

hipError_t launch_route(const moe_config& c, const void* x, const void* wr, const float* bias,
                        int32_t* topk_idx, float* topk_gate, int32_t* load, void* ws,
                        hipStream_t s) {
  hipError_t err;
  if (c.num_tokens == 0 || route_uses_fused(c)) {
    // (the split path's logits kernel clears the load counts itself)
    err = launch_fill_i32(load, 0, c.num_experts, s);
    if (err != hipSuccess || c.num_tokens == 0) return err;
  }
  const int T = c.num_tokens, d = c.hidden, E = c.num_experts, K = c.top_k;
  const int G = c.num_groups > 1 ? c.num_groups : 1;
  const int M = G > 1 ? c.topk_groups : 1;
  if (route_uses_fused(c)) {
    const int tiled = route_tiles_router(c);
    if (tiled) {
      err = launch_pack(1, 1, E, d, 2, wr, nullptr, ws, s);
      if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL(route_fused_bf16, dim3((T + kFusedTokens - 1) / kFusedTokens), dim3(kThreads),
                       0, s, static_cast<const uint16_t*>(x),
                       static_cast<const uint16_t*>(tiled ? ws : wr), tiled, bias, T, d, E, K, G, M,
                       c.score_fn, c.norm, topk_idx, topk_gate, load);
    return hipGetLastError();
  }
  float* part = static_cast<float*>(ws);
  int splits = 1;
  if (c.act_dtype == MOE_DTYPE_BF16) {
    splits = route_k_splits(c);
    const int nk = d / 64;
    const int sps = (nk + splits - 1) / splits;
    hipLaunchKernelGGL(route_logits_bf16, dim3((T + 15) / 16, (E + 63) / 64, splits), dim3(256),
                       0, s, static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(wr),
                       T, d, E, sps, part, load);
  } else {
    const int64_t n = static_cast<int64_t>(T) * E;
    hipLaunchKernelGGL(route_logits_f32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256),
                       0, s, static_cast<const float*>(x), static_cast<const float*>(wr), T, d, E,
                       part, load);
  }
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(route_topk, dim3((T + 3) / 4), dim3(256), 0, s, part, splits, bias, T, E, K,
                     G, M, c.score_fn, c.norm, topk_idx, topk_gate, load);
  return hipGetLastError();
}

}  // namespace moe
