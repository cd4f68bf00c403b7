// Dispatch of routed tokens to their experts without dropping any: a stable
// counting sort of the T*K (token, slot) pairs by expert id, then a gather of
// the token rows into expert-contiguous order for the grouped GEMMs.
//
// Method: no token is dropped and every (token, selected expert) pair is
// computed ("DeepSeekMoE架构解析" section 1; course notes "省钱第一招"
// section 六); the gather of selected expert work follows the section 3.1
// sketch of the same page.
//
// Kernels:
//   1. perm_hist   : per-chunk expert histogram (LDS atomics).
//   2. perm_scan   : one block; expert offsets (exclusive scan of the totals)
//                    and each chunk's starting row per expert.
//   3. perm_rank   : stable rank of every pair inside its expert. One wave
//                    takes 64 consecutive pairs; lanes with equal expert ids
//                    are matched with 8 ballots over the id bits, the rank is
//                    the popcount of matching lower lanes, and the group
//                    leader advances the expert's running row with one LDS
//                    atomic whose old value is broadcast back.
//   4. perm_gather : one wave per output row, 16-byte coalesced copies.
//   perm_single    : 1-3 in one block when T*K <= 4096 (decode batches).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kChunk = 4096;            // pairs per block in hist/rank
constexpr int kWaveChunk = kChunk / 4;  // pairs per wave in rank

__global__ __launch_bounds__(256) void perm_hist(const int32_t* __restrict__ idx, int64_t TK,
                                                 int E, int32_t* __restrict__ hist_out) {
  __shared__ int h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int64_t base = static_cast<int64_t>(blockIdx.x) * kChunk;
  for (int i = tid; i < kChunk; i += 256) {
    const int64_t f = base + i;
    if (f < TK) {
      const int e = idx[f];
      if (e >= 0 && e < E) atomicAdd(&h[e], 1);
    }
  }
  __syncthreads();
  if (tid < E) hist_out[static_cast<size_t>(blockIdx.x) * E + tid] = h[tid];
}

// hist[b][e] (counts) -> hist[b][e] = first row of chunk b's pairs of expert e.
__global__ __launch_bounds__(256) void perm_scan(int32_t* __restrict__ hist, int nblk, int E,
                                                 int64_t TK, int32_t* __restrict__ offsets,
                                                 int32_t* __restrict__ perm_slot) {
  __shared__ int tot[256];
  const int tid = threadIdx.x;
  int mine = 0;
  if (tid < E)
    for (int b = 0; b < nblk; ++b) mine += hist[static_cast<size_t>(b) * E + tid];
  tot[tid] = tid < E ? mine : 0;
  __syncthreads();
  // inclusive Hillis-Steele scan over 256 entries
  for (int o = 1; o < 256; o <<= 1) {
    const int v = tid >= o ? tot[tid - o] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  const int excl = tot[tid] - (tid < E ? mine : 0);
  if (tid < E) {
    offsets[tid] = excl;
    int run = excl;
    for (int b = 0; b < nblk; ++b) {
      int32_t* p = hist + static_cast<size_t>(b) * E + tid;
      const int c = *p;
      *p = run;
      run += c;
    }
  }
  const int total = tot[255];
  if (tid == 0) offsets[E] = total;
  // rows left over by out-of-range expert ids (never produced by moe_route)
  for (int64_t p = total + tid; p < TK; p += 256) perm_slot[p] = -1;
}

__global__ __launch_bounds__(256) void perm_rank(const int32_t* __restrict__ idx, int64_t TK,
                                                 int E, const int32_t* __restrict__ start,
                                                 int32_t* __restrict__ perm_slot) {
  __shared__ int cnt[4][256];
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  for (int i = tid; i < 4 * 256; i += 256) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int64_t wbase = static_cast<int64_t>(blockIdx.x) * kChunk + static_cast<int64_t>(w) * kWaveChunk;
  // per-wave histogram of its sub-chunk
  for (int i = l; i < kWaveChunk; i += kWave) {
    const int64_t f = wbase + i;
    if (f < TK) {
      const int e = idx[f];
      if (e >= 0 && e < E) atomicAdd(&cnt[w][e], 1);
    }
  }
  __syncthreads();
  // running row per (wave, expert): chunk start + earlier waves' counts
  if (tid < E) {
    int run = start[static_cast<size_t>(blockIdx.x) * E + tid];
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const int c = cnt[ww][tid];
      cnt[ww][tid] = run;
      run += c;
    }
  }
  __syncthreads();
  for (int it = 0; it < kWaveChunk; it += kWave) {
    const int64_t f = wbase + it + l;
    int e = -1;
    if (f < TK) {
      e = idx[f];
      if (e < 0 || e >= E) e = -1;
    }
    const bool part = e >= 0;
    uint64_t peers = __ballot(part);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t m = __ballot((e >> b) & 1);
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    const int leader = part ? __ffsll(static_cast<long long>(peers)) - 1 : l;
    int old = 0;
    if (part && l == leader) old = atomicAdd(&cnt[w][e], __popcll(peers));
    // every lane takes part in the shuffle; each reads its group leader
    old = __shfl(old, leader, kWave);
    if (part) {
      const int64_t p = static_cast<int64_t>(old) + __popcll(peers & lanemask_lt());
      if (p >= 0 && p < TK) perm_slot[p] = static_cast<int32_t>(f);
    }
  }
}

// All of 1-3 in one block, for T*K <= kChunk (decode-sized batches): the
// per-wave counts give the expert totals, their exclusive scan the offsets,
// and the same ranking pass as perm_rank places every pair. One launch in
// place of three; the result is the same stable order. The pairs are split
// evenly over the four waves (in order: wave w takes the w-th quarter, whole
// 64-pair groups), so a small batch keeps every wave busy.
__global__ __launch_bounds__(256) void perm_single(const int32_t* __restrict__ idx, int64_t TK,
                                                   int E, int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ perm_slot) {
  __shared__ int cnt[4][256];
  __shared__ int tot[256];
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  for (int i = tid; i < 4 * 256; i += 256) (&cnt[0][0])[i] = 0;
  __syncthreads();
  const int wchunk = static_cast<int>((TK + 4 * kWave - 1) / (4 * kWave)) * kWave;   // <= kWaveChunk
  const int64_t wbase = static_cast<int64_t>(w) * wchunk;
  for (int i = l; i < wchunk; i += kWave) {
    const int64_t f = wbase + i;
    if (f < TK) {
      const int e = idx[f];
      if (e >= 0 && e < E) atomicAdd(&cnt[w][e], 1);
    }
  }
  __syncthreads();
  const int mine = tid < E ? cnt[0][tid] + cnt[1][tid] + cnt[2][tid] + cnt[3][tid] : 0;
  tot[tid] = mine;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {   // inclusive Hillis-Steele scan
    const int v = tid >= o ? tot[tid - o] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    int run = tot[tid] - mine;
    offsets[tid] = run;
#pragma unroll
    for (int ww = 0; ww < 4; ++ww) {
      const int c = cnt[ww][tid];
      cnt[ww][tid] = run;
      run += c;
    }
  }
  const int total = tot[255];
  if (tid == 0) offsets[E] = total;
  for (int64_t p = total + tid; p < TK; p += 256) perm_slot[p] = -1;
  __syncthreads();
  for (int it = 0; it < wchunk; it += kWave) {
    const int64_t f = wbase + it + l;
    int e = -1;
    if (f < TK) {
      e = idx[f];
      if (e < 0 || e >= E) e = -1;
    }
    const bool part = e >= 0;
    uint64_t peers = __ballot(part);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const uint64_t m = __ballot((e >> b) & 1);
      peers &= ((e >> b) & 1) ? m : ~m;
    }
    const int leader = part ? __ffsll(static_cast<long long>(peers)) - 1 : l;
    int old = 0;
    if (part && l == leader) old = atomicAdd(&cnt[w][e], __popcll(peers));
    old = __shfl(old, leader, kWave);
    if (part) {
      const int64_t p = static_cast<int64_t>(old) + __popcll(peers & lanemask_lt());
      if (p >= 0 && p < TK) perm_slot[p] = static_cast<int32_t>(f);
    }
  }
}

__global__ __launch_bounds__(256) void perm_gather(const uint8_t* __restrict__ x,
                                                   const int32_t* __restrict__ perm_slot,
                                                   int64_t TK, int T, int K, int row_bytes,
                                                   uint8_t* __restrict__ xp) {
  const int64_t p = static_cast<int64_t>(blockIdx.x) * 4 + wave_id();
  if (p >= TK) return;
  const int f = perm_slot[p];
  const int t = f >= 0 ? f / K : -1;
  u32x4* dst = reinterpret_cast<u32x4*>(xp + static_cast<size_t>(p) * row_bytes);
  const int nvec = row_bytes / 16;
  if (t >= 0 && t < T) {
    const u32x4* src = reinterpret_cast<const u32x4*>(x + static_cast<size_t>(t) * row_bytes);
    for (int v = lane_id(); v < nvec; v += kWave) dst[v] = src[v];
  } else {
    for (int v = lane_id(); v < nvec; v += kWave) dst[v] = u32x4{0u, 0u, 0u, 0u};
  }
}

// Per-sequence expert histogram: block q counts the ids of tokens
// q*L .. min(T, (q+1)*L) - 1.
__global__ __launch_bounds__(256) void seq_hist(const int32_t* __restrict__ idx, int T, int K,
                                                int E, int L, int32_t* __restrict__ out) {
  __shared__ int h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int64_t q = blockIdx.x;
  const int64_t f0 = q * L * K;
  const int64_t f1 = (q + 1) * L < T ? (q + 1) * L * K : static_cast<int64_t>(T) * K;
  for (int64_t f = f0 + tid; f < f1; f += 256) {
    const int e = idx[f];
    if (e >= 0 && e < E) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  if (tid < E) out[q * E + tid] = h[tid];
}

}  // namespace

hipError_t launch_sequence_loads(const moe_config& c, const int32_t* topk_idx, int seq_len,
                                 int32_t* seq_load, hipStream_t s) {
  const int T = c.num_tokens;
  if (T == 0) return hipSuccess;
  const int64_t nq = (static_cast<int64_t>(T) + seq_len - 1) / seq_len;
  hipLaunchKernelGGL(seq_hist, dim3(static_cast<unsigned>(nq)), dim3(256), 0, s, topk_idx, T,
                     c.top_k, c.num_experts, seq_len, seq_load);
  return hipGetLastError();
}

size_t permute_ws_bytes(const moe_config& c) {
  const int64_t TK = static_cast<int64_t>(c.num_tokens) * c.top_k;
  const int64_t nblk = (TK + kChunk - 1) / kChunk;
  return align_up(static_cast<size_t>(nblk > 0 ? nblk : 1) * c.num_experts * 4, 256);
}

hipError_t launch_permute(const moe_config& c, const int32_t* topk_idx, const void* x,
                          int32_t* expert_offsets, int32_t* perm_slot, void* x_perm, void* ws,
                          hipStream_t s) {
  const int E = c.num_experts;
  const int64_t TK = static_cast<int64_t>(c.num_tokens) * c.top_k;
  const int nblk = static_cast<int>((TK + kChunk - 1) / kChunk);
  int32_t* hist = static_cast<int32_t*>(ws);
  if (TK == 0) {
    return launch_fill_i32(expert_offsets, 0, E + 1, s);
  }
  hipError_t err;
  if (nblk == 1) {
    hipLaunchKernelGGL(perm_single, dim3(1), dim3(256), 0, s, topk_idx, TK, E, expert_offsets,
                       perm_slot);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  } else {
    hipLaunchKernelGGL(perm_hist, dim3(nblk), dim3(256), 0, s, topk_idx, TK, E, hist);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(perm_scan, dim3(1), dim3(256), 0, s, hist, nblk, E, TK, expert_offsets,
                       perm_slot);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL(perm_rank, dim3(nblk), dim3(256), 0, s, topk_idx, TK, E, hist, perm_slot);
    if ((err = hipGetLastError()) != hipSuccess) return err;
  }
  if (!x_perm) return hipSuccess;   // the caller reads x through perm_slot itself
  const int elem = c.act_dtype == MOE_DTYPE_F32 ? 4 : 2;
  const int row_bytes = c.hidden * elem;
  hipLaunchKernelGGL(perm_gather, dim3(static_cast<unsigned>((TK + 3) / 4)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(x), perm_slot, TK, c.num_tokens, c.top_k,
                     row_bytes, static_cast<uint8_t*>(x_perm));
  return hipGetLastError();
}

}  // namespace moe
