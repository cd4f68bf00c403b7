// Achievable-peak probes (include/moe_peaks.h): MFMA and FMA issue loops and
// streaming read / copy kernels, for MI355X (gfx950). They measure what the
// part sustains, the denominator beside its published peaks; nothing here
// computes any part of the MoE layer.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "common.hpp"
#include "libmoe.h"
#include "moe_peaks.h"

namespace moe {
namespace {

constexpr int kLoopThreads = 512;   // 8 waves, two per SIMD, as the expert GEMMs
constexpr int kStreamThreads = 256;

template <int N, int I = 0, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    unroll<N, I + 1>(f);
  }
}

// 32-bit integer mixer (xorshift-multiply), used only to give the operands
// varied bit patterns.
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7FEB352Du;
  x ^= x >> 15;
  x *= 0x846CA68Bu;
  x ^= x >> 16;
  return x;
}

// Four dwords of operand bits: bf16 values of magnitude [2^-7, 2^-6) with
// random sign and mantissa, or E4M3 codes of magnitude [0.5, 1) (exponent
// field 6: never NaN).
template <bool FP8>
__device__ __forceinline__ u32x4 operand(uint32_t& s) {
  const uint32_t mask = FP8 ? 0x87878787u : 0x807F807Fu;
  const uint32_t bias = FP8 ? 0x30303030u : 0x3C003C00u;
  u32x4 v;
  s = mix32(s + 0x9E3779B9u); v.x = (s & mask) | bias;
  s = mix32(s + 0x9E3779B9u); v.y = (s & mask) | bias;
  s = mix32(s + 0x9E3779B9u); v.z = (s & mask) | bias;
  s = mix32(s + 0x9E3779B9u); v.w = (s & mask) | bias;
  return v;
}

__device__ __forceinline__ f32x4 mfma_16x16x128_fp8(const u32x4& a0, const u32x4& a1,
                                                    const u32x4& b0, const u32x4& b1,
                                                    const f32x4& c) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a = {static_cast<int>(a0.x), static_cast<int>(a0.y), static_cast<int>(a0.z),
                   static_cast<int>(a0.w), static_cast<int>(a1.x), static_cast<int>(a1.y),
                   static_cast<int>(a1.z), static_cast<int>(a1.w)};
  const i32x8 b = {static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z),
                   static_cast<int>(b0.w), static_cast<int>(b1.x), static_cast<int>(b1.y),
                   static_cast<int>(b1.z), static_cast<int>(b1.w)};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Instructions one wave issues per loop iteration, and flops per instruction.
template <int KIND> struct Form;
template <> struct Form<MOE_PEAK_MFMA_BF16_32X32X16> { static constexpr int chains = 4, per_iter = 16; static constexpr double flops = 32.0 * 32 * 16 * 2; };
template <> struct Form<MOE_PEAK_MFMA_BF16_16X16X32> { static constexpr int chains = 8, per_iter = 32; static constexpr double flops = 16.0 * 16 * 32 * 2; };
template <> struct Form<MOE_PEAK_MFMA_FP8_32X32X64>  { static constexpr int chains = 4, per_iter = 16; static constexpr double flops = 32.0 * 32 * 64 * 2; };
template <> struct Form<MOE_PEAK_MFMA_FP8_16X16X128> { static constexpr int chains = 8, per_iter = 32; static constexpr double flops = 16.0 * 16 * 128 * 2; };
template <> struct Form<MOE_PEAK_FMA_F32>            { static constexpr int chains = 8, per_iter = 32; static constexpr double flops = 64.0 * 2; };

// Each iteration: 4 rounds; in round u chain c takes operand registers
// (c + u) % 4 and (c + 2u + 1) % 4, so consecutive instructions see
// different bits. Chains are independent, which keeps the pipe full.
template <int KIND>
__global__ __launch_bounds__(kLoopThreads) void mfma_loop(int iters, float* __restrict__ out) {
  constexpr bool FP8 = KIND == MOE_PEAK_MFMA_FP8_32X32X64 || KIND == MOE_PEAK_MFMA_FP8_16X16X128;
  constexpr int C = Form<KIND>::chains;
  const int gid = blockIdx.x * kLoopThreads + threadIdx.x;
  uint32_t s = mix32(static_cast<uint32_t>(gid) * 0x85EBCA6Bu + 0x165667B1u);
  float total = 0.f;
  if constexpr (KIND == MOE_PEAK_FMA_F32) {
    float v[C];
    for (int c = 0; c < C; ++c) v[c] = static_cast<float>(mix32(s + c) & 0xFFFF) * 1e-5f;
    const float a = 0.9990234375f, b[4] = {1e-3f, -2e-3f, 3e-3f, -1e-3f};
    for (int it = 0; it < iters; ++it) {
      unroll<4>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        unroll<C>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          v[c] = fmaf(v[c], a, b[(c + u) & 3]);
        });
      });
    }
    for (int c = 0; c < C; ++c) total += v[c];
  } else {
    u32x4 A[4], B[4];
    for (int i = 0; i < 4; ++i) {
      A[i] = operand<FP8>(s);
      B[i] = operand<FP8>(s);
    }
    if constexpr (KIND == MOE_PEAK_MFMA_BF16_32X32X16 || KIND == MOE_PEAK_MFMA_FP8_32X32X64) {
      f32x16 acc[C];
      for (int c = 0; c < C; ++c) acc[c] = f32x16{};
      for (int it = 0; it < iters; ++it) {
        unroll<4>([&](auto uc) {
          constexpr int u = decltype(uc)::value;
          unroll<C>([&](auto cc) {
            constexpr int c = decltype(cc)::value, ia = (c + u) & 3, ib = (c + 2 * u + 1) & 3;
            if constexpr (FP8)
              acc[c] = mfma_32x32x64_fp8(A[ia], A[(ia + 1) & 3], B[ib], B[(ib + 1) & 3], acc[c]);
            else
              acc[c] = mfma_32x32x16(A[ia], B[ib], acc[c]);
          });
        });
      }
      for (int c = 0; c < C; ++c)
        for (int e = 0; e < 16; ++e) total += acc[c][e];
    } else {
      f32x4 acc[C];
      for (int c = 0; c < C; ++c) acc[c] = f32x4{};
      for (int it = 0; it < iters; ++it) {
        unroll<4>([&](auto uc) {
          constexpr int u = decltype(uc)::value;
          unroll<C>([&](auto cc) {
            constexpr int c = decltype(cc)::value, ia = (c + u) & 3, ib = (c + 2 * u + 1) & 3;
            if constexpr (FP8)
              acc[c] = mfma_16x16x128_fp8(A[ia], A[(ia + 1) & 3], B[ib], B[(ib + 1) & 3], acc[c]);
            else
              acc[c] = mfma_16x16x32(A[ia], B[ib], acc[c]);
          });
        });
      }
      for (int c = 0; c < C; ++c)
        for (int e = 0; e < 4; ++e) total += acc[c][e];
    }
  }
  out[gid] = total;
}

// Streaming kernels: the buffer is cut into chunks of kChunk16 16-byte
// words (32 KB), dealt to blocks grid-stride; in a chunk, thread t moves
// words u * 256 + t for u = 0 .. 7, all eight loads issued before any use.
constexpr int kUnroll = 8;
constexpr size_t kChunk16 = static_cast<size_t>(kStreamThreads) * kUnroll;

// NT: the loads carry the non-temporal hint (the form the decode GEMMs use
// for their weights).
template <bool NT>
__global__ __launch_bounds__(kStreamThreads) void stream_read(const u32x4* __restrict__ src,
                                                             size_t n16, uint32_t* __restrict__ out) {
  auto ld = [&](size_t i) { return NT ? __builtin_nontemporal_load(src + i) : src[i]; };
  const size_t nchunks = (n16 + kChunk16 - 1) / kChunk16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const size_t base = c * kChunk16 + threadIdx.x;
    if ((c + 1) * kChunk16 <= n16) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = ld(base + u * kStreamThreads);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    } else {
      for (int u = 0; u < kUnroll; ++u)
        if (base + u * kStreamThreads < n16) acc ^= ld(base + u * kStreamThreads);
    }
  }
  out[static_cast<size_t>(blockIdx.x) * kStreamThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

__global__ __launch_bounds__(kStreamThreads) void stream_copy(const u32x4* __restrict__ src,
                                                             u32x4* __restrict__ dst, size_t n16) {
  const size_t nchunks = (n16 + kChunk16 - 1) / kChunk16;
  for (size_t c = blockIdx.x; c < nchunks; c += gridDim.x) {
    const size_t base = c * kChunk16 + threadIdx.x;
    if ((c + 1) * kChunk16 <= n16) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = src[base + u * kStreamThreads];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) dst[base + u * kStreamThreads] = v[u];
    } else {
      for (int u = 0; u < kUnroll; ++u)
        if (base + u * kStreamThreads < n16) dst[base + u * kStreamThreads] = src[base + u * kStreamThreads];
    }
  }
}

// L2 probe: block b sweeps its region (region16 words, a multiple of
// 8 * 512) `iters` times, 512 threads, eight 16-byte loads per thread per step.
__global__ __launch_bounds__(kLoopThreads) void l2_read(const u32x4* __restrict__ src,
                                                       size_t region16, int iters,
                                                       uint32_t* __restrict__ out) {
  const u32x4* base = src + static_cast<size_t>(blockIdx.x) * region16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it) {
    for (size_t i = threadIdx.x; i < region16; i += kUnroll * kLoopThreads) {
      u32x4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) v[u] = base[i + u * kLoopThreads];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
    }
  }
  out[static_cast<size_t>(blockIdx.x) * kLoopThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

template <int KIND>
double flops_of(int32_t blocks, int32_t iters) {
  return static_cast<double>(blocks) * (kLoopThreads / kWave) * iters * Form<KIND>::per_iter *
         Form<KIND>::flops;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// One v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, unit scales) per
// wave: problem p reads A [32 rows][64] and B [32 columns][64] codes and
// C [32][32] fp32 at its own offsets and writes D = A B^T + C. Lane l
// supplies row / column l % 32, codes 32 (l / 32) .. +31 of each (the
// layout of mfma_32x32x64_fp8); the result element 4i + j of lane l is
// D[8i + 4(l / 32) + j][l % 32].
__global__ __launch_bounds__(64) void fp8_mfma_once(const uint8_t* __restrict__ a,
                                                    const uint8_t* __restrict__ b,
                                                    const float* __restrict__ c,
                                                    float* __restrict__ d) {
  const int l = threadIdx.x, g = l >> 5, r = l & 31;
  const size_t p = blockIdx.x;
  const uint8_t* ap = a + p * 2048 + r * 64 + 32 * g;
  const uint8_t* bp = b + p * 2048 + r * 64 + 32 * g;
  const u32x4 a0 = *reinterpret_cast<const u32x4*>(ap), a1 = *reinterpret_cast<const u32x4*>(ap + 16);
  const u32x4 b0 = *reinterpret_cast<const u32x4*>(bp), b1 = *reinterpret_cast<const u32x4*>(bp + 16);
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[4 * i + j] = c[p * 1024 + (8 * i + 4 * g + j) * 32 + r];
  acc = mfma_32x32x64_fp8(a0, a1, b0, b1, acc);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) d[p * 1024 + (8 * i + 4 * g + j) * 32 + r] = acc[4 * i + j];
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

double moe_peak_mfma_flops(int kind, int32_t blocks, int32_t iters) {
  if (blocks < 1 || iters < 1) return 0.0;
  switch (kind) {
    case MOE_PEAK_MFMA_BF16_32X32X16: return flops_of<MOE_PEAK_MFMA_BF16_32X32X16>(blocks, iters);
    case MOE_PEAK_MFMA_BF16_16X16X32: return flops_of<MOE_PEAK_MFMA_BF16_16X16X32>(blocks, iters);
    case MOE_PEAK_MFMA_FP8_32X32X64: return flops_of<MOE_PEAK_MFMA_FP8_32X32X64>(blocks, iters);
    case MOE_PEAK_MFMA_FP8_16X16X128: return flops_of<MOE_PEAK_MFMA_FP8_16X16X128>(blocks, iters);
    case MOE_PEAK_FMA_F32: return flops_of<MOE_PEAK_FMA_F32>(blocks, iters);
    default: return 0.0;
  }
}

int moe_peak_mfma(int kind, int32_t blocks, int32_t iters, float* out, void* stream) {
  if (moe_peak_mfma_flops(kind, blocks, iters) == 0.0) return MOE_ERR_SHAPE;
  if (!out) return MOE_ERR_NULL;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(blocks)), block(kLoopThreads);
  switch (kind) {
    case MOE_PEAK_MFMA_BF16_32X32X16: hipLaunchKernelGGL(mfma_loop<MOE_PEAK_MFMA_BF16_32X32X16>, grid, block, 0, s, iters, out); break;
    case MOE_PEAK_MFMA_BF16_16X16X32: hipLaunchKernelGGL(mfma_loop<MOE_PEAK_MFMA_BF16_16X16X32>, grid, block, 0, s, iters, out); break;
    case MOE_PEAK_MFMA_FP8_32X32X64: hipLaunchKernelGGL(mfma_loop<MOE_PEAK_MFMA_FP8_32X32X64>, grid, block, 0, s, iters, out); break;
    case MOE_PEAK_MFMA_FP8_16X16X128: hipLaunchKernelGGL(mfma_loop<MOE_PEAK_MFMA_FP8_16X16X128>, grid, block, 0, s, iters, out); break;
    default: hipLaunchKernelGGL(mfma_loop<MOE_PEAK_FMA_F32>, grid, block, 0, s, iters, out); break;
  }
  return status_of(hipGetLastError());
}

int moe_peak_stream_read(const void* src, size_t bytes, int32_t blocks, uint32_t* out,
                         void* stream) {
  if (!src || !out) return MOE_ERR_NULL;
  if (blocks < 1 || bytes == 0 || bytes % 16 != 0 || !aligned16(src)) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(stream_read<false>, dim3(static_cast<unsigned>(blocks)), dim3(kStreamThreads),
                     0, reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     bytes / 16, out);
  return status_of(hipGetLastError());
}

int moe_peak_stream_read_nt(const void* src, size_t bytes, int32_t blocks, uint32_t* out,
                            void* stream) {
  if (!src || !out) return MOE_ERR_NULL;
  if (blocks < 1 || bytes == 0 || bytes % 16 != 0 || !aligned16(src)) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(stream_read<true>, dim3(static_cast<unsigned>(blocks)), dim3(kStreamThreads),
                     0, reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     bytes / 16, out);
  return status_of(hipGetLastError());
}

int moe_peak_l2_read(const void* src, size_t region_bytes, int32_t blocks, int32_t iters,
                     uint32_t* out, void* stream) {
  if (!src || !out) return MOE_ERR_NULL;
  if (blocks < 1 || iters < 1 || region_bytes == 0 || region_bytes % 65536 != 0 || !aligned16(src))
    return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(l2_read, dim3(static_cast<unsigned>(blocks)), dim3(kLoopThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     region_bytes / 16, iters, out);
  return status_of(hipGetLastError());
}

int moe_peak_stream_copy(const void* src, void* dst, size_t bytes, int32_t blocks, void* stream) {
  if (!src || !dst) return MOE_ERR_NULL;
  if (blocks < 1 || bytes == 0 || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst))
    return MOE_ERR_SHAPE;
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (a < b + bytes && b < a + bytes) return MOE_ERR_SHAPE;     // overlapping ranges
  hipLaunchKernelGGL(stream_copy, dim3(static_cast<unsigned>(blocks)), dim3(kStreamThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(src),
                     static_cast<u32x4*>(dst), bytes / 16);
  return status_of(hipGetLastError());
}

int moe_probe_fp8_mfma(const void* a, const void* b, const float* c, float* d, int32_t n,
                       void* stream) {
  if (!a || !b || !c || !d) return MOE_ERR_NULL;
  if (n < 1 || !aligned16(a) || !aligned16(b)) return MOE_ERR_SHAPE;
  hipLaunchKernelGGL(fp8_mfma_once, dim3(static_cast<unsigned>(n)), dim3(64), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const uint8_t*>(a),
                     static_cast<const uint8_t*>(b), c, d);
  return status_of(hipGetLastError());
}

}  // extern "C"
