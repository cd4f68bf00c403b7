// Device-side building blocks shared by the libmoe kernels (gfx950 / CDNA4).
//
// Conventions used throughout:
//  * Waves are 64 lanes; blocks are 256 threads (4 waves) unless noted.
//  * MFMA: the expert GEMMs and the fused router use
//    v_mfma_f32_32x32x16_bf16 (mfma_32x32x16 below), the fine-grained fp8
//    GEMMs v_mfma_scale_f32_32x32x64_f8f6f4 (mfma_32x32x64_fp8), the split-K
//    router logits v_mfma_f32_16x16x32_bf16 (mfma_16x16x32); each wrapper
//    states its lane layout.
//  * GEMMs are written in the "weights as rows" orientation: the first MFMA
//    operand is a block of weight rows (output features), the second a block
//    of token rows, so one lane ends up holding 4 consecutive output features
//    of one token and can store them as one 8-byte vector.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
}

// v_mfma_f32_16x16x32_bf16: lane l supplies 8 consecutive K-elements of row
// (l % 16) of the first operand and of column (l % 16) of the second (lane
// group g = l / 16 owns K-elements 8g .. 8g+7); the 16x16 fp32 result
// leaves rows 4g .. 4g+3 of column (l % 16) in lane l.
__device__ __forceinline__ f32x4 mfma_16x16x32(const u32x4& a, const u32x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: lane l supplies 8 consecutive K-elements of row
// (l % 32) of the first operand and of column (l % 32) of the second (lane
// group g = l / 32 owns K-elements 8g .. 8g+7); the 32x32 fp32 result leaves
// rows 8i + 4g + j (i, j = 0..3) of column (l % 32) in element 4i + j.
__device__ __forceinline__ f32x16 mfma_32x32x16(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                  __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 codes with unit block scales
// (E8M0 exponent 127 = 1.0): lane l supplies 32 codes of row (l % 32) of
// the first operand (a0 = the first 16, a1 the next) and the matching 32 of
// column (l % 32) of the second; the result layout is that of
// mfma_32x32x16. The instruction pairs the k-th code a lane supplies for A
// with the k-th code the lane of the same half supplies for B, so any K
// order that both operands share gives the same sum.
__device__ __forceinline__ f32x16 mfma_32x32x64_fp8(const u32x4& a0, const u32x4& a1,
                                                    const u32x4& b0, const u32x4& b1,
                                                    const f32x16& c) {
  typedef int i32x8 __attribute__((ext_vector_type(8)));
  const i32x8 a = {static_cast<int>(a0.x), static_cast<int>(a0.y), static_cast<int>(a0.z),
                   static_cast<int>(a0.w), static_cast<int>(a1.x), static_cast<int>(a1.y),
                   static_cast<int>(a1.z), static_cast<int>(a1.w)};
  const i32x8 b = {static_cast<int>(b0.x), static_cast<int>(b0.y), static_cast<int>(b0.z),
                   static_cast<int>(b0.w), static_cast<int>(b1.x), static_cast<int>(b1.y),
                   static_cast<int>(b1.z), static_cast<int>(b1.w)};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// fp32 -> OCP E4M3FN code, round to nearest even, for finite |v| <= 448
// (larger magnitudes saturate to 448). Normal range: round the fp32
// significand to 3 fraction bits (add-and-truncate at bit 20, whose carry
// into the exponent is the correct result) and rebias the exponent from 127
// to 7; below 2^-6 the value is a multiple of the subnormal step 2^-9,
// rounded with rintf (ties to even) after an exact scaling by 2^9.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t sign = (b >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a >= 0.015625f) {                                  // 2^-6
    uint32_t m = b & 0x7FFFFFFFu;
    m += 0x7FFFFu + ((m >> 20) & 1u);
    const int e = static_cast<int>(m >> 23) - 127 + 7;
    code = (static_cast<uint32_t>(e) << 3) | ((m >> 20) & 7u);
    code = e > 15 || code > 0x7Eu ? 0x7Eu : code;
  } else {
    code = static_cast<uint32_t>(rintf(a * 512.0f));     // 0 .. 8 (8 = 2^-6, code 0x08)
  }
  return sign | code;
}

// 4 fp8 E4M3 codes (one dword) -> 4 bf16 (two dwords). Every E4M3 value is
// exactly representable in bf16, so the conversion is lossless.
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(uint32_t q) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, false);
  bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q, 1.0f, true);
  u32x2 r;
  r.x = __builtin_bit_cast(uint32_t, lo);
  r.y = __builtin_bit_cast(uint32_t, hi);
  return r;
}

// 16 fp8 codes -> two MFMA operands of 8 bf16 each (codes 0..7, 8..15).
__device__ __forceinline__ void fp8x16_to_bf16x16(const u32x4& q, u32x4& a0, u32x4& a1) {
  u32x2 p0 = fp8x4_to_bf16x4(q.x), p1 = fp8x4_to_bf16x4(q.y);
  u32x2 p2 = fp8x4_to_bf16x4(q.z), p3 = fp8x4_to_bf16x4(q.w);
  a0 = u32x4{p0.x, p0.y, p1.x, p1.y};
  a1 = u32x4{p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// SiLU with the hardware exp2 and reciprocal (about 1e-6 relative error, far
// below the bf16 rounding of the value it feeds).
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + expf(-z)); }

template <typename T>
__device__ __forceinline__ T load_nt(const T* p) { return *p; }

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// Wave-wide reductions with a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Lanes below the calling lane, as a 64-bit mask.
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

// Blocks are dispatched round-robin over the 8 XCDs (each with its own L2).
// Remap a block id so that XCD x receives a contiguous range of work items,
// which keeps the tiles that share a weight block on one L2.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int xcd_contiguous(int bid, int total, bool& valid) {
  const int per = (total + kNumXcd - 1) / kNumXcd;
  const int xcd = bid % kNumXcd, slot = bid / kNumXcd;
  const int item = xcd * per + slot;
  valid = slot < per && item < total;
  return item;
}

}  // namespace moe
