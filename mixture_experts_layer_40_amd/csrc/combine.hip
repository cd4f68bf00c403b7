// Layer output combine and the auxiliary-loss-free bias update.
//
// Combine: y_t = shared(x_t) + sum_k g_{t,k} E_{k}(x_t) -- the always-on
// shared expert plus the gate-weighted routed experts ("DeepSeekMoE架构解析"
// section 1 and the weighted sum of its section 3.1 sketch; no residual).
// The gate has already been applied per (token, slot) by the down-projection
// epilogue; here the K slot rows and the shared row are summed in fp32 in a
// fixed order, so the result is deterministic.
//
// Bias update: section 2.2 of the same page -- after each batch an
// overloaded expert's bias drops by gamma and an underloaded one's rises by
// gamma (course notes "省钱第一招" section 五: outside the gradient).
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

// One thread per 8 consecutive features of one token: out_slots in the slot
// dtype, the residual in the activation dtype, y_shared fp32, y in the
// output dtype.
template <bool SLOT_BF16, bool RES_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ slots,
                                                      const float* __restrict__ ysh,
                                                      const void* __restrict__ res, int T, int K,
                                                      int d, void* __restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int vpr = d / 8;
  if (i >= static_cast<int64_t>(T) * vpr) return;
  const int64_t t = i / vpr;
  const int c = static_cast<int>(i % vpr) * 8;
  float acc[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) acc[q] = 0.f;
  if (res) {     // the residual stream (layer input), in the activation dtype
    if (RES_BF16) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(res) + t * d + c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] = bf16_to_f32(static_cast<uint16_t>(v[q] & 0xFFFFu));
        acc[2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(v[q] >> 16));
      }
    } else {
      const float* rp = static_cast<const float*>(res) + t * d + c;
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(rp);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(rp + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) { acc[q] = v0[q]; acc[4 + q] = v1[q]; }
    }
  }
  if (ysh) {
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(ysh + t * d + c);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(ysh + t * d + c + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      acc[q] = res ? acc[q] + v0[q] : v0[q];
      acc[4 + q] = res ? acc[4 + q] + v1[q] : v1[q];
    }
  }
  for (int k = 0; k < K; ++k) {
    const int64_t o = (t * K + k) * d + c;
    if (SLOT_BF16) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(slots) + o);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc[2 * q] += bf16_to_f32(static_cast<uint16_t>(v[q] & 0xFFFFu));
        acc[2 * q + 1] += bf16_to_f32(static_cast<uint16_t>(v[q] >> 16));
      }
    } else {
      const float* sp = static_cast<const float*>(slots) + o;
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(sp);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(sp + 4);
#pragma unroll
      for (int q = 0; q < 4; ++q) { acc[q] += v0[q]; acc[4 + q] += v1[q]; }
    }
  }
  if (OUT_BF16) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + t * d + c) = o;
  } else {
    float* yp = static_cast<float*>(y) + t * d + c;
    *reinterpret_cast<f32x4*>(yp) = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *reinterpret_cast<f32x4*>(yp + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

__global__ __launch_bounds__(256) void bias_update_kernel(const int32_t* __restrict__ load, int E,
                                                          float gamma, float* __restrict__ bias) {
  __shared__ long long tot[256];
  const int tid = threadIdx.x;
  const long long mine = tid < E ? static_cast<long long>(load[tid]) : 0;
  tot[tid] = mine;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (tid < o) tot[tid] += tot[tid + o];
    __syncthreads();
  }
  if (tid < E) {
    const long long diff = mine * E - tot[0];  // sign(load_i - mean), decided in integers
    const float b = bias[tid];
    bias[tid] = diff > 0 ? __fsub_rn(b, gamma) : (diff < 0 ? __fadd_rn(b, gamma) : b);
  }
}

__global__ void fill_i32(int32_t* p, int32_t v, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_combine(const moe_config& c, const void* out_slots, const void* y_shared,
                          const void* residual, void* y, hipStream_t s) {
  const int T = c.num_tokens, K = c.top_k, d = c.hidden;
  if (T == 0) return hipSuccess;
  const int64_t n = static_cast<int64_t>(T) * (d / 8);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256)), block(256);
  const float* ysh = static_cast<const float*>(y_shared);
  // fp32 activations come with fp32 slots and an fp32 output (moe_validate)
  const bool sb = c.slot_dtype == MOE_DTYPE_BF16, ab = c.act_dtype == MOE_DTYPE_BF16;
  const bool ob = c.out_dtype == MOE_DTYPE_BF16;
  if (!ab) hipLaunchKernelGGL((combine_kernel<false, false, false>), grid, block, 0, s, out_slots, ysh, residual, T, K, d, y);
  else if (sb && ob) hipLaunchKernelGGL((combine_kernel<true, true, true>), grid, block, 0, s, out_slots, ysh, residual, T, K, d, y);
  else if (sb) hipLaunchKernelGGL((combine_kernel<true, true, false>), grid, block, 0, s, out_slots, ysh, residual, T, K, d, y);
  else if (ob) hipLaunchKernelGGL((combine_kernel<false, true, true>), grid, block, 0, s, out_slots, ysh, residual, T, K, d, y);
  else hipLaunchKernelGGL((combine_kernel<false, true, false>), grid, block, 0, s, out_slots, ysh, residual, T, K, d, y);
  return hipGetLastError();
}

// Round a double to the nearest bf16 (ties to even) without double rounding:
// first to fp32 with round-to-odd (truncate, then set the last bit when
// anything was cut off), then fp32 -> bf16 to nearest even. Rounding to odd
// at a precision of at least two more bits than the target (fp32 keeps 24,
// bf16 8, over the same exponent range) followed by rounding to nearest
// gives the single correctly rounded result (Boldo and Melquiond, "Emulation
// of FMA and correctly rounded sums: proved algorithms using rounding to
// odd", IEEE Trans. Computers 57(4), 2008). Only 32-bit operations and the
// two conversions, so it costs a few instructions per element.
__device__ __forceinline__ uint16_t f64_to_bf16_rne(double v) {
  const float f = static_cast<float>(v);                // to nearest even
  uint32_t b = __float_as_uint(f);
  const double back = static_cast<double>(f);
  if (back != v) {
    if (fabs(back) > fabs(v)) b -= 1u;                  // step back toward zero: truncation
    b |= 1u;                                            // inexact: odd
  }
  b += 0x7FFFu + ((b >> 16) & 1u);                      // fp32 -> bf16 to nearest even
  return static_cast<uint16_t>(b >> 16);
}

// RMSNorm of one token per block ("DeepSeekMoE架构解析" section 4.1, eps 1e-6),
// in double precision: the squares of bf16 / fp32 inputs and, at the
// magnitudes used, their sum are exact in any order; then the mean, + eps,
// the square root, the division and the product by w are each one correctly
// rounded double operation, in this order; the result is rounded once to the
// activation dtype. A thread keeps its row elements (16-byte pieces) in
// registers between the two passes and writes back the same pieces, so u may
// alias x.
// For bf16 output each element is first formed in float as
// (x * (1 / root)) * w, within 3.1 float units in the last place of the
// double result (three roundings of 2^-24); a bf16 rounding boundary lies
// 2^15 such units from the nearest representable values, so unless the
// float value is within 8 units of one (or tiny) it rounds to the bf16 value
// the double result rounds to. The pieces with such an element (a few in a
// thousand) are left unwritten and redone through the double path at the
// end. Six waves per SIMD (the launch bound) hide the row loads' latency.
template <bool BF16>
__global__ __launch_bounds__(256, 6) void rmsnorm_kernel(const void* __restrict__ x,
                                                      const float* __restrict__ w, int d,
                                                      double eps, void* u) {
  constexpr int kMaxPieces = 8;                 // d <= 256 threads * 8 pieces * 8 (bf16)
  constexpr int EPP = BF16 ? 8 : 4;             // elements per 16-byte piece
  __shared__ double part[4];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x;
  const int npieces = d / EPP;
  const u32x4* src = reinterpret_cast<const u32x4*>(static_cast<const char*>(x) +
                                                    t * d * (BF16 ? 2 : 4));
  u32x4 keep[kMaxPieces];
  double acc = 0.0;
#pragma unroll
  for (int i = 0; i < kMaxPieces; ++i) {
    const int p = tid + 256 * i;
    if (p < npieces) {
      keep[i] = src[p];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (BF16) {
          const double a = bf16_to_f32(static_cast<uint16_t>(keep[i][q] & 0xFFFFu));
          const double c = bf16_to_f32(static_cast<uint16_t>(keep[i][q] >> 16));
          acc = fma(a, a, acc);
          acc = fma(c, c, acc);
        } else {
          const double a = __uint_as_float(keep[i][q]);
          acc = fma(a, a, acc);
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, kWave);
  if (lane_id() == 0) part[wave_id()] = acc;
  __syncthreads();
  const double ss = (part[0] + part[1]) + (part[2] + part[3]);
  const double root = sqrt(ss / d + eps);
  const float rinv32 = static_cast<float>(1.0 / root);
  u32x4* dst = reinterpret_cast<u32x4*>(static_cast<char*>(u) + t * d * (BF16 ? 2 : 4));
  uint32_t redo = 0;   // pieces to redo through the double path
#pragma unroll
  for (int i = 0; i < kMaxPieces; ++i) {
    const int p = tid + 256 * i;
    if (p < npieces) {
      u32x4 o;
      const int j0 = p * EPP;
      bool near = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (BF16) {
          const float a = bf16_to_f32(static_cast<uint16_t>(keep[i][q] & 0xFFFFu));
          const float c = bf16_to_f32(static_cast<uint16_t>(keep[i][q] >> 16));
          const float ya = (a * rinv32) * w[j0 + 2 * q];
          const float yc = (c * rinv32) * w[j0 + 2 * q + 1];
          const uint32_t ba = __float_as_uint(ya), bc = __float_as_uint(yc);
          near |= abs(static_cast<int>(ba & 0xFFFFu) - 0x8000) <= 8 || fabsf(ya) < 0x1p-120f;
          near |= abs(static_cast<int>(bc & 0xFFFFu) - 0x8000) <= 8 || fabsf(yc) < 0x1p-120f;
          const uint32_t lo = (ba + 0x7FFFu + ((ba >> 16) & 1u)) >> 16;
          const uint32_t hi = (bc + 0x7FFFu + ((bc >> 16) & 1u)) >> 16;
          o[q] = lo | (hi << 16);
        } else {
          const double a = __uint_as_float(keep[i][q]);
          o[q] = __float_as_uint(__double2float_rn((a / root) * static_cast<double>(w[j0 + q])));
        }
      }
      if (BF16 && near) redo |= 1u << i;   // left unwritten: x stays readable there
      else dst[p] = o;
    }
  }
  if (BF16 && redo) {
    // each element (x / root) * w, correctly rounded to bf16; x is re-read
    // from memory, which holds it still when u aliases x (these pieces were
    // not written above, and no other thread writes them)
#pragma unroll 1
    for (int i = 0; i < kMaxPieces; ++i) {
      if (!((redo >> i) & 1u)) continue;
      const int p = tid + 256 * i, j0 = p * EPP;
      const u32x4 xv = src[p];
      u32x4 o;
#pragma unroll 1
      for (int q = 0; q < 4; ++q) {
        const double a = bf16_to_f32(static_cast<uint16_t>(xv[q] & 0xFFFFu));
        const double c = bf16_to_f32(static_cast<uint16_t>(xv[q] >> 16));
        const uint32_t lo = f64_to_bf16_rne((a / root) * static_cast<double>(w[j0 + 2 * q]));
        const uint32_t hi = f64_to_bf16_rne((c / root) * static_cast<double>(w[j0 + 2 * q + 1]));
        o[q] = lo | (hi << 16);
      }
      dst[p] = o;
    }
  }
}

hipError_t launch_rmsnorm(const moe_config& c, const void* x, const float* weight, double eps,
                          void* u, hipStream_t s) {
  const int T = c.num_tokens, d = c.hidden;
  if (T == 0) return hipSuccess;
  if (c.act_dtype == MOE_DTYPE_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<true>, dim3(T), dim3(256), 0, s, x, weight, d, eps, u);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<false>, dim3(T), dim3(256), 0, s, x, weight, d, eps, u);
  return hipGetLastError();
}

hipError_t launch_bias_update(int32_t E, const int32_t* load, float gamma, float* bias,
                              hipStream_t s) {
  hipLaunchKernelGGL(bias_update_kernel, dim3(1), dim3(256), 0, s, load, E, gamma, bias);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t* p, int32_t value, int64_t n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_i32, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, p,
                     value, n);
  return hipGetLastError();
}

}  // namespace moe
