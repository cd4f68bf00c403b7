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

// One thread per 8 consecutive features of one token: out_slots in the
// activation dtype, y_shared fp32, y in the output dtype.
template <bool SLOT_BF16, bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_kernel(const void* __restrict__ slots,
                                                      const float* __restrict__ ysh, int T, int K,
                                                      int d, void* __restrict__ y) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int vpr = d / 8;
  if (i >= static_cast<int64_t>(T) * vpr) return;
  const int64_t t = i / vpr;
  const int c = static_cast<int>(i % vpr) * 8;
  float acc[8];
  if (ysh) {
    const f32x4 v0 = *reinterpret_cast<const f32x4*>(ysh + t * d + c);
    const f32x4 v1 = *reinterpret_cast<const f32x4*>(ysh + t * d + c + 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) { acc[q] = v0[q]; acc[4 + q] = v1[q]; }
  } else {
#pragma unroll
    for (int q = 0; q < 8; ++q) acc[q] = 0.f;
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
                          void* y, hipStream_t s) {
  const int T = c.num_tokens, K = c.top_k, d = c.hidden;
  if (T == 0) return hipSuccess;
  const int64_t n = static_cast<int64_t>(T) * (d / 8);
  const dim3 grid(static_cast<unsigned>((n + 255) / 256)), block(256);
  const float* ysh = static_cast<const float*>(y_shared);
  const bool sb = c.act_dtype == MOE_DTYPE_BF16, ob = c.out_dtype == MOE_DTYPE_BF16;
  if (sb && ob) hipLaunchKernelGGL((combine_kernel<true, true>), grid, block, 0, s, out_slots, ysh, T, K, d, y);
  else if (sb) hipLaunchKernelGGL((combine_kernel<true, false>), grid, block, 0, s, out_slots, ysh, T, K, d, y);
  else hipLaunchKernelGGL((combine_kernel<false, false>), grid, block, 0, s, out_slots, ysh, T, K, d, y);
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
