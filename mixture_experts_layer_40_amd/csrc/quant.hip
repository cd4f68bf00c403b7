// Online quantisation of the layer input to fp8 in 1 x 128 tiles
// ("DeepSeekMoE架构解析" section 4.3: tile-wise activation scales, the
// max-abs taken as the data is read).
//
// Per tile of 128 consecutive channels of one token: amax = max |x|,
// scale = amax / 448 (fp32, rounded once; 1 for an all-zero tile), code =
// the E4M3 value nearest to x / scale (fp32 division rounded once, ties to
// even). One wave holds four tiles, 16 lanes x 8 bf16 values each: one
// 16-byte load per lane, the max over the 16 lanes by shuffles, 8 bytes of
// codes per lane and one scale per tile written back.
#include "common.hpp"
#include "launch.hpp"

namespace moe {

namespace {

__global__ __launch_bounds__(256) void quant_tiles_bf16(const uint16_t* __restrict__ x,
                                                        int64_t ntiles, int tiles_per_row,
                                                        uint8_t* __restrict__ xq,
                                                        float* __restrict__ xs) {
  const int l = lane_id();
  const int64_t tile = (static_cast<int64_t>(blockIdx.x) * 4 + wave_id()) * 4 + (l >> 4);
  if (tile >= ntiles) return;        // whole 16-lane groups leave together
  const int sub = l & 15;
  const int64_t row = tile / tiles_per_row;
  const int64_t col = (tile - row * tiles_per_row) * 128 + sub * 8;
  const int64_t off = row * tiles_per_row * 128 + col;
  const u32x4 v = *reinterpret_cast<const u32x4*>(x + off);
  float f[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f[2 * q] = bf16_to_f32(static_cast<uint16_t>(v[q] & 0xFFFFu));
    f[2 * q + 1] = bf16_to_f32(static_cast<uint16_t>(v[q] >> 16));
  }
  float m = 0.f;
#pragma unroll
  for (int q = 0; q < 8; ++q) m = fmaxf(m, fabsf(f[q]));
#pragma unroll
  for (int o = 8; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 16));
  const float sc = m > 0.f ? __fdiv_rn(m, 448.0f) : 1.0f;
  u32x2 codes = {0u, 0u};
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint32_t c = f32_to_e4m3(__fdiv_rn(f[q], sc));
    if (q < 4) codes.x |= c << (8 * q);
    else codes.y |= c << (8 * (q - 4));
  }
  *reinterpret_cast<u32x2*>(xq + off) = codes;
  if (sub == 0) xs[tile] = sc;
}

}  // namespace

hipError_t launch_quantize_act(const moe_config& c, const void* x, void* xq, float* xs,
                               hipStream_t s) {
  const int64_t ntiles = static_cast<int64_t>(c.num_tokens) * (c.hidden / 128);
  if (ntiles == 0) return hipSuccess;
  const int64_t blocks = (ntiles + 15) / 16;     // 4 waves x 4 tiles
  hipLaunchKernelGGL(quant_tiles_bf16, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const uint16_t*>(x), ntiles, c.hidden / 128,
                     static_cast<uint8_t*>(xq), xs);
  return hipGetLastError();
}

}  // namespace moe
