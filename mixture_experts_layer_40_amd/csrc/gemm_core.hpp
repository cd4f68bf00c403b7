// The K loop shared by the grouped expert GEMMs and the router GEMM on
// gfx950: v_mfma_f32_32x32x16_bf16 (or, for fp8 codes on both sides,
// v_mfma_scale_f32_32x32x64_f8f6f4) with weight rows as the first operand,
// token rows as the second, tokens staged through LDS by direct loads.
#pragma once

#include "common.hpp"

namespace moe {

// ---------------------------------------------------------------------------
// bf16 activations, bf16 or fp8 weights, MFMA 32x32x16.
//
// A block computes 256 weight rows (8 fragments of 32) x BM tokens
// (BM = 32..256): either 8 waves, two per SIMD, each owning one fragment and
// all BM tokens (RF = 1), or 4 waves, one per SIMD, each owning two
// fragments (RF = 2: 512 registers per lane, the accumulators in AGPRs, and
// each token fragment read from LDS feeds two MFMAs, which halves the LDS
// reads per flop). In the expert GEMMs, gate/up fragments hold 16 gate and
// the 16 up rows of the same intermediate columns (see ffn.hip).
// Weight rows are never shared between waves: each lane streams its 64
// bytes of a fragment per 64-wide K stage (lane group g = l/32 takes
// K-elements 32g .. 32g+31 of the stage, 8 per MFMA step) straight into a
// register ring NSA stages deep. The token tile, read by all the block's waves, goes
// global -> LDS by direct loads, MOE_TOKEN_STAGES buffers deep; 16-byte
// chunks are XOR-swizzled by row pair, so the 16 rows one ds_read_b128 serves
// land on 16 distinct bank groups. Each stage's memory requests are spread
// over its MFMAs. The K loop is specialised on the number NT of 32-token
// fragments the tile really has: branch-free, and a tile with 3 rows costs
// one fragment.
//
// F8B (fine-grained fp8, "DeepSeekMoE架构解析" section 4.3): weights and
// tokens are both E4M3 codes and a stage is 128 K-elements -- one block of
// the 128 x 128 weight scales and of the 1 x 128 token scales, and the same
// bytes per stage as the bf16 loop (4 KB of a 32-row tiled fragment, 128
// bytes per token row), so the DMA and the counter waits are unchanged. A
// stage is two 32x32x64 fp8 MFMAs per token fragment into a block partial
// that starts from zero; the caller's hook `post(NT, s, blk)` then adds the
// partials, times their scales, into its fp32 accumulators. The fp8 MFMA
// aligns its 64 products (and its C input) to the largest before summing,
// losing bits below about 2^-12 of that sum, so a long accumulation kept
// inside the MFMA chain would lose accuracy as the sum grows; promoting
// each 128-wide block to VALU fp32 bounds the loss by the block's own
// magnitude (the promotion of "DeepSeekMoE架构解析" section 4.3).
// ---------------------------------------------------------------------------
constexpr int kThreads = 512;
#ifndef MOE_TOKEN_STAGES
#define MOE_TOKEN_STAGES 3
#endif

template <int V>
struct IntC {
  static constexpr int value = V;
};
template <int N, int I = 0, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(IntC<I>{});
    static_for<N, I + 1>(f);
  }
}

typedef __attribute__((address_space(3))) void lds_ptr_t;
typedef __attribute__((address_space(1))) void glb_ptr_t;

// One 16-byte global -> LDS copy per lane, bypassing registers: lane l of the
// wave writes its 16 bytes at lds_wave_base + 16 * l.
__device__ __forceinline__ void dma16(const void* src, void* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((glb_ptr_t*)src, (lds_ptr_t*)lds_wave_base, 16, 0, 0);
}

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

struct NoPost {
  template <class N, class A>
  __device__ __forceinline__ void operator()(N, int, A&) const {}
};

// NTW: the weight loads carry the non-temporal hint. A launch of few-token
// tiles (decode) is a stream of expert weights read once, and with the hint
// the part moves such a stream from HBM at ≈7.0 TB/s against ≈6.0 with plain
// loads (a per-CU streaming probe, every CU busy): the decode layer call
// drops from 1.30 to 1.20 ms. Launches of many-token tiles, whose sibling
// tiles re-read a weight block through the caches, ran 1-2 % slower with
// it, and the router re-reads its weight rows in every block: both keep
// plain loads.
template <bool FP8, int NSA, int BM, bool F8B = false, int RF = 1, bool NTW = false>
struct MainLoop {
  static_assert(!(FP8 && F8B), "F8B takes fp8 codes on both sides; FP8 widens weights to bf16");
  static_assert(RF == 1 || (RF == 2 && !F8B), "two fragments per wave: bf16 / fp8-row loops only");
  // RF weight fragments per wave: kThreads / RF threads per block, so the
  // block still covers 8 fragments (256 rows); with RF = 2 each token
  // fragment read from LDS feeds two MFMAs.
  static constexpr int TH = kThreads / RF;
  static constexpr int NTF = BM / 32;
  static constexpr int AW = FP8 ? 2 : 4;       // 16-byte loads per fragment per stage
  static constexpr size_t WB = FP8 ? 1 : 2;    // bytes per weight
  static constexpr int ND = MOE_TOKEN_STAGES;  // LDS token stages (ND-1 in flight)
  static constexpr int gcd(int x, int y) { return y == 0 ? x : gcd(y, x % y); }
  static constexpr int U = ND * NSA / gcd(ND, NSA);   // unroll: lcm(ND, NSA)

  // acc[t] += W fragment x token fragment t, over the whole K axis. Every
  // load and MFMA is unconditional: token rows past the expert's end read
  // its last row, prefetches past the last stage re-read the last stage, and
  // when a stage has fewer 16-byte chunks than threads the extra threads
  // repeat a chunk (writing the same bytes to the same place).
  // kdim counts 16-bit units of a token row (fp8 rows: bytes / 2); one
  // stage is 64 such units.
  template <int NT>
  __device__ __forceinline__ static void run(const uint8_t* const (&aptr)[RF], const uint16_t* act,
                                             int row0, const int32_t* act_rows, int act_div,
                                             int mvalid, int kdim, int astage, int avs,
                                             uint16_t* bs0, uint16_t* bs1, uint16_t* bs2,
                                             uint16_t* bs3, f32x16 (&acc)[RF * NTF]) {
    run<NT>(aptr, act, row0, act_rows, act_div, mvalid, kdim, astage, avs, bs0, bs1, bs2, bs3,
            acc, NoPost{});
  }

  template <int NT, class Post>
  __device__ __forceinline__ static void run(const uint8_t* const (&aptr)[RF], const uint16_t* act,
                                             int row0, const int32_t* act_rows, int act_div,
                                             int mvalid, int kdim, int astage, int avs,
                                             uint16_t* bs0, uint16_t* bs1, uint16_t* bs2,
                                             uint16_t* bs3, f32x16 (&acc)[RF * NTF], Post&& post) {
    constexpr int CH = NT * 32 * 8;                     // 16-byte chunks per token stage
    constexpr int BCH = (CH + TH - 1) / TH;             // copies per thread per stage
    const int l = lane_id(), g = l >> 5, r32 = l & 31;
    const int w = __builtin_amdgcn_readfirstlane(wave_id());
    const int nk = kdim / 64;

    // Copy i of a wave fills 64 consecutive 16-byte LDS slots starting at
    // slot q0; slot q holds token row q/8, physical chunk q%8, which carries
    // the logical K-chunk (q%8) ^ ((row/2)%8).
    const uint16_t* bsrc[BCH];
    int bdst[BCH];
#pragma unroll
    for (int i = 0; i < BCH; ++i) {
      const int q0 = (w * kWave + TH * i) % CH;
      const int q = q0 + l, row = q >> 3, ch = (q & 7) ^ ((row >> 1) & 7);
      const int p = row0 + (row < mvalid ? row : mvalid - 1);
      const int src = act_rows ? max(act_rows[p], 0) / act_div : p;
      bsrc[i] = act + static_cast<size_t>(src) * kdim + ch * 8;
      bdst[i] = q0 * 8;
    }

    u32x4 ra[NSA][RF * AW];
    auto load_w = [](const uint8_t* p) {
      if constexpr (NTW) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
      return *reinterpret_cast<const u32x4*>(p);
    };
    // This lane's AW 16-byte pieces of K stage ks of fragment f: at
    // aptr[f] + ks * astage + v * avs (rows layout: 16 consecutive bytes of
    // its row; tiled layout: one 1 KB stripe per piece, so each load
    // instruction reads 1 KB).
    auto load_a = [&](u32x4 (&dst)[RF * AW], int ks) {
#pragma unroll
      for (int f = 0; f < RF; ++f) {
        const uint8_t* p = aptr[f] + static_cast<size_t>(ks) * astage;
#pragma unroll
        for (int v = 0; v < AW; ++v) dst[f * AW + v] = load_w(p + v * avs);
      }
    };
    auto load_b = [&](uint16_t* buf, int ks) {
#pragma unroll
      for (int i = 0; i < BCH; ++i) dma16(bsrc[i] + ks * 64, buf + bdst[i]);
    };
    auto read_b = [&](u32x4& dst, const uint16_t* b0, int t, int s) {
      const int tok = 32 * t + r32, ch = 4 * g + s;
      dst = *reinterpret_cast<const u32x4*>(b0 + tok * 64 + ((ch ^ ((tok >> 1) & 7)) * 8));
    };
    // One 64-wide K stage: four MFMA steps. Fragment t of step s+1 is read
    // from LDS just before the MFMA of fragment t of step s (order pinned).
    // The stage's NV memory requests (issue(0 .. NV-1)) are spread evenly
    // over its 4*NT MFMAs: issued in one burst they queue at the CU's
    // address unit and hold every wave's MFMAs back behind them.
    constexpr int NV = BCH + RF * AW;
    // F8B: the two 64-wide halves m of a 128-wide stage; lane group g takes
    // codes 32g .. 32g+31 of each half: weight pieces 2m, 2m+1 and token
    // chunks 4m+2g, 4m+2g+1 (the same K order on both operands).
    auto read_b8 = [&](u32x4 (&dst)[2], const uint16_t* b0, int t, int m) {
      const int tok = 32 * t + r32, c0 = 4 * m + 2 * g, sw = (tok >> 1) & 7;
      const uint16_t* row = b0 + tok * 64;
      dst[0] = *reinterpret_cast<const u32x4*>(row + ((c0 ^ sw) * 8));
      dst[1] = *reinterpret_cast<const u32x4*>(row + (((c0 + 1) ^ sw) * 8));
    };
    auto compute8 = [&](const u32x4 (&src)[RF * AW], const uint16_t* b0, f32x16 (&blk)[NT],
                        auto&& issue) {
      u32x4 bfr[2][NT][2];
#pragma unroll
      for (int t = 0; t < NT; ++t) read_b8(bfr[0][t], b0, t, 0);
#pragma unroll
      for (int m = 0; m < 2; ++m) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (m == 0) read_b8(bfr[1][t], b0, t, 1);
          blk[t] = mfma_32x32x64_fp8(src[2 * m], src[2 * m + 1], bfr[m][t][0], bfr[m][t][1],
                                     m == 0 ? f32x16{} : blk[t]);
          const int i = m * NT + t;
          static_for<NV>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            if ((k * 2 * NT) / NV == i) issue(kc);
          });
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    auto compute = [&](const u32x4 (&src)[RF * AW], const uint16_t* b0, auto&& issue) {
      u32x4 bfr[2][NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) read_b(bfr[0][t], b0, t, 0);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        u32x4 op[RF];
#pragma unroll
        for (int f = 0; f < RF; ++f) {
          if constexpr (FP8) {
            u32x4 lo, hi;
            fp8x16_to_bf16x16(src[f * AW + (s >> 1)], lo, hi);
            op[f] = (s & 1) ? hi : lo;
          } else {
            op[f] = src[f * AW + s];
          }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (s < 3) read_b(bfr[(s + 1) & 1][t], b0, t, s + 1);
#pragma unroll
          for (int f = 0; f < RF; ++f)
            acc[f * NTF + t] = mfma_32x32x16(op[f], bfr[s & 1][t], acc[f * NTF + t]);
          const int i = s * NT + t;
          static_for<NV>([&](auto kc) {
            constexpr int k = decltype(kc)::value;
            if ((k * 4 * NT) / NV == i) issue(kc);
          });
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    // RF = 2: the 4*NT token-fragment reads of a stage, in (step, fragment)
    // order, run LA reads ahead of the MFMA pairs that use them through a
    // ring of LA + 1 registers (in place of a whole step's fragments).
    auto compute2 = [&](const u32x4 (&src)[RF * AW], const uint16_t* b0, auto&& issue) {
      constexpr int LA = 3, J = 4 * NT;
      u32x4 bq[LA + 1];
      static_for<(LA < J ? LA : J)>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        read_b(bq[j], b0, j % NT, j / NT);
      });
      static_for<J>([&](auto jc) {
        constexpr int j = decltype(jc)::value, s = j / NT, t = j % NT;
        if constexpr (j + LA < J) read_b(bq[(j + LA) % (LA + 1)], b0, (j + LA) % NT, (j + LA) / NT);
#pragma unroll
        for (int f = 0; f < RF; ++f) {
          u32x4 op;
          if constexpr (FP8) {
            u32x4 lo, hi;
            fp8x16_to_bf16x16(src[f * AW + (s >> 1)], lo, hi);
            op = (s & 1) ? hi : lo;
          } else {
            op = src[f * AW + s];
          }
          acc[f * NTF + t] = mfma_32x32x16(op, bq[j % (LA + 1)], acc[f * NTF + t]);
        }
        static_for<NV>([&](auto kc) {
          constexpr int k = decltype(kc)::value;
          if constexpr ((k * J) / NV == j) issue(kc);
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    };
    auto buf = [&](int i) { return i == 0 ? bs0 : (i == 1 ? bs1 : (i == 2 ? bs2 : bs3)); };

    // Issue order (the counter waits below depend on it): prologue
    // T(0) .. T(ND-2), W(0) .. W(NSA-2); stage s: the pieces of T(s+ND-1),
    // then those of W(s+NSA-1), spread over its MFMAs.
#pragma unroll
    for (int p = 0; p < ND - 1; ++p) load_b(buf(p), min(p, nk - 1));
#pragma unroll
    for (int p = 0; p < NSA - 1; ++p) load_a(ra[p], min(p, nk - 1));
    __builtin_amdgcn_sched_barrier(0);
    // Everything of the prologue landed. T(1) and the first weights were
    // requested together with T(0), so this costs little more than waiting
    // for T(0), and it leaves the K loop one clean state to carry (with
    // requests of the prologue still counted, the compiler's own waits at
    // the loop head fall back to draining every request each iteration).
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    // One K stage s; u = s mod U fixes its LDS buffer and ring slot at
    // compile time.
    auto stage = [&](auto uc, int s) {
      constexpr int u = decltype(uc)::value;
      uint16_t* tdst = buf((u + ND - 1) % ND);          // its readers passed the last barrier
      const int ts = min(s + ND - 1, nk - 1);
      u32x4 (&wdst)[RF * AW] = ra[(u + NSA - 1) % NSA]; // consumed in the previous stage
      const size_t woff = static_cast<size_t>(min(s + NSA - 1, nk - 1)) * astage;
      // requests 0 .. BCH-1: T(s+ND-1); BCH .. NV-1: W(s+NSA-1), fragment by fragment
      auto issue = [&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k < BCH) {
          dma16(bsrc[k] + ts * 64, tdst + bdst[k]);
        } else {
          constexpr int f = (k - BCH) / AW, v = (k - BCH) % AW;
          wdst[f * AW + v] = load_w(aptr[f] + woff + v * avs);
        }
      };
      // W(s) landed: after its last piece came the requests of NSA-2 stages
      wait_vmcnt<(NSA - 2) * NV>();
      if constexpr (F8B) {
        f32x16 blk[NT];
        compute8(ra[u % NSA], buf(u % ND), blk, issue);
        post(IntC<NT>{}, s, blk);
      } else if constexpr (RF == 2) {
        compute2(ra[u % NSA], buf(u % ND), issue);
      } else {
        compute(ra[u % NSA], buf(u % ND), issue);
      }
      __builtin_amdgcn_sched_barrier(0);
      // T(s+1) landed: after it were issued the W of its stage and the
      // T and W of ND-2 stages. A plain barrier: the fence of __syncthreads
      // would wait for every copy in flight; this stage's LDS reads are
      // complete, their MFMAs issued.
      wait_vmcnt<RF * AW + (ND - 2) * NV>();
      __builtin_amdgcn_s_barrier();
    };
    // Whole groups of U stages, then the remainder, outside the loop so the
    // loop carries one pipeline state (a break inside it would merge the
    // states of every stage into the loop head and force full drains).
    const int full = nk - nk % U;
    for (int base = 0; base < full; base += U) {
      static_for<U>([&](auto uc) { stage(uc, base + decltype(uc)::value); });
    }
    static_for<U - 1>([&](auto uc) {
      if (full + decltype(uc)::value < nk) stage(uc, full + decltype(uc)::value);
    });
  }
};

}  // namespace moe
