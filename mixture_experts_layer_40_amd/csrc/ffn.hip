// Grouped SwiGLU expert GEMMs: routed experts over expert-contiguous rows and
// the always-on shared expert(s) over all tokens.
//
// Method: fine-grained routed experts plus shared experts ("DeepSeekMoE架构解析"
// section 1); each expert is a SwiGLU FFN E(v) = W2 (SiLU(W1 v) * (W3 v)) and
// each routed output is weighted by its gate (section 2.1, eq. 13) before the
// weighted sum (section 3.1 sketch). The shared experts are passed
// concatenated (W1, W3 stacked by rows, W2 by columns), which is the same sum.
//
// CDNA4 design (bf16 / fp8 weights):
//  * Orientation: weight rows are the first MFMA operand (v_mfma 32x32x16),
//    token rows the second. A block computes 256 weight rows (8 fragments
//    of 32) x up to 256 tokens of one expert. At 128/256-token tiles it is 4
//    waves, one per SIMD, each owning two fragments and all tokens of the
//    tile (accumulators in AGPRs; each token fragment read from LDS feeds
//    two MFMAs); at 32/64-token tiles 8 waves, two per SIMD, one fragment
//    each. Weight rows are never shared between waves, so every wave streams
//    its rows from HBM straight into MFMA operand registers, two stages ahead
//    (fp8 codes are widened to bf16 in registers, exactly). In the tiled
//    weight layout each of those loads reads a whole 1 KB stripe.
//  * The token tile, which all the block's waves read, goes global -> LDS by direct
//    LDS loads (no registers), three stages deep; 16-byte chunks are
//    XOR-swizzled by row pair so the 16 rows one ds_read_b128 serves land on
//    16 distinct groups of the 64 banks.
//  * Skew: the K loop is specialised on the number of 32-token fragments a
//    tile really has, so an expert with 3 rows costs one fragment of MFMA
//    work while its weights are still read exactly once per token tile.
//  * Tiles are ordered (expert, weight block, token block) with the token
//    block fastest and dealt to XCDs in contiguous ranges, so the token tiles
//    that share a weight block run together on one XCD and its L2.
//  * Gate/up: a wave's 32 rows are 16 gate (W1) rows and the 16 up (W3) rows
//    of the same intermediate columns, so SiLU(g) * u is formed in registers
//    and H is written once in bf16.
//  * Down: the epilogue multiplies by the fp8 row scale and the token's gate
//    and writes the row straight to its (token, slot) position.
#include <math.h>

#include <algorithm>

#include "common.hpp"
#include "gemm_core.hpp"
#include "launch.hpp"

namespace moe {

namespace {

constexpr int kBNGate = 128;      // intermediate columns per gate/up tile (x2 rows: W1 + W3)
constexpr int kBNDown = 256;      // output rows per down tile
constexpr int kBMF32 = 32;        // tokens per tile (fp32 path)
constexpr int kBNF32 = 32;        // columns per tile (fp32 path)

enum { kGateUp = 0, kDown = 1 };

// One set of GEMM groups over one pair of weight tensors: E expert groups
// over expert-contiguous rows (offsets != null) or one group of fixed_m rows.
struct GemmSet {
  const void* act;            // activations (bf16 or fp32), kdim per row
  const int32_t* act_rows;    // row p of the GEMM reads act row act_rows[p] / act_div
  int act_div;                //   (null: act row p)
  const void* wa;             // gate/up: W1 (or the tiled gate/up tensor); down: W2
  const void* wb;             // gate/up: W3 (rows layout)
  const float* sa;            // fp8 row scales of wa ([E, n]) or null
  const float* sb;            // fp8 row scales of wb
  const int32_t* offsets;     // [E+1] expert row offsets, or null = one group of fixed_m rows
  const int32_t* sched;       // [E+1] first tile of each expert (with offsets)
  int fixed_m;
  int E;
  int kdim;                   // reduction length
  int n;                      // weight rows per expert (gate/up: per W1/W3)
  int nb;                     // weight blocks per expert
  int64_t wstride;            // elements per expert of wa / wb
  void* h;                    // gate/up output [rows, n]
  const int32_t* perm_slot;   // down: row -> output row (null = identity)
  const float* gate;          // down: gate per output row (null = 1)
  void* out;                  // down output [slots, n]
  int out_f32;                // down output is fp32 (else bf16)
  int tiled;                  // weights in the tiled layout (wa only; see pack_tiles)
  // fine-grained fp8 (grouped_gemm_f8b): act holds E4M3 codes; sa / sb are
  // 128 x 128 block scales [E, n/128, kdim/128] of wa (W1 or W2) / W3
  const float* ascale;        // token tile scales [act rows, kdim/128]
  float* hscale;              // gate/up: h tile scales out [rows, n/128]
};

// A launch covers the tiles of one or two sets (set 0's tiles first), e.g.
// the shared expert and the routed experts in one grid.
struct GemmArgs {
  GemmSet s[2];
  int nsets;
  const int32_t* xb;  // [kNumXcd + 1] first tile of each XCD's range (see ffn_schedule), or null
};

struct Tile {
  int set, e, row0, mvalid, nblk;
};

__device__ __forceinline__ int set_tiles(const GemmSet& g, int bm) {
  return g.offsets ? g.sched[g.E] : ((g.fixed_m + bm - 1) / bm) * g.nb;
}

// Tile `tile` of one set: its expert, row range and weight block.
__device__ __forceinline__ void decode_set_tile(const GemmSet& g, int bm, int tile, Tile& t) {
  int e = 0, local = tile, rbeg = 0, m = g.fixed_m;
  if (g.offsets) {
    int lo = 0, hi = g.E - 1;  // largest e with sched[e] <= tile
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (g.sched[mid] <= tile) lo = mid; else hi = mid - 1;
    }
    e = lo;
    local = tile - g.sched[e];
    rbeg = g.offsets[e];
    m = g.offsets[e + 1] - rbeg;
  }
  // An expert's rows are split into mt = ceil(m / bm) tiles of nearly equal
  // size (multiples of 32 rows): the tiles that share a weight block then
  // run for about as long, in step, and the later ones find its lines in L2.
  const int mt = (m + bm - 1) / bm;
  const int mb = local % mt;
  const int per = (((m + mt - 1) / mt) + 31) & ~31;
  t.e = e;
  t.nblk = local / mt;
  t.row0 = rbeg + mb * per;
  t.mvalid = min(per, m - mb * per);
}

// Decode this block's tile; false when the block has no work. Block b runs
// on XCD x = b % 8 (blocks are dealt to the XCDs in turn) as the j-th block
// (j = b / 8) of that XCD, and takes the j-th tile of XCD x's range of the
// launch's tiles (set 0's, then set 1's), so the tiles that share a weight
// block run together on one L2. With a.xb the ranges are those ffn_schedule
// balanced by estimated cost; else each set is cut into 8 equal slices,
// XCD x taking slice x of set 0 and then slice x of set 1.
__device__ __forceinline__ bool decode_tile(const GemmArgs& a, int bm, Tile& t) {
  const int n0 = set_tiles(a.s[0], bm);
  const int n1 = a.nsets > 1 ? set_tiles(a.s[1], bm) : 0;
  const int x = blockIdx.x % kNumXcd, j = blockIdx.x / kNumXcd;
  int tile;
  if (a.xb) {
    tile = a.xb[x] + j;
    if (tile >= a.xb[x + 1]) return false;
  } else {
    const int p0 = (n0 + kNumXcd - 1) / kNumXcd, p1 = (n1 + kNumXcd - 1) / kNumXcd;
    const int c0 = min(max(n0 - x * p0, 0), p0);     // set-0 tiles of this XCD
    if (j < c0) {
      tile = x * p0 + j;
    } else {
      const int k = j - c0;
      if (k >= p1 || x * p1 + k >= n1) return false;
      tile = n0 + x * p1 + k;
    }
  }
  t.set = tile < n0 ? 0 : 1;
  if (t.set) tile -= n0;
  decode_set_tile(a.s[t.set], bm, tile, t);
  return true;
}

// The K loop (MainLoop) and its building blocks are in gemm_core.hpp.

template <int MODE, bool FP8, int BM, int NSA, int RF = 1>
__global__ __launch_bounds__(kThreads / RF) void grouped_gemm_mfma(GemmArgs args) {
  constexpr int NTF = BM / 32;
  __shared__ __attribute__((aligned(16))) uint16_t bs0[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t bs1[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t bs2[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t bs3[MOE_TOKEN_STAGES > 3 ? BM * 64 : 8];

  Tile tl;
  if (!decode_tile(args, BM, tl)) return;
  const GemmSet& a = args.s[tl.set];

  const int l = lane_id(), w = wave_id(), g = l >> 5, r32 = l & 31;
  const int ntf = (tl.mvalid + 31) >> 5;

  // ---- this wave's RF 32-row weight fragments (rb0 .. rb0 + RF - 1) ----
  // Rows layout: lane l reads row (l % 32) of a fragment, K-elements
  // 32g .. 32g+31 of each 64-wide stage (g = l / 32), 16 bytes at a time.
  // Tiled layout: fragment rb, stage ks is one contiguous tile of 32 x 64
  // weights; lane l's piece v sits at byte v * 1024 + 16 l of it.
  // Fragments past the weight rows read fragment 0 and store nothing.
  const uint8_t* aptr[RF];
  constexpr int wbytes = FP8 ? 1 : 2;
  const int nk = a.kdim / 64;
  const int astage = a.tiled ? 32 * 64 * wbytes : 64 * wbytes, avs = a.tiled ? 1024 : 16;
  const int rb0 = (MODE == kGateUp ? tl.nblk * kBNGate / 16 : tl.nblk * kBNDown / 32) + RF * w;
  auto frag_row0 = [&](int f) { return MODE == kGateUp ? 16 * (rb0 + f) : 32 * (rb0 + f); };
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    const int rbv = frag_row0(f) < a.n ? rb0 + f : 0;
    if (a.tiled) {
      aptr[f] = static_cast<const uint8_t*>(a.wa) + static_cast<size_t>(tl.e) * a.wstride * wbytes +
                static_cast<size_t>(rbv) * nk * astage + 16 * l;
    } else if (MODE == kGateUp) {
      const int row = 16 * rbv + (r32 & 15);
      aptr[f] = static_cast<const uint8_t*>(r32 < 16 ? a.wa : a.wb) +
                (static_cast<size_t>(tl.e) * a.wstride + static_cast<size_t>(row) * a.kdim + 32 * g) * wbytes;
    } else {
      const int row = 32 * rbv + r32;
      aptr[f] = static_cast<const uint8_t*>(a.wa) +
                (static_cast<size_t>(tl.e) * a.wstride + static_cast<size_t>(row) * a.kdim + 32 * g) * wbytes;
    }
  }

  f32x16 acc[RF * NTF];
#pragma unroll
  for (int t = 0; t < RF * NTF; ++t) acc[t] = f32x16{};

  const uint16_t* act = static_cast<const uint16_t*>(a.act);
  // non-temporal weight loads for the few-token tiles, whose launches only
  // stream weights (see MainLoop); the many-token tiles keep plain loads
  using ML = MainLoop<FP8, NSA, BM, false, RF, (BM <= 64)>;
  switch (ntf) {
#define MOE_NT_CASE(n) \
    case n: if constexpr (n <= NTF) ML::template run<n>(aptr, act, tl.row0, a.act_rows, a.act_div, tl.mvalid, a.kdim, astage, avs, bs0, bs1, bs2, bs3, acc); break;
    MOE_NT_CASE(1) MOE_NT_CASE(2) MOE_NT_CASE(3) MOE_NT_CASE(4)
    MOE_NT_CASE(5) MOE_NT_CASE(6) MOE_NT_CASE(7) MOE_NT_CASE(8)
#undef MOE_NT_CASE
    default: break;
  }

  // Down: each token column's output slot and gate, fetched for all of the
  // tile's token fragments at once (two rounds of loads per tile): fetched
  // fragment by fragment next to the stores, every load's wait also drained
  // the stores before it, and the 2 x NTF round trips cost about 23 us per
  // tile, 40 % of a down tile at d = 2048.
  int slot_t[NTF];
  float gate_t[NTF];
  if (MODE == kDown) {
#pragma unroll
    for (int t = 0; t < NTF; ++t) {
      const int tok = 32 * t + r32;
      const int p = tl.row0 + tok;
      const bool live = t < ntf && tok < tl.mvalid;
      slot_t[t] = !live ? -1 : (a.perm_slot ? a.perm_slot[p] : p);
    }
#pragma unroll
    for (int t = 0; t < NTF; ++t)
      gate_t[t] = (a.gate && slot_t[t] >= 0) ? a.gate[slot_t[t]] : 1.f;
  }

#pragma unroll
  for (int f = 0; f < RF; ++f) {
  const int nrow0 = frag_row0(f);  // gate/up: first of 16 intermediate columns; down: first of 32 rows
  if (nrow0 >= a.n) continue;
  f32x16* facc = acc + f * NTF;
  if (MODE == kGateUp) {
    uint16_t* h = static_cast<uint16_t*>(a.h);
#pragma unroll
    for (int i = 0; i < 2; ++i) {          // result rows 8i+4g+q: gate; +16: up
      const int col = nrow0 + 8 * i + 4 * g;
      float sg[4] = {1.f, 1.f, 1.f, 1.f}, su[4] = {1.f, 1.f, 1.f, 1.f};
      if (FP8) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          sg[q] = a.sa[static_cast<size_t>(tl.e) * a.n + col + q];
          su[q] = a.sb[static_cast<size_t>(tl.e) * a.n + col + q];
        }
      }
#pragma unroll
      for (int t = 0; t < NTF; ++t) {
        const int tok = 32 * t + r32;
        if (t < ntf && tok < tl.mvalid) {
          float hv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q)
            hv[q] = silu_fast(facc[t][4 * i + q] * sg[q]) * (facc[t][4 * (i + 2) + q] * su[q]);
          u32x2 v;
          v.x = pack_bf16x2(hv[0], hv[1]);
          v.y = pack_bf16x2(hv[2], hv[3]);
          *reinterpret_cast<u32x2*>(h + static_cast<size_t>(tl.row0 + tok) * a.n + col) = v;
        }
      }
    }
  } else {
#pragma unroll
    for (int t = 0; t < NTF; ++t) {
      const int slot = slot_t[t];
      if (slot < 0) continue;           // past the tile's rows, or a slot with no expert
      const float gv = gate_t[t];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = nrow0 + 8 * i + 4 * g;
        float ov[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float sc = FP8 ? a.sa[static_cast<size_t>(tl.e) * a.n + col + q] : 1.f;
          ov[q] = (facc[t][4 * i + q] * sc) * gv;
        }
        const size_t o = static_cast<size_t>(slot) * a.n + col;
        if (a.out_f32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o) = f32x4{ov[0], ov[1], ov[2], ov[3]};
        } else {
          u32x2 v;
          v.x = pack_bf16x2(ov[0], ov[1]);
          v.y = pack_bf16x2(ov[2], ov[3]);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o) = v;
        }
      }
    }
  }
  }
}

// ---------------------------------------------------------------------------
// Fine-grained fp8 ("DeepSeekMoE架构解析" section 4.3): E4M3 weights with one
// fp32 scale per 128 x 128 block and E4M3 tokens with one per 1 x 128 tile,
// fp8 MFMA with fp32 accumulation. One K stage is one 128-wide block: its
// partial sum (two MFMAs from zero) is added to the fp32 accumulators by
// the VALU, times c = (weight block scale) x (token tile scale); the scales
// of the tile's tokens and of each wave's weight rows are staged in LDS.
// Gate/up writes h as E4M3 codes with one scale per 1 x 128 tile: a tile of
// this kernel holds exactly the 128 intermediate columns of one h tile for
// every token, so the tile's max-abs is a block-wide reduction.
// ---------------------------------------------------------------------------
constexpr int kF8MaxKB = 64;      // kdim <= 8192

template <int MODE, int BM, int NSA>
__global__ __launch_bounds__(kThreads) void grouped_gemm_f8b(GemmArgs args) {
  constexpr int NTF = BM / 32;
  __shared__ __attribute__((aligned(16))) uint16_t bs0[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t bs1[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t bs2[BM * 64];
  __shared__ __attribute__((aligned(16))) uint16_t bs3[MOE_TOKEN_STAGES > 3 ? BM * 64 : 8];
  __shared__ float tok_scale[BM][kF8MaxKB + 1];   // +1: the 32 rows of a read hit 32 banks
  __shared__ float w_scale[kThreads / kWave][2][kF8MaxKB];
  __shared__ float red[kThreads / kWave][BM];

  Tile tl;
  if (!decode_tile(args, BM, tl)) return;
  const GemmSet& a = args.s[tl.set];
  const int tid = threadIdx.x, l = lane_id(), w = wave_id(), g = l >> 5, r32 = l & 31;
  const int ntf = (tl.mvalid + 31) >> 5;
  const int nkb = a.kdim / 128;

  // this wave's 32-row fragment of the tiled weights (32 x 128 codes per stage)
  const int rb = tl.nblk * 8 + w;
  const int nrow0 = MODE == kGateUp ? 16 * rb : 32 * rb;
  const bool wvalid = nrow0 < a.n;
  const int rbv = wvalid ? rb : 0;
  constexpr int astage = 32 * 128, avs = 1024;
  const uint8_t* aptr = static_cast<const uint8_t*>(a.wa) + static_cast<size_t>(tl.e) * a.wstride +
                        static_cast<size_t>(rbv) * nkb * astage + 16 * l;
  const uint8_t* aps[1] = {aptr};

  // token tile scales (rows past the expert's end repeat its last row)
  for (int i = tid; i < BM * nkb; i += kThreads) {
    const int row = i / nkb, kb = i - row * nkb;
    const int p = tl.row0 + (row < tl.mvalid ? row : tl.mvalid - 1);
    const int src = a.act_rows ? max(a.act_rows[p], 0) / a.act_div : p;
    tok_scale[row][kb] = a.ascale[static_cast<size_t>(src) * nkb + kb];
  }
  // weights: gate/up waves share the tile's W1 and W3 blocks; a down wave's
  // 32 rows lie in one 128-row block
  if (l < nkb) {
    const int nbr = a.n / 128;
    const int blk = MODE == kGateUp ? tl.nblk : (32 * rbv) / 128;
    const size_t o = (static_cast<size_t>(tl.e) * nbr + blk) * nkb;
    const float* s1 = a.sa + o;
    const float* s3 = MODE == kGateUp ? a.sb + o : s1;
    w_scale[w][0][l] = s1[l];
    w_scale[w][1][l] = s3[l];
  }
  __syncthreads();

  f32x16 acc[NTF];
#pragma unroll
  for (int t = 0; t < NTF; ++t) acc[t] = f32x16{};
  // acc += block partial x scales; gate/up: elements 0..7 are W1 rows,
  // 8..15 W3 rows; down: one weight block per wave
  auto post = [&](auto ntc, int s, auto& blk) {
    constexpr int NT = decltype(ntc)::value;
    const float sw1 = w_scale[w][0][s], sw3 = w_scale[w][1][s];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const float st = tok_scale[32 * t + r32][s];
      const float c1 = st * sw1, c3 = st * sw3;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[t][e] = fmaf(blk[t][e], c1, acc[t][e]);
#pragma unroll
      for (int e = 8; e < 16; ++e) acc[t][e] = fmaf(blk[t][e], c3, acc[t][e]);
    }
  };

  const uint16_t* act = static_cast<const uint16_t*>(a.act);
  const int kdim16 = a.kdim / 2;                  // a row of codes in 16-bit units
  using ML = MainLoop<false, NSA, BM, true, 1, (BM <= 64)>;
  switch (ntf) {
#define MOE_NT_CASE(n) \
    case n: if constexpr (n <= NTF) ML::template run<n>(aps, act, tl.row0, a.act_rows, a.act_div, tl.mvalid, kdim16, astage, avs, bs0, bs1, bs2, bs3, acc, post); break;
    MOE_NT_CASE(1) MOE_NT_CASE(2) MOE_NT_CASE(3) MOE_NT_CASE(4)
#undef MOE_NT_CASE
    default: break;
  }

  if (MODE == kGateUp) {
    // every wave of a gate/up tile is valid (n % 128 == 0) and takes part in
    // the block-wide max-abs
    float hv[NTF][8];
#pragma unroll
    for (int t = 0; t < NTF; ++t) {
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          hv[t][4 * i + q] = silu(acc[t][4 * i + q]) * acc[t][4 * (i + 2) + q];
          m = fmaxf(m, fabsf(hv[t][4 * i + q]));
        }
      m = fmaxf(m, __shfl_xor(m, 32, kWave));
      if (g == 0) red[w][32 * t + r32] = m;
    }
    __syncthreads();
    uint8_t* hq = static_cast<uint8_t*>(a.h);
    const int nts = a.n / 128;
#pragma unroll
    for (int t = 0; t < NTF; ++t) {
      const int tok = 32 * t + r32;
      if (!(t < ntf && tok < tl.mvalid)) continue;
      float amax = red[0][tok];
#pragma unroll
      for (int ww = 1; ww < kThreads / kWave; ++ww) amax = fmaxf(amax, red[ww][tok]);
      const float sc = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
      const size_t row = static_cast<size_t>(tl.row0 + tok);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        uint32_t packed = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) packed |= f32_to_e4m3(__fdiv_rn(hv[t][4 * i + q], sc)) << (8 * q);
        *reinterpret_cast<uint32_t*>(hq + row * a.n + nrow0 + 8 * i + 4 * g) = packed;
      }
      if (w == 0 && g == 0) a.hscale[row * nts + tl.nblk] = sc;
    }
  } else {
    if (!wvalid) return;
    // every token column's slot and gate in two rounds of loads (as in
    // grouped_gemm_mfma's down epilogue)
    int slot_t[NTF];
    float gate_t[NTF];
#pragma unroll
    for (int t = 0; t < NTF; ++t) {
      const int tok = 32 * t + r32;
      const int p = tl.row0 + tok;
      const bool live = t < ntf && tok < tl.mvalid;
      slot_t[t] = !live ? -1 : (a.perm_slot ? a.perm_slot[p] : p);
    }
#pragma unroll
    for (int t = 0; t < NTF; ++t)
      gate_t[t] = (a.gate && slot_t[t] >= 0) ? a.gate[slot_t[t]] : 1.f;
#pragma unroll
    for (int t = 0; t < NTF; ++t) {
      const int slot = slot_t[t];
      if (slot < 0) continue;           // past the tile's rows, or a slot with no expert
      const float gv = gate_t[t];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = nrow0 + 8 * i + 4 * g;
        const size_t o = static_cast<size_t>(slot) * a.n + col;
        const float o0 = acc[t][4 * i] * gv, o1 = acc[t][4 * i + 1] * gv;
        const float o2 = acc[t][4 * i + 2] * gv, o3 = acc[t][4 * i + 3] * gv;
        if (a.out_f32) {
          *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + o) = f32x4{o0, o1, o2, o3};
        } else {
          u32x2 v;
          v.x = pack_bf16x2(o0, o1);
          v.y = pack_bf16x2(o2, o3);
          *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(a.out) + o) = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 activations and weights: LDS-tiled fp32 FMA (32 tokens x 32 columns
// per block, 4 outputs per thread, K in chunks of 32).
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void grouped_gemm_f32(GemmArgs args) {
  __shared__ float xs[kBMF32][33];
  __shared__ float ws1[kBNF32][33];
  __shared__ float ws3[kBNF32][33];
  Tile tl;
  if (!decode_tile(args, kBMF32, tl)) return;
  const GemmSet& a = args.s[tl.set];
  const int tid = threadIdx.x;
  const int tok = tid >> 3, c0 = (tid & 7) * 4;
  const int n0 = tl.nblk * kBNF32;
  const float* act = static_cast<const float*>(a.act);
  const float* wa = static_cast<const float*>(a.wa) + static_cast<size_t>(tl.e) * a.wstride;
  const float* wb = MODE == kGateUp ? static_cast<const float*>(a.wb) + static_cast<size_t>(tl.e) * a.wstride : nullptr;
  float acc1[4] = {0.f, 0.f, 0.f, 0.f}, acc3[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < a.kdim; k0 += 32) {
    for (int i = tid; i < 32 * 32; i += 256) {
      const int r = i >> 5, c = i & 31;
      const int src = r < tl.mvalid ? (a.act_rows ? max(a.act_rows[tl.row0 + r], 0) / a.act_div
                                                  : tl.row0 + r) : 0;
      xs[r][c] = r < tl.mvalid ? act[static_cast<size_t>(src) * a.kdim + k0 + c] : 0.f;
      const int wr = n0 + r;
      ws1[r][c] = wr < a.n ? wa[static_cast<size_t>(wr) * a.kdim + k0 + c] : 0.f;
      if (MODE == kGateUp) ws3[r][c] = wr < a.n ? wb[static_cast<size_t>(wr) * a.kdim + k0 + c] : 0.f;
    }
    __syncthreads();
    for (int k = 0; k < 32; ++k) {
      const float xv = xs[tok][k];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        acc1[q] = fmaf(xv, ws1[c0 + q][k], acc1[q]);
        if (MODE == kGateUp) acc3[q] = fmaf(xv, ws3[c0 + q][k], acc3[q]);
      }
    }
    __syncthreads();
  }
  if (tok >= tl.mvalid) return;
  const int p = tl.row0 + tok;
  if (MODE == kGateUp) {
    float* h = static_cast<float*>(a.h);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = n0 + c0 + q;
      if (col < a.n) h[static_cast<size_t>(p) * a.n + col] = silu(acc1[q]) * acc3[q];
    }
  } else {
    const int slot = a.perm_slot ? a.perm_slot[p] : p;
    if (slot < 0) return;
    const float gv = a.gate ? a.gate[slot] : 1.f;
    float* out = static_cast<float*>(a.out);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int col = n0 + c0 + q;
      if (col < a.n) out[static_cast<size_t>(slot) * a.n + col] = acc1[q] * gv;
    }
  }
}

// Estimated cost of a tile, in K stages times (kStageWeight + token
// fragments): each stage streams the tile's weight rows whatever its token
// count, then runs one MFMA chain per 32-token fragment. Measured at the V3
// prefill shape, a one-fragment tile took 105 us (gate/up) and 34 us (down)
// against 184 and 72 us for eight fragments; 7 sits between the two.
constexpr int kStageWeight = 7;

// One grouped launch's tile table: its routed set's nb weight blocks per
// token tile and nk K stages, its shared set's nbs and nks (nbs = 0: no
// shared set), the blocks each XCD has in the launch (cap), and where the
// table goes: out[e] = the first routed tile of expert e, out[E] = routed
// tiles, then out[E + 1 + x] (x = 0 .. kNumXcd) = the first tile of XCD x's
// range in the launch's sequence (shared tiles first, then routed).
struct SchedSpec {
  int nb, nk, nbs, nks, cap;
  int32_t* out;
};

// Token tiles of an expert with m rows (split as decode_set_tile does) and
// the cost of one weight block over all of them, in the units above.
__device__ __forceinline__ void tile_row_cost(int m, int bm, int& mt, int& ntf, int& cost) {
  mt = (m + bm - 1) / bm;
  ntf = 0;
  cost = 0;
  if (mt == 0) return;
  const int per = (((m + mt - 1) / mt) + 31) & ~31;
  ntf = per / 32;
  const int ntl = (m - (mt - 1) * per + 31) / 32;
  cost = (mt - 1) * (kStageWeight + ntf) + (kStageWeight + ntl);
}

// Tile tables of up to two grouped launches over the same expert rows (one
// block; E <= 256): per expert its first tile, and the launch's tiles cut
// into kNumXcd contiguous ranges of about equal estimated cost, so that no
// XCD is left with more work than the others (the blocks of an XCD take its
// range in order). A range never exceeds the blocks an XCD has in the
// launch, so every tile is covered.
__global__ __launch_bounds__(256) void ffn_schedule(const int32_t* __restrict__ offsets, int E,
                                                    int bm, int T, SchedSpec s1, SchedSpec s2) {
  __shared__ int mt_[256], ntf_[256], rc_[256], before_[256];
  __shared__ long long csum[256];
  __shared__ int bound[kNumXcd + 1];
  const int tid = threadIdx.x;
  int mt = 0, ntf = 0, rc = 0;
  if (tid < E) tile_row_cost(offsets[tid + 1] - offsets[tid], bm, mt, ntf, rc);
  mt_[tid] = mt;
  ntf_[tid] = ntf;
  rc_[tid] = rc;
  before_[tid] = mt;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {   // inclusive scan of token tiles
    const int v = tid >= o ? before_[tid - o] : 0;
    __syncthreads();
    before_[tid] += v;
    __syncthreads();
  }
  const int all_mt = before_[255];
  __syncthreads();                      // every thread has read the total before it changes
  before_[tid] -= mt;                   // token tiles of the experts before this one
  __syncthreads();
  int mts = 0, ntfs = 0, rcs = 0;
  tile_row_cost(T, bm, mts, ntfs, rcs);
  for (int k = 0; k < 2; ++k) {
    const SchedSpec& sp = k == 0 ? s1 : s2;
    if (!sp.out) break;
    if (tid < E) sp.out[tid] = before_[tid] * sp.nb;
    if (tid == 0) sp.out[E] = all_mt * sp.nb;
    csum[tid] = static_cast<long long>(sp.nb) * rc * sp.nk;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {  // inclusive scan of expert costs
      const long long v = tid >= o ? csum[tid - o] : 0;
      __syncthreads();
      csum[tid] += v;
      __syncthreads();
    }
    const int n_sh = sp.nbs > 0 ? mts * sp.nbs : 0;
    const long long c_sh = sp.nbs > 0 ? static_cast<long long>(sp.nbs) * rcs * sp.nks : 0;
    const int n_all = n_sh + all_mt * sp.nb;
    const long long c_all = c_sh + csum[255];
    if (tid >= 1 && tid < kNumXcd) {
      const long long tau = c_all * tid / kNumXcd;
      int bx;
      if (tau < c_sh) {
        bx = static_cast<int>(tau * n_sh / c_sh);        // shared tiles cost about the same
      } else {
        const long long r = tau - c_sh;
        int lo = 0, hi = E - 1;                          // first expert whose inclusive cost > r
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if (csum[mid] > r) hi = mid; else lo = mid + 1;
        }
        const int e = lo;
        const long long q = r - (e > 0 ? csum[e - 1] : 0);
        const long long row = static_cast<long long>(rc_[e]) * sp.nk;
        int rows = row > 0 ? static_cast<int>(q / row) : 0;
        rows = min(rows, sp.nb - 1);
        const long long rem = q - rows * row;
        const long long stc = static_cast<long long>(kStageWeight + ntf_[e]) * sp.nk;
        const int j = max(0, min(mt_[e] - 1, static_cast<int>(stc > 0 ? rem / stc : 0)));
        bx = n_sh + before_[e] * sp.nb + rows * mt_[e] + j;
      }
      bound[tid] = bx;
    }
    __syncthreads();
    if (tid == 0) {
      int prev = 0;
      sp.out[E + 1] = 0;
      for (int x = 1; x < kNumXcd; ++x) {
        const int lo = max(prev, n_all - (kNumXcd - x) * sp.cap);
        const int hi = min(prev + sp.cap, n_all);
        const int bx = min(max(bound[x], lo), hi);
        sp.out[E + 1 + x] = bx;
        prev = bx;
      }
      sp.out[E + 1 + kNumXcd] = n_all;
    }
    __syncthreads();
  }
}

// Rows -> tiled weight layout (a pure relocation of 16-byte pieces).
// Tiled matrix of a group: R rows x C columns (R % 32 == 0, C % 64 == 0),
// cut into tiles of 32 rows x 64 columns, tile (rb, ks) at index rb*C/64+ks,
// each AW*1024 bytes (AW = 64 * wbytes / 32). Piece v of lane l in a tile
// holds row 32rb + l%32, columns 64ks + 32(l/32) + v*(16/wbytes) onwards,
// at byte v*1024 + 16l. interleave: row 32rb + r of the tiled matrix is
// row 16rb + r of `a` for r < 16 and row 16rb + r - 16 of `b` otherwise
// (gate and up rows of the same 16 intermediate columns in one tile);
// else it is row 32rb + r of `a`.
__global__ __launch_bounds__(256) void pack_tiles(const uint8_t* __restrict__ a,
                                                  const uint8_t* __restrict__ b,
                                                  uint8_t* __restrict__ dst, int64_t groups,
                                                  int rows_out, int cols, int wbytes,
                                                  int interleave) {
  const int aw = 64 * wbytes / 32;
  const int nk = cols / 64;
  const int64_t row_bytes = static_cast<int64_t>(cols) * wbytes;
  const int64_t src_group = static_cast<int64_t>(interleave ? rows_out / 2 : rows_out) * row_bytes;
  const int64_t per_group = static_cast<int64_t>(rows_out) * row_bytes / 16;
  const int64_t total = groups * per_group;
  for (int64_t o = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; o < total;
       o += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t e = o / per_group, local = o % per_group;
    const int64_t tile = local / (aw * 64);
    const int within = static_cast<int>(local % (aw * 64));
    const int v = within / 64, lane = within % 64;
    const int rb = static_cast<int>(tile / nk), ks = static_cast<int>(tile % nk);
    const int rr = lane % 32, gg = lane / 32;
    const uint8_t* src;
    int64_t row;
    if (interleave) {
      src = rr < 16 ? a : b;
      row = 16LL * rb + (rr & 15);
    } else {
      src = a;
      row = 32LL * rb + rr;
    }
    const int64_t col_byte = (64LL * ks + 32 * gg) * wbytes + 16LL * v;
    const u32x4 val = *reinterpret_cast<const u32x4*>(src + e * src_group + row * row_bytes + col_byte);
    *reinterpret_cast<u32x4*>(dst + o * 16) = val;
  }
}

// Blocks of a grouped launch whose sets have at most n0 and n1 tiles: every
// XCD takes up to ceil(n0 / 8) + ceil(n1 / 8) of them (see decode_tile).
int64_t grid_for(int64_t n0, int64_t n1 = 0) {
  return kNumXcd * ((n0 + kNumXcd - 1) / kNumXcd + (n1 + kNumXcd - 1) / kNumXcd);
}

// Token-tile size for a group: the smallest of 32 / 64 / 128 / 256 that covers
// the expected rows per expert (decode-like groups stream weights with one
// token fragment; prefill groups amortise each weight tile over up to 256
// tokens, which halves the L2-to-CU bytes per MFMA against 128).
#ifndef MOE_MAX_BM
#define MOE_MAX_BM 256
#endif
int pick_bm(int64_t rows_per_group) {
  if (rows_per_group <= 32) return 32;
  if (rows_per_group <= 64) return 64;
  if (rows_per_group <= 128 || MOE_MAX_BM == 128) return 128;
  return 256;
}

// Build-time knobs: depth (K stages) of the weight register ring of the
// 128/256-token kernels (MOE_NS_BIG) and of the 32-token ones
// (MOE_NS_SMALL); 3 measured best or equal (2 is 12 % slower at two
// fragments per wave; deeper rings change nothing for decode, and do not
// fit the registers of the 256-token tiles).
template <int MODE, bool FP8>
void launch_mfma(int bm, dim3 gd, hipStream_t s, const GemmArgs& a) {
#ifndef MOE_NS_BIG
#define MOE_NS_BIG 3
#endif
#ifndef MOE_NS_SMALL
#define MOE_NS_SMALL 3
#endif
  constexpr int NS_BIG = MOE_NS_BIG;
  constexpr int NS_SMALL = MOE_NS_SMALL;
#ifndef MOE_RF
#define MOE_RF 2
#endif
  // Weight fragments per wave of the 128/256-token kernels: 2 (4 waves, one
  // per SIMD) measured 5 % faster on the V3-shape gate/up launch than 1
  // (8 waves, two per SIMD), 3 % on the layer.
  constexpr int RF = MOE_RF;
  switch (bm) {
    case 32: hipLaunchKernelGGL((grouped_gemm_mfma<MODE, FP8, 32, NS_SMALL>), gd, dim3(kThreads), 0, s, a); break;
    case 64: hipLaunchKernelGGL((grouped_gemm_mfma<MODE, FP8, 64, NS_SMALL>), gd, dim3(kThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL((grouped_gemm_mfma<MODE, FP8, 128, NS_BIG, RF>), gd, dim3(kThreads / RF), 0, s, a); break;
    default: hipLaunchKernelGGL((grouped_gemm_mfma<MODE, FP8, 256, NS_BIG, RF>), gd, dim3(kThreads / RF), 0, s, a); break;
  }
}

// n0, n1: bounds on the tiles of the launch's first and second set.
hipError_t run_gemm(int mode, bool f32, bool fp8, int bm, const GemmArgs& a, int64_t n0,
                    int64_t n1, hipStream_t s) {
  const int64_t grid = grid_for(n0, n1);
  if (grid <= 0) return hipSuccess;
  const dim3 gd(static_cast<unsigned>(grid)), bd(256);
  if (f32) {
    if (mode == kGateUp) hipLaunchKernelGGL(grouped_gemm_f32<kGateUp>, gd, bd, 0, s, a);
    else hipLaunchKernelGGL(grouped_gemm_f32<kDown>, gd, bd, 0, s, a);
  } else if (fp8) {
    if (mode == kGateUp) launch_mfma<kGateUp, true>(bm, gd, s, a);
    else launch_mfma<kDown, true>(bm, gd, s, a);
  } else {
    if (mode == kGateUp) launch_mfma<kGateUp, false>(bm, gd, s, a);
    else launch_mfma<kDown, false>(bm, gd, s, a);
  }
  return hipGetLastError();
}

struct Blocking {
  int bm, nb1, nb2;
};

// rows_per_group: expected rows per expert (T*K/E routed, T shared)
Blocking blocking(const moe_config& c, int n_inter, int64_t rows_per_group) {
  if (c.act_dtype == MOE_DTYPE_F32)
    return {kBMF32, (n_inter + kBNF32 - 1) / kBNF32, (c.hidden + kBNF32 - 1) / kBNF32};
  return {pick_bm(rows_per_group), (n_inter + kBNGate - 1) / kBNGate, (c.hidden + kBNDown - 1) / kBNDown};
}

size_t elem_bytes(const moe_config& c) { return c.act_dtype == MOE_DTYPE_F32 ? 4 : 2; }

bool is_f32(const moe_config& c) { return c.act_dtype == MOE_DTYPE_F32; }
bool is_fp8(const moe_config& c) { return c.weight_dtype == MOE_DTYPE_FP8_E4M3; }
int tiled(const moe_config& c) { return c.weight_layout == MOE_LAYOUT_TILED; }

// The routed experts' gate/up set: rows grouped by expert; token rows read
// through act_rows (x and perm_slot) or directly (x_perm, act_rows null).
GemmSet routed_gate_up(const moe_config& c, const Blocking& b, const void* act,
                       const int32_t* act_rows, const int32_t* offsets, const int32_t* sched,
                       const void* w1, const void* w3, const float* s1, const float* s3, void* h) {
  GemmSet g{};
  g.act = act; g.act_rows = act_rows; g.act_div = c.top_k;
  g.wa = w1; g.wb = w3; g.sa = s1; g.sb = s3;
  g.offsets = offsets; g.sched = sched; g.fixed_m = 0; g.E = c.num_experts;
  g.kdim = c.hidden; g.n = c.inter; g.nb = b.nb1; g.h = h;
  g.tiled = tiled(c);
  g.wstride = static_cast<int64_t>(c.inter) * c.hidden * (g.tiled ? 2 : 1);
  return g;
}

GemmSet routed_down(const moe_config& c, const Blocking& b, const void* h, const int32_t* offsets,
                    const int32_t* sched, const int32_t* perm_slot, const float* gate,
                    const void* w2, const float* s2, void* out_slots) {
  GemmSet g{};
  g.act = h; g.wa = w2; g.sa = s2;
  g.offsets = offsets; g.sched = sched; g.fixed_m = 0; g.E = c.num_experts;
  g.kdim = c.inter; g.n = c.hidden; g.nb = b.nb2;
  g.wstride = static_cast<int64_t>(c.hidden) * c.inter;
  g.perm_slot = perm_slot; g.gate = gate; g.out = out_slots;
  g.out_f32 = c.slot_dtype == MOE_DTYPE_F32;
  g.tiled = tiled(c);
  return g;
}

GemmSet shared_gate_up(const moe_config& c, const Blocking& b, const void* x, const void* w1s,
                       const void* w3s, const float* s1s, const float* s3s, void* hs) {
  GemmSet g{};
  g.act = x; g.wa = w1s; g.wb = w3s; g.sa = s1s; g.sb = s3s;
  g.fixed_m = c.num_tokens; g.E = 1;
  g.kdim = c.hidden; g.n = c.num_shared * c.shared_inter; g.nb = b.nb1; g.h = hs;
  g.tiled = tiled(c);
  return g;
}

GemmSet shared_down(const moe_config& c, const Blocking& b, const void* hs, const void* w2s,
                    const float* s2s, void* y_shared) {
  GemmSet g{};
  g.act = hs; g.wa = w2s; g.sa = s2s;
  g.fixed_m = c.num_tokens; g.E = 1;
  g.kdim = c.num_shared * c.shared_inter; g.n = c.hidden; g.nb = b.nb2;
  g.out = y_shared; g.out_f32 = 1;
  g.tiled = tiled(c);
  return g;
}

hipError_t schedule(const int32_t* offsets, int E, int bm, int T, const SchedSpec& s1,
                    hipStream_t s, const SchedSpec& s2 = SchedSpec{0, 0, 0, 0, 0, nullptr}) {
  hipLaunchKernelGGL(ffn_schedule, dim3(1), dim3(256), 0, s, offsets, E, bm, T, s1, s2);
  return hipGetLastError();
}

// Blocks per XCD of a launch with at most n0 and n1 tiles in its two sets.
int xcd_cap(int64_t n0, int64_t n1) {
  return static_cast<int>((n0 + kNumXcd - 1) / kNumXcd + (n1 + kNumXcd - 1) / kNumXcd);
}

int64_t routed_max_tiles(const moe_config& c, int bm, int nb) {
  const int64_t TK = static_cast<int64_t>(c.num_tokens) * c.top_k;
  return ((TK + bm - 1) / bm + c.num_experts) * nb;
}

// The tiles of a grouped launch (the shared expert's first, when it has one;
// bs is then its blocking, with the routed token tile b.bm) and the spec of
// its tile table, which ffn_schedule writes to `sched`.
struct LaunchTiles {
  int64_t n_shared, n_routed;  // bounds on the tiles of the two sets
  SchedSpec spec;
};

LaunchTiles launch_tiles(const moe_config& c, const Blocking& b, const Blocking* bs, int mode,
                         int32_t* sched) {
  const int T = c.num_tokens, SI = c.num_shared * c.shared_inter;
  LaunchTiles l{};
  const int nb = mode == kGateUp ? b.nb1 : b.nb2;
  l.n_routed = routed_max_tiles(c, b.bm, nb);
  int nbs = 0;
  if (bs) {
    nbs = mode == kGateUp ? bs->nb1 : bs->nb2;
    l.n_shared = static_cast<int64_t>((T + b.bm - 1) / b.bm) * nbs;
  }
  const int nk = (mode == kGateUp ? c.hidden : c.inter) / 64;
  const int nks = (mode == kGateUp ? c.hidden : SI) / 64;
  l.spec = SchedSpec{nb, nk, nbs, nks, xcd_cap(l.n_shared, l.n_routed), sched};
  return l;
}

// ---- fine-grained fp8 (grouped_gemm_f8b) -----------------------------------

template <int MODE>
void launch_f8b_bm(int bm, dim3 gd, hipStream_t s, const GemmArgs& a) {
  switch (bm) {
    case 32: hipLaunchKernelGGL((grouped_gemm_f8b<MODE, 32, 3>), gd, dim3(kThreads), 0, s, a); break;
    case 64: hipLaunchKernelGGL((grouped_gemm_f8b<MODE, 64, 3>), gd, dim3(kThreads), 0, s, a); break;
    default: hipLaunchKernelGGL((grouped_gemm_f8b<MODE, 128, 3>), gd, dim3(kThreads), 0, s, a); break;
  }
}

hipError_t run_f8b(int mode, int bm, const GemmArgs& a, int64_t n0, int64_t n1, hipStream_t s) {
  const int64_t grid = grid_for(n0, n1);
  if (grid <= 0) return hipSuccess;
  const dim3 gd(static_cast<unsigned>(grid));
  if (mode == kGateUp) launch_f8b_bm<kGateUp>(bm, gd, s, a);
  else launch_f8b_bm<kDown>(bm, gd, s, a);
  return hipGetLastError();
}

// Token tiles of at most 128 rows (two sets of accumulators do not fit 256).
Blocking blocking_f8b(const moe_config& c, int n_inter, int64_t rows_per_group) {
  return {std::min(pick_bm(rows_per_group), 128), n_inter / 128, (c.hidden + kBNDown - 1) / kBNDown};
}

GemmSet f8b_gate_up(const moe_config& c, const Blocking& b, const void* xq, const float* xs,
                    const int32_t* act_rows, const int32_t* offsets, const int32_t* sched,
                    int n, int fixed_m, const void* w13, const float* s1, const float* s3,
                    void* hq, float* hs) {
  GemmSet g{};
  g.act = xq; g.ascale = xs; g.act_rows = act_rows; g.act_div = c.top_k;
  g.wa = w13; g.sa = s1; g.sb = s3;
  g.offsets = offsets; g.sched = sched; g.fixed_m = fixed_m; g.E = offsets ? c.num_experts : 1;
  g.kdim = c.hidden; g.n = n; g.nb = b.nb1; g.h = hq; g.hscale = hs;
  g.tiled = 1;
  g.wstride = 2LL * n * c.hidden;                // bytes of one expert's tiled gate/up tensor
  return g;
}

GemmSet f8b_down(const moe_config& c, const Blocking& b, const void* hq, const float* hs,
                 const int32_t* offsets, const int32_t* sched, int kdim, int fixed_m,
                 const int32_t* perm_slot, const float* gate, const void* w2, const float* s2,
                 void* out, int out_f32) {
  GemmSet g{};
  g.act = hq; g.ascale = hs;
  g.wa = w2; g.sa = s2;
  g.offsets = offsets; g.sched = sched; g.fixed_m = fixed_m; g.E = offsets ? c.num_experts : 1;
  g.kdim = kdim; g.n = c.hidden; g.nb = b.nb2;
  g.tiled = 1;
  g.wstride = static_cast<int64_t>(c.hidden) * kdim;
  g.perm_slot = perm_slot; g.gate = gate; g.out = out; g.out_f32 = out_f32;
  return g;
}

}  // namespace

// The largest tile count (= grid, up to a multiple of 8) of any grouped
// GEMM launch this configuration can make; tiles are indexed in int.
int64_t grouped_tiles_bound(const moe_config& c) {
  const int E = c.num_experts, T = c.num_tokens;
  const int64_t SI = static_cast<int64_t>(c.num_shared) * c.shared_inter;
  const int64_t TK = static_cast<int64_t>(T) * c.top_k;
  if (TK == 0) return 0;
  int64_t m = 0;
  for (int f8 = 0; f8 < 2; ++f8) {
    if (f8 && !(is_fp8(c) && SI <= 8192 && c.hidden % 128 == 0 && c.inter % 128 == 0)) continue;
    const Blocking b = f8 ? blocking_f8b(c, c.inter, (TK + E - 1) / E) : blocking(c, c.inter, (TK + E - 1) / E);
    const Blocking bs = f8 ? blocking_f8b(c, static_cast<int>(SI), T)
                           : blocking(c, static_cast<int>(std::min<int64_t>(SI, 1 << 30)), T);
    const int64_t mt = (T + b.bm - 1) / b.bm;
    const int64_t mts = (T + bs.bm - 1) / bs.bm;
    for (int down = 0; down < 2; ++down) {
      const int64_t nb = down ? b.nb2 : b.nb1, nbs = down ? bs.nb2 : bs.nb1;
      const int64_t routed = (TK / b.bm + E + 1) * nb;          // routed bound (as routed_max_tiles)
      const int64_t shared = c.num_shared > 0 ? std::max(mt * nbs, mts * nbs) : 0;
      m = std::max(m, grid_for(shared, routed));
    }
  }
  return m;
}

// The tile table of a grouped launch: E + 1 tile starts and the kNumXcd + 1
// XCD range starts.
size_t sched_ws_bytes(const moe_config& c) {
  return align_up(static_cast<size_t>(c.num_experts + 1 + kNumXcd + 1) * 4, 256);
}

size_t h_bytes(const moe_config& c) {
  return align_up(static_cast<size_t>(c.num_tokens) * c.top_k * c.inter * elem_bytes(c), 256);
}

size_t ffn_ws_bytes(const moe_config& c) { return h_bytes(c) + sched_ws_bytes(c); }

size_t shared_ws_bytes(const moe_config& c) {
  return align_up(static_cast<size_t>(c.num_tokens) * c.num_shared * c.shared_inter * elem_bytes(c), 256);
}

size_t experts_ws_bytes(const moe_config& c) {
  return h_bytes(c) + (c.num_shared > 0 ? shared_ws_bytes(c) : 0) + 2 * sched_ws_bytes(c);
}

hipError_t launch_gate_up(const moe_config& c, const void* x_perm, const int32_t* expert_offsets,
                          const void* w1, const void* w3, const float* s1, const float* s3,
                          void* h, void* ws, hipStream_t s) {
  const int E = c.num_experts;
  const int64_t TK = static_cast<int64_t>(c.num_tokens) * c.top_k;
  if (TK == 0) return hipSuccess;
  const Blocking b = blocking(c, c.inter, (TK + E - 1) / E);
  int32_t* sched = static_cast<int32_t*>(ws);
  const LaunchTiles lt = launch_tiles(c, b, nullptr, kGateUp, sched);
  hipError_t err = schedule(expert_offsets, E, b.bm, c.num_tokens, lt.spec, s);
  if (err != hipSuccess) return err;
  GemmArgs a{};
  a.nsets = 1;
  a.s[0] = routed_gate_up(c, b, x_perm, nullptr, expert_offsets, sched, w1, w3, s1, s3, h);
  a.xb = sched + E + 1;
  return run_gemm(kGateUp, is_f32(c), is_fp8(c), b.bm, a, lt.n_routed, 0, s);
}

hipError_t launch_down(const moe_config& c, const void* h, const int32_t* expert_offsets,
                       const int32_t* perm_slot, const float* topk_gate, const void* w2,
                       const float* s2, void* out_slots, void* ws, hipStream_t s) {
  const int E = c.num_experts;
  const int64_t TK = static_cast<int64_t>(c.num_tokens) * c.top_k;
  if (TK == 0) return hipSuccess;
  const Blocking b = blocking(c, c.inter, (TK + E - 1) / E);
  int32_t* sched = static_cast<int32_t*>(ws);
  const LaunchTiles lt = launch_tiles(c, b, nullptr, kDown, sched);
  hipError_t err = schedule(expert_offsets, E, b.bm, c.num_tokens, lt.spec, s);
  if (err != hipSuccess) return err;
  GemmArgs a{};
  a.nsets = 1;
  a.s[0] = routed_down(c, b, h, expert_offsets, sched, perm_slot, topk_gate, w2, s2, out_slots);
  a.xb = sched + E + 1;
  return run_gemm(kDown, is_f32(c), is_fp8(c), b.bm, a, lt.n_routed, 0, s);
}

hipError_t launch_expert_ffn(const moe_config& c, const void* x_perm,
                             const int32_t* expert_offsets, const int32_t* perm_slot,
                             const float* topk_gate, const void* w1, const void* w3,
                             const void* w2, const float* s1, const float* s3, const float* s2,
                             void* out_slots, void* ws, hipStream_t s) {
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  void* h = wsb;
  void* sched = wsb + h_bytes(c);
  hipError_t err = launch_gate_up(c, x_perm, expert_offsets, w1, w3, s1, s3, h, sched, s);
  if (err != hipSuccess) return err;
  return launch_down(c, h, expert_offsets, perm_slot, topk_gate, w2, s2, out_slots, sched, s);
}

hipError_t launch_shared_ffn(const moe_config& c, const void* x, const void* w1s,
                             const void* w3s, const void* w2s, const float* s1s,
                             const float* s3s, const float* s2s, void* y_shared, void* ws,
                             hipStream_t s) {
  const int T = c.num_tokens, SI = c.num_shared * c.shared_inter;
  if (T == 0) return hipSuccess;
  const Blocking b = blocking(c, SI, T);
  const int64_t mt = (T + b.bm - 1) / b.bm;
  GemmArgs a1{};
  a1.nsets = 1;
  a1.s[0] = shared_gate_up(c, b, x, w1s, w3s, s1s, s3s, ws);
  hipError_t err = run_gemm(kGateUp, is_f32(c), is_fp8(c), b.bm, a1, mt * b.nb1, 0, s);
  if (err != hipSuccess) return err;
  GemmArgs a2{};
  a2.nsets = 1;
  a2.s[0] = shared_down(c, b, ws, w2s, s2s, y_shared);
  return run_gemm(kDown, is_f32(c), is_fp8(c), b.bm, a2, mt * b.nb2, 0, s);
}

// Shared and routed experts in one gate/up and one down launch (shared tiles
// first), the routed token rows read from x through perm_slot.
hipError_t launch_experts_gate_up(const moe_config& c, const void* x,
                                  const int32_t* expert_offsets, const int32_t* perm_slot,
                                  const void* w1, const void* w3, const float* s1,
                                  const float* s3, const void* w1s, const void* w3s,
                                  const float* s1s, const float* s3s, void* h, void* hs,
                                  void* ws, hipStream_t s, bool scheduled) {
  const int E = c.num_experts, T = c.num_tokens, SI = c.num_shared * c.shared_inter;
  const int64_t TK = static_cast<int64_t>(T) * c.top_k;
  if (TK == 0) return hipSuccess;
  const Blocking b = blocking(c, c.inter, (TK + E - 1) / E);
  int32_t* sched = static_cast<int32_t*>(ws);
  const Blocking bs = c.num_shared > 0 ? blocking(c, SI, T) : Blocking{};  // its nb1 (token tile b.bm)
  const LaunchTiles lt = launch_tiles(c, b, c.num_shared > 0 ? &bs : nullptr, kGateUp, sched);
  hipError_t err = scheduled ? hipSuccess : schedule(expert_offsets, E, b.bm, T, lt.spec, s);
  if (err != hipSuccess) return err;
  GemmArgs a{};
  if (c.num_shared > 0) a.s[a.nsets++] = shared_gate_up(c, bs, x, w1s, w3s, s1s, s3s, hs);
  a.s[a.nsets++] = routed_gate_up(c, b, x, perm_slot, expert_offsets, sched, w1, w3, s1, s3, h);
  a.xb = sched + E + 1;
  return run_gemm(kGateUp, is_f32(c), is_fp8(c), b.bm, a, lt.n_shared, lt.n_routed, s);
}

hipError_t launch_experts_down(const moe_config& c, const void* h, const void* hs,
                               const int32_t* expert_offsets, const int32_t* perm_slot,
                               const float* topk_gate, const void* w2, const float* s2,
                               const void* w2s, const float* s2s, void* out_slots,
                               void* y_shared, void* ws, hipStream_t s, bool scheduled) {
  const int E = c.num_experts, T = c.num_tokens, SI = c.num_shared * c.shared_inter;
  const int64_t TK = static_cast<int64_t>(T) * c.top_k;
  if (TK == 0) return hipSuccess;
  const Blocking b = blocking(c, c.inter, (TK + E - 1) / E);
  int32_t* sched = static_cast<int32_t*>(ws);
  const Blocking bs = c.num_shared > 0 ? blocking(c, SI, T) : Blocking{};
  const LaunchTiles lt = launch_tiles(c, b, c.num_shared > 0 ? &bs : nullptr, kDown, sched);
  hipError_t err = scheduled ? hipSuccess : schedule(expert_offsets, E, b.bm, T, lt.spec, s);
  if (err != hipSuccess) return err;
  GemmArgs a{};
  if (c.num_shared > 0) a.s[a.nsets++] = shared_down(c, bs, hs, w2s, s2s, y_shared);
  a.s[a.nsets++] = routed_down(c, b, h, expert_offsets, sched, perm_slot, topk_gate, w2, s2,
                               out_slots);
  a.xb = sched + E + 1;
  return run_gemm(kDown, is_f32(c), is_fp8(c), b.bm, a, lt.n_shared, lt.n_routed, s);
}

hipError_t launch_experts(const moe_config& c, const void* x, const int32_t* expert_offsets,
                          const int32_t* perm_slot, const float* topk_gate, const void* w1,
                          const void* w3, const void* w2, const float* s1, const float* s3,
                          const float* s2, const void* w1s, const void* w3s, const void* w2s,
                          const float* s1s, const float* s3s, const float* s2s, void* out_slots,
                          void* y_shared, void* ws, hipStream_t s) {
  uint8_t* wsb = static_cast<uint8_t*>(ws);
  void* h = wsb;
  void* hs = c.num_shared > 0 ? wsb + h_bytes(c) : nullptr;
  uint8_t* sched_up = wsb + h_bytes(c) + (c.num_shared > 0 ? shared_ws_bytes(c) : 0);
  uint8_t* sched_down = sched_up + sched_ws_bytes(c);
  const int E = c.num_experts;
  const int64_t TK = static_cast<int64_t>(c.num_tokens) * c.top_k;
  if (TK == 0) return hipSuccess;
  // both launches' tile tables in one pass
  const Blocking b = blocking(c, c.inter, (TK + E - 1) / E);
  const int SI = c.num_shared * c.shared_inter;
  const Blocking bs = c.num_shared > 0 ? blocking(c, SI, c.num_tokens) : Blocking{};
  const Blocking* bsp = c.num_shared > 0 ? &bs : nullptr;
  const LaunchTiles up = launch_tiles(c, b, bsp, kGateUp, reinterpret_cast<int32_t*>(sched_up));
  const LaunchTiles down = launch_tiles(c, b, bsp, kDown, reinterpret_cast<int32_t*>(sched_down));
  hipError_t err = schedule(expert_offsets, E, b.bm, c.num_tokens, up.spec, s, down.spec);
  if (err != hipSuccess) return err;
  err = launch_experts_gate_up(c, x, expert_offsets, perm_slot, w1, w3, s1, s3, w1s, w3s, s1s, s3s,
                               h, hs, sched_up, s, true);
  if (err != hipSuccess) return err;
  return launch_experts_down(c, h, hs, expert_offsets, perm_slot, topk_gate, w2, s2, w2s, s2s,
                             out_slots, y_shared, sched_down, s, true);
}

// ---- fine-grained fp8 experts ------------------------------------------------

size_t hq_bytes(const moe_config& c) {
  return align_up(static_cast<size_t>(c.num_tokens) * c.top_k * c.inter, 256);
}
size_t hs_bytes(const moe_config& c) {
  return align_up(static_cast<size_t>(c.num_tokens) * c.top_k * (c.inter / 128) * 4, 256);
}
size_t hsq_bytes(const moe_config& c) {
  return align_up(static_cast<size_t>(c.num_tokens) * c.num_shared * c.shared_inter, 256);
}
size_t hss_bytes(const moe_config& c) {
  return align_up(static_cast<size_t>(c.num_tokens) * (c.num_shared * c.shared_inter / 128) * 4, 256);
}

size_t experts_fp8_ws_bytes(const moe_config& c) {
  size_t b = hq_bytes(c) + hs_bytes(c) + sched_ws_bytes(c);
  if (c.num_shared > 0) b += hsq_bytes(c) + hss_bytes(c);
  return b;
}

hipError_t launch_experts_fp8_gate_up(const moe_config& c, const void* xq, const float* xs,
                                      const int32_t* expert_offsets, const int32_t* perm_slot,
                                      const void* w13, const float* s1, const float* s3,
                                      const void* w13s, const float* s1s, const float* s3s,
                                      void* hq, float* hs, void* hsq, float* hss, void* ws,
                                      hipStream_t s) {
  const int E = c.num_experts, T = c.num_tokens, SI = c.num_shared * c.shared_inter;
  const int64_t TK = static_cast<int64_t>(T) * c.top_k;
  if (TK == 0) return hipSuccess;
  const Blocking b = blocking_f8b(c, c.inter, (TK + E - 1) / E);
  int32_t* sched = static_cast<int32_t*>(ws);
  const Blocking bs = c.num_shared > 0 ? blocking_f8b(c, SI, T) : Blocking{};
  const LaunchTiles lt = launch_tiles(c, b, c.num_shared > 0 ? &bs : nullptr, kGateUp, sched);
  hipError_t err = schedule(expert_offsets, E, b.bm, T, lt.spec, s);
  if (err != hipSuccess) return err;
  GemmArgs a{};
  if (c.num_shared > 0)
    a.s[a.nsets++] = f8b_gate_up(c, bs, xq, xs, nullptr, nullptr, nullptr, SI, T, w13s, s1s, s3s,
                                 hsq, hss);
  a.s[a.nsets++] = f8b_gate_up(c, b, xq, xs, perm_slot, expert_offsets, sched, c.inter, 0, w13,
                               s1, s3, hq, hs);
  a.xb = sched + E + 1;
  return run_f8b(kGateUp, b.bm, a, lt.n_shared, lt.n_routed, s);
}

hipError_t launch_experts_fp8_down(const moe_config& c, const void* hq, const float* hs,
                                   const void* hsq, const float* hss,
                                   const int32_t* expert_offsets, const int32_t* perm_slot,
                                   const float* topk_gate, const void* w2, const float* s2,
                                   const void* w2s, const float* s2s, void* out_slots,
                                   void* y_shared, void* ws, hipStream_t s) {
  const int E = c.num_experts, T = c.num_tokens, SI = c.num_shared * c.shared_inter;
  const int64_t TK = static_cast<int64_t>(T) * c.top_k;
  if (TK == 0) return hipSuccess;
  const Blocking b = blocking_f8b(c, c.inter, (TK + E - 1) / E);
  int32_t* sched = static_cast<int32_t*>(ws);
  const Blocking bs = c.num_shared > 0 ? blocking_f8b(c, SI, T) : Blocking{};
  const LaunchTiles lt = launch_tiles(c, b, c.num_shared > 0 ? &bs : nullptr, kDown, sched);
  hipError_t err = schedule(expert_offsets, E, b.bm, T, lt.spec, s);
  if (err != hipSuccess) return err;
  GemmArgs a{};
  if (c.num_shared > 0)
    a.s[a.nsets++] = f8b_down(c, bs, hsq, hss, nullptr, nullptr, SI, T, nullptr, nullptr, w2s, s2s,
                              y_shared, 1);
  a.s[a.nsets++] = f8b_down(c, b, hq, hs, expert_offsets, sched, c.inter, 0, perm_slot, topk_gate,
                            w2, s2, out_slots, c.slot_dtype == MOE_DTYPE_F32);
  a.xb = sched + E + 1;
  return run_f8b(kDown, b.bm, a, lt.n_shared, lt.n_routed, s);
}

hipError_t launch_experts_fp8(const moe_config& c, const void* xq, const float* xs,
                              const int32_t* expert_offsets, const int32_t* perm_slot,
                              const float* topk_gate, const void* w13, const void* w2,
                              const float* s1, const float* s3, const float* s2,
                              const void* w13s, const void* w2s, const float* s1s,
                              const float* s3s, const float* s2s, void* out_slots,
                              void* y_shared, void* ws, hipStream_t s) {
  uint8_t* p = static_cast<uint8_t*>(ws);
  void* hq = p;
  p += hq_bytes(c);
  float* hs = reinterpret_cast<float*>(p);
  p += hs_bytes(c);
  void* hsq = nullptr;
  float* hss = nullptr;
  if (c.num_shared > 0) {
    hsq = p;
    p += hsq_bytes(c);
    hss = reinterpret_cast<float*>(p);
    p += hss_bytes(c);
  }
  void* sched = p;
  hipError_t err = launch_experts_fp8_gate_up(c, xq, xs, expert_offsets, perm_slot, w13, s1, s3,
                                              w13s, s1s, s3s, hq, hs, hsq, hss, sched, s);
  if (err != hipSuccess) return err;
  return launch_experts_fp8_down(c, hq, hs, hsq, hss, expert_offsets, perm_slot, topk_gate, w2, s2,
                                 w2s, s2s, out_slots, y_shared, sched, s);
}

hipError_t launch_pack(int which, int64_t groups, int rows, int cols, int wbytes,
                       const void* a, const void* b, void* dst, hipStream_t s) {
  const int interleave = which == 0;
  const int rows_out = interleave ? 2 * rows : rows;
  const int64_t total = groups * rows_out * static_cast<int64_t>(cols) * wbytes / 16;
  if (total == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((total + 255) / 256, 8192);
  hipLaunchKernelGGL(pack_tiles, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const uint8_t*>(a), static_cast<const uint8_t*>(b),
                     static_cast<uint8_t*>(dst), groups, rows_out, cols, wbytes, interleave);
  return hipGetLastError();
}

}  // namespace moe
