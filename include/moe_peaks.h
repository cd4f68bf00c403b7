/* moe_peaks.h — achievable-peak probes for MI355X (gfx950), built as
 * libmoe_peaks.so beside libmoe.so.
 *
 * The DeepSeekMoE layer's kernels are measured against the part's published
 * peaks (HBM 8 TB/s; dense MFMA 2.5 PFLOP/s bf16, 5.0 PFLOP/s fp8) and
 * against what this GPU really sustains under the same conditions. These
 * probes measure the latter: a loop of independent MFMAs of one instruction
 * form (the rate the expert GEMMs could reach if they did nothing but
 * MFMAs), an fp32 FMA loop, and streaming read / copy kernels (the rate HBM
 * delivers to a kernel that only moves bytes). They compute nothing of the
 * layer. The caller times a call with HIP events on `stream` and divides the
 * work the call reports (moe_peak_mfma_flops, or the byte count) by it.
 *
 * Conventions as in libmoe.h: device pointers, caller-owned; calls are
 * asynchronous on `stream` (a hipStream_t, NULL = the null stream); return
 * codes MOE_OK / MOE_ERR_* from libmoe.h; arguments are checked on the host
 * before any launch (MOE_ERR_NULL, MOE_ERR_SHAPE), so a rejected call does
 * no device work.
 */
#ifndef MOE_PEAKS_H
#define MOE_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* MFMA / FMA loop forms */
#define MOE_PEAK_MFMA_BF16_32X32X16 0  /* v_mfma_f32_32x32x16_bf16 (the bf16 / fp8-row GEMMs)  */
#define MOE_PEAK_MFMA_BF16_16X16X32 1  /* v_mfma_f32_16x16x32_bf16 (the split-K router)         */
#define MOE_PEAK_MFMA_FP8_32X32X64  2  /* v_mfma_scale_f32_32x32x64_f8f6f4, E4M3 x E4M3         */
#define MOE_PEAK_MFMA_FP8_16X16X128 3  /* v_mfma_scale_f32_16x16x128_f8f6f4, E4M3 x E4M3        */
#define MOE_PEAK_FMA_F32            4  /* v_fma_f32 (the fp32 path; packed fp32 is not used)    */

/* Run `blocks` blocks of 512 threads (8 waves, as the expert GEMMs), each
 * wave issuing `iters` rounds of independent instructions of form `kind` on
 * finite pseudo-random operands (changing from one instruction to the next,
 * so operand buses toggle as with real data). Each thread writes one float
 * (a sum of its accumulators) to out[blocks * 512], which keeps the work
 * observable. MOE_ERR_SHAPE for an unknown kind, blocks < 1 or iters < 1;
 * MOE_ERR_NULL for out == NULL. */
int moe_peak_mfma(int kind, int32_t blocks, int32_t iters, float* out, void* stream);

/* Floating-point operations one moe_peak_mfma call with these arguments
 * performs (2 per multiply-add); 0 for invalid arguments. */
double moe_peak_mfma_flops(int kind, int32_t blocks, int32_t iters);

/* Read `bytes` bytes of src (bytes % 16 == 0, src 16-byte aligned) with
 * 16-byte loads: 32 KB chunks dealt grid-stride to `blocks` blocks of 256
 * threads, each thread with eight loads in flight per chunk. Thread i writes
 * the XOR of the 32-bit words it read to out[i] (out has blocks * 256
 * entries; the XOR of all of out is the XOR of every word of src). */
int moe_peak_stream_read(const void* src, size_t bytes, int32_t blocks, uint32_t* out,
                         void* stream);

/* moe_peak_stream_read with the non-temporal hint on every load, the form
 * the 32- and 64-token expert GEMMs use for their weights (same arguments,
 * same result in out). */
int moe_peak_stream_read_nt(const void* src, size_t bytes, int32_t blocks, uint32_t* out,
                            void* stream);

/* L2 -> CU read rate: block b re-reads its own region_bytes of src
 * (src + b * region_bytes; region_bytes a positive multiple of 64 KB, src
 * 16-byte aligned, blocks * region_bytes bytes readable) `iters` times with
 * 16-byte loads, 512 threads per block, eight loads in flight per thread.
 * A region larger than a CU's 32 KB L1 whose blocks' regions, summed per XCD
 * (blocks are dealt to the 8 XCDs in turn), fit its 4 MB L2 measures the L2
 * hit rate; thread i writes the XOR of the words it read to out[i] (out has
 * blocks * 512 entries). Bytes read = blocks * region_bytes * iters. */
int moe_peak_l2_read(const void* src, size_t region_bytes, int32_t blocks, int32_t iters,
                     uint32_t* out, void* stream);

/* dst[0 .. bytes) = src[0 .. bytes) with 16-byte loads and stores
 * (bytes % 16 == 0, both 16-byte aligned, no overlap), in the chunks of
 * moe_peak_stream_read. */
int moe_peak_stream_copy(const void* src, void* dst, size_t bytes, int32_t blocks, void* stream);

/* Accuracy of the fp8 MFMA the fine-grained fp8 GEMMs use
 * (v_mfma_scale_f32_32x32x64_f8f6f4 on E4M3 codes, unit scales): for each
 * of n problems p, D_p = A_p B_p^T + C_p with A_p = a[p] as [32 rows][64]
 * E4M3 codes, B_p = b[p] as [32 columns][64] codes (2048 bytes each), C_p =
 * c[p] and D_p = d[p] as [32][32] fp32, one instruction per problem. The
 * caller compares D with the exact sums: fp8 GEMM accumulation inside the
 * matrix unit keeps limited precision ("DeepSeekMoE架构解析" section 4.3,
 * the reason its scheme promotes partial sums to fp32 every 128 elements),
 * and the fine-grained fp8 parity check states the bound it assumes per
 * instruction. a, b 16-byte aligned; codes 0x7F / 0xFF (NaN) give
 * undefined results. MOE_ERR_NULL / MOE_ERR_SHAPE (n < 1, misaligned). */
int moe_probe_fp8_mfma(const void* a, const void* b, const float* c, float* d, int32_t n,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PEAKS_H */
