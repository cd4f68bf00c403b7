/*
 * libmoe -- the DeepSeekMoE layer forward pass on one AMD Instinct MI355X
 * (gfx950), as a C ABI.
 *
 * Sources of the method (web pages):
 *   [DSMoE]  "DeepSeekMoE架构解析：共享+路由专家协同与无丢弃门控设计" (jsqmd.com):
 *            section 1 (shared + fine-grained routed experts, no token
 *            dropping), section 2.1 (eqs. 13-15: sigmoid affinity, top-K,
 *            normalisation over the selected experts), section 2.2 (eq. 16
 *            and the bias update rule), section 3.1 (layer sketch: router
 *            weights, bias vector, gathered gate values, weighted sum).
 *   [V3ARCH] "DeepSeek-V3：MoE大模型架构" (aiqz.cc): section 路由机制 and its
 *            Python demo (selected scores divided by 1 + their sum).
 *   [COURSE] "省钱第一招：把一个大厨换成专家团" (blog.zero43.top): section 三
 *            (2 shared + 64 routed experts, 2+6 active), section 四 (the
 *            2024 gates are not renormalised), section 五 (bias outside the
 *            training objective), section 六 (no dropped tokens).
 *
 * Call sequence for one layer call (all on one stream, or the shared expert
 * on a second stream joined before moe_combine):
 *
 *   moe_route -> moe_permute -> moe_expert_ffn --+--> moe_combine
 *   moe_shared_ffn ------------------------------+
 *   (per batch, optionally) moe_bias_update
 *
 * or, with the routed and shared experts in one pair of grouped launches
 * that read the routed token rows straight from x (no gathered copy):
 *
 *   moe_route -> moe_permute (x_perm = NULL) -> moe_experts -> moe_combine
 *
 * Conventions shared by every call:
 *   - Every pointer except `cfg` and `status` strings is a DEVICE pointer to
 *     row-major contiguous memory that the caller owns and keeps alive until
 *     the enqueued work has finished. Every device pointer must be 16-byte
 *     aligned (hipMalloc and torch's allocator give 256): the kernels move
 *     rows in 16-byte pieces, and a misaligned pointer is rejected with
 *     MOE_ERR_SHAPE. The library allocates nothing, keeps
 *     no global state between calls and never synchronises the stream.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     call that returns an error has enqueued nothing. MOE_OK means
 *     "enqueued": device faults surface at the caller's next
 *     synchronisation.
 *   - num_tokens == 0 is a no-op that returns MOE_OK (for moe_route the
 *     load vector is still zeroed).
 *   - `stream` is a hipStream_t passed as void* (0 = the null stream).
 *   - Activations (x, x_perm, h) have the activation dtype of `cfg` (fp32 or
 *     bf16); the router weights have it too. The routed slot rows out_slots
 *     have cfg->slot_dtype (fp32 by default). The shared-expert
 *     output y_shared is always fp32 and the layer output y has
 *     cfg->out_dtype, so the sum of the shared and routed terms is formed
 *     and kept at fp32 accumulation precision. Expert weights have the weight dtype: fp32, bf16 (with
 *     bf16 activations) or fp8 E4M3 (OCP E4M3FN codes, with bf16
 *     activations) plus one fp32 scale per output row.
 *   - Inputs must be finite; results for non-finite inputs are undefined.
 *   - Calls on different streams with disjoint outputs may run concurrently.
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
#define MOE_OK               0
#define MOE_ERR_NULL         1  /* a required pointer is NULL                  */
#define MOE_ERR_SHAPE        2  /* sizes out of range or not supported          */
#define MOE_ERR_DTYPE        3  /* dtype enum unknown or combination invalid    */
#define MOE_ERR_UNSUPPORTED  4  /* valid request the library does not implement */
#define MOE_ERR_WORKSPACE    5  /* workspace NULL or smaller than required      */
#define MOE_ERR_HIP          6  /* the HIP runtime reported a launch error      */
#define MOE_ERR_SCRATCH      7  /* needs more than moe_permute_noalloc's fixed
                                   scratch array holds                         */

/* ---- enums --------------------------------------------------------------- */
#define MOE_SCORE_SIGMOID 0  /* s = sigmoid(u^T e_i), per expert ([DSMoE] eq. 15)          */
#define MOE_SCORE_SOFTMAX 1  /* s = softmax over all routed experts (2024 layout, [COURSE]) */

#define MOE_NORM_SELECTED 0  /* g = s / sum of the K selected s ([DSMoE] eq. 13)           */
#define MOE_NORM_NONE     1  /* g = s of the selected experts ([COURSE] section 四)        */
#define MOE_NORM_ONE_PLUS_SELECTED 2  /* g = s / (1 + sum of the K selected s) ([V3ARCH]
                                         section 路由机制 and its demo: the 1 is the shared expert) */

#define MOE_DTYPE_F32      0
#define MOE_DTYPE_BF16     1
#define MOE_DTYPE_FP8_E4M3 2  /* weights only */

#define MOE_LAYOUT_ROWS  0  /* expert weights row-major, as the shapes below state  */
#define MOE_LAYOUT_TILED 1  /* expert weights pre-tiled by moe_pack_weights          */

#define MOE_PACK_GATE_UP 0  /* W1 and W3 of each expert -> one tiled gate/up tensor */
#define MOE_PACK_DOWN    1  /* W2 of each expert -> one tiled tensor                */

#define MOE_WS_ROUTE   0
#define MOE_WS_PERMUTE 1
#define MOE_WS_FFN     2
#define MOE_WS_SHARED  3
#define MOE_WS_GEMM    4  /* moe_expert_gate_up / moe_expert_down */
#define MOE_WS_EXPERTS 5  /* moe_experts */
#define MOE_WS_EXPERTS_FP8 6  /* moe_experts_fp8 */

/* Layer shape and options. Limits (checked by moe_validate): num_tokens >= 0
 * with num_tokens * top_k < 2^30; 1 <= num_experts <=
 * 256; 1 <= top_k <= num_experts; hidden and inter are positive multiples
 * of 64; num_shared >= 0 and, when positive, num_shared * shared_inter is a
 * positive multiple of 64 (num_shared == 0 means no shared expert). A shape
 * whose grouped expert GEMMs would need more than 2^30 tiles in one launch
 * (tokens x hidden far beyond any one-GPU layer) gives MOE_ERR_UNSUPPORTED. */
typedef struct moe_config {
  int32_t num_tokens;    /* T: tokens in the batch                               */
  int32_t hidden;        /* d: hidden size                                       */
  int32_t num_experts;   /* E: routed experts                                    */
  int32_t top_k;         /* K: routed experts per token ([DSMoE] K_r)            */
  int32_t inter;         /* I: routed expert intermediate width                  */
  int32_t num_shared;    /* S: shared experts (always on, [DSMoE] section 1)     */
  int32_t shared_inter;  /* Is: intermediate width of each shared expert         */
  int32_t score_fn;      /* MOE_SCORE_*                                          */
  int32_t norm;          /* MOE_NORM_*                                           */
  int32_t act_dtype;     /* MOE_DTYPE_F32 or MOE_DTYPE_BF16                      */
  int32_t weight_dtype;  /* MOE_DTYPE_F32 (with f32 act), BF16 or FP8_E4M3 (bf16) */
  int32_t out_dtype;     /* layer output y: MOE_DTYPE_F32, or MOE_DTYPE_BF16 with
                            bf16 activations (then y carries one more bf16 rounding) */
  int32_t weight_layout; /* MOE_LAYOUT_ROWS, or MOE_LAYOUT_TILED (bf16 / fp8 weights):
                            the expert-FFN calls then take the moe_pack_weights
                            tensors -- w1 (w1s) = the tiled gate/up tensor, w3 (w3s)
                            = NULL, w2 (w2s) = the tiled down tensor; scales are
                            unchanged. Same results bit for bit; each weight load
                            then reads whole 1 KB stripes, which HBM serves faster
                            than the rows layout's 64-byte pieces of 32 rows. */
  int32_t num_groups;    /* G: node-limited routing ([DSMoE] section 2.3) when > 1: the
                            E experts form G groups of E/G consecutive experts; 0 or 1
                            = no group limit. Requires E % G == 0 and G <= 64.       */
  int32_t topk_groups;   /* M: groups kept per token (1..G, with M * E/G >= K); used
                            only when num_groups > 1.                                */
  int32_t slot_dtype;    /* the gate-weighted routed rows out_slots: MOE_DTYPE_F32
                            (0, the default: each routed term reaches the fp32 sum of
                            moe_combine unrounded), or MOE_DTYPE_BF16 with bf16
                            activations (half the bytes; each term then carries one
                            bf16 rounding, up to 2^-8 of itself, into the sum). */
} moe_config;

/* Validate a configuration without touching the GPU. Returns a status code. */
int moe_validate(const moe_config* cfg);

/* Bytes of workspace the call named by `which` (MOE_WS_*) needs for `cfg`,
 * or 0 if it needs none (or cfg is invalid). Workspaces need 256-byte
 * alignment and must not be shared by calls that may run concurrently. */
size_t moe_workspace_size(const moe_config* cfg, int which);

/* Human-readable name of a status code (static storage, never NULL). */
const char* moe_status_string(int status);

/* ---- moe_pack_weights -----------------------------------------------------
 * One-time relocation of expert weights into the tiled layout that the
 * expert-FFN calls read with MOE_LAYOUT_TILED (no arithmetic: every byte is
 * copied once, so results are identical to the rows layout).
 *   which = MOE_PACK_GATE_UP: src_a = W1, src_b = W3, each [groups, rows,
 *           cols]; dst holds 2 * groups * rows * cols weights. Tiled row
 *           32c + r (c = 0 .. rows/16 - 1) of group e is W1[e, 16c + r] for
 *           r < 16 and W3[e, 16c + r - 16] otherwise.
 *   which = MOE_PACK_DOWN:    src_a = W2 [groups, rows, cols], src_b = NULL;
 *           dst holds groups * rows * cols weights; tiled row i is W2[e, i].
 * Tiled layout of one group (R tiled rows, C = cols): tiles of 32 rows x 64
 * columns, tile (rb, ks) at byte offset (rb * C/64 + ks) * 2048 * wb (wb =
 * bytes per weight); inside a tile, the 16 bytes at offset v*1024 + 16*l
 * (l = 0..63, v = 0..32*wb/16 - 1) hold row 32rb + l%32, columns 64ks +
 * 32*(l/32) + v*16/wb onwards. Groups follow each other.
 * Routed experts: gate/up groups = E, rows = I, cols = d; down groups = E,
 * rows = d, cols = I. Shared experts: groups = 1, rows = S*Is, cols = d
 * (gate/up); rows = d, cols = S*Is (down).
 * weight_dtype MOE_DTYPE_BF16 or MOE_DTYPE_FP8_E4M3 (else MOE_ERR_DTYPE);
 * groups >= 1; rows a positive multiple of 32 (gate/up: of 16); cols a
 * positive multiple of 64 (else MOE_ERR_SHAPE); src and dst must not
 * overlap. */
int moe_pack_weights(int which, int32_t groups, int32_t rows, int32_t cols, int32_t weight_dtype,
                     const void* src_a, const void* src_b, void* dst, void* stream);

/* ---- moe_route ------------------------------------------------------------
 * Gating of [DSMoE] section 2.1 with the bias of section 2.2 (eq. 16):
 *   logits[t,i] = sum_j x[t,j] * w_router[i,j]          (u_t^T e_i)
 *   s[t,i]      = sigmoid(logits) or softmax_i(logits)  (cfg->score_fn)
 *   key[t,i]    = s[t,i] + bias[i]   (bias == NULL: key = s)
 *   topk_idx[t] = the K experts with the largest key, in key-descending
 *                 order, the lower expert index first among equal keys;
 *                 with num_groups = G > 1 ([DSMoE] section 2.3): group g =
 *                 experts g*E/G .. (g+1)*E/G - 1 has affinity sum_{i in g}
 *                 s[t,i] (scores, without the bias), the topk_groups groups
 *                 of largest affinity are kept (lower group index first
 *                 among equal sums) and the K experts are taken among theirs
 *   topk_gate[t,k] = s[t, topk_idx[t,k]] / sum_k' s[t, topk_idx[t,k']]
 *                 (MOE_NORM_SELECTED), s[t, topk_idx[t,k]] (MOE_NORM_NONE), or
 *                 s[t, topk_idx[t,k]] / (1 + sum_k' s[t, topk_idx[t,k']])
 *                 (MOE_NORM_ONE_PLUS_SELECTED);
 *                 the bias never enters the gate values
 *   load[i]     = number of (t, k) with topk_idx[t,k] == i (overwritten;
 *                 sums to T*K: no token is dropped)
 * x [T, d] act dtype; w_router [E, d] act dtype (row i = centroid e_i);
 * bias [E] fp32 or NULL; topk_idx [T, K] int32; topk_gate [T, K] fp32;
 * load [E] int32. Logits are accumulated in fp32; scores and keys are fp32.
 * Workspace: moe_workspace_size(cfg, MOE_WS_ROUTE) bytes (may be 0, then ws
 * may be NULL): the split-K partial logits (fp32 activations, or fewer than
 * 4096 tokens), or on the fused bf16 path with E a multiple of 32 a copy of
 * w_router that the call writes in the tiled layout of moe_pack_weights
 * (MOE_PACK_DOWN, one group) and reads instead, each weight load then being
 * one contiguous 1 KB stripe (a relocation only: results are unchanged).
 * The size for cfg also serves the same call with fewer tokens. */
int moe_route(const moe_config* cfg, const void* x, const void* w_router, const float* bias,
              int32_t* topk_idx, float* topk_gate, int32_t* load,
              void* ws, size_t ws_bytes, void* stream);

/* ---- moe_permute ----------------------------------------------------------
 * Groups the T*K (token, slot) pairs by expert for the grouped expert GEMMs
 * (the gather of [DSMoE] section 3.1), stable in token order. No pair is
 * dropped ([DSMoE] section 1): every selected (token, expert) gets a row.
 *   expert_offsets[e] = number of pairs with expert < e,  expert_offsets[E]
 *   = T*K; rows expert_offsets[e] .. expert_offsets[e+1]-1 hold, in
 *   increasing slot order, the slots f = t*K + k with topk_idx[t,k] == e;
 *   perm_slot[p] = the slot at row p;   x_perm[p, :] = x[perm_slot[p] / K, :]
 * The offsets are counted from topk_idx itself (they equal the exclusive
 * scan of moe_route's load vector). Entries of topk_idx outside [0, E) are
 * never produced by moe_route; if present they get no row, the last rows
 * get perm_slot = -1 and zero x_perm rows, and expert_offsets[E] < T*K.
 * topk_idx [T, K] int32; x [T, d] act dtype; expert_offsets [E+1] int32;
 * perm_slot [T*K] int32; x_perm [T*K, d] act dtype, or NULL to skip the row
 * gather (x is then not read and may be NULL; moe_experts reads the rows of
 * x through perm_slot itself). Integer results are exact. Workspace:
 * moe_workspace_size(cfg, MOE_WS_PERMUTE) bytes. */
int moe_permute(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                int32_t* expert_offsets, int32_t* perm_slot, void* x_perm,
                void* ws, size_t ws_bytes, void* stream);

/* ---- moe_permute_noalloc --------------------------------------------------
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation: moe_permute
 * with the same arguments, results and kernels, minus the workspace. The
 * counting sort's per-chunk histogram lives in a fixed 1 MiB device array
 * inside the library instead (each GPU the library runs on holds its own
 * copy until the process ends; its address is looked up once per device on
 * the first call there). That bounds the request to moe_workspace_size(cfg,
 * MOE_WS_PERMUTE) <= 1 MiB, i.e. ceil(T*K / 4096) * E <= 262144 (T*K up to
 * 4,194,304 pairs at E = 256); a larger one returns MOE_ERR_SCRATCH before
 * anything is enqueued. Nothing in the array needs clearing between calls
 * (every entry a call reads was written earlier in the same call), and the
 * call allocates nothing. Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (on different streams) race and must be
 * ordered by the caller. MOE_ERR_HIP if the device address cannot be
 * found. */
int moe_permute_noalloc(const moe_config* cfg, const int32_t* topk_idx, const void* x,
                        int32_t* expert_offsets, int32_t* perm_slot, void* x_perm,
                        void* stream);

/* ---- moe_expert_ffn -------------------------------------------------------
 * The routed SwiGLU experts ([DSMoE] section 1: fine-grained experts of
 * intermediate width I) on the grouped rows, weighted by their gates and
 * written back to their slots (the weighted sum's terms, [DSMoE] section 3.1):
 *   for row p of expert e, with slot f = perm_slot[p]:
 *     h = SiLU(W1_e x_perm[p]) * (W3_e x_perm[p])         (SiLU(z) = z*sigmoid(z))
 *     out_slots[f, :] = topk_gate[f] * (W2_e h)
 * w1, w3 [E, I, d]; w2 [E, d, I] in the weight dtype (MOE_LAYOUT_TILED:
 * w1 and w2 from moe_pack_weights, w3 = NULL). For fp8 weights s1, s3
 * [E, I] and s2 [E, d] are the fp32 scales of each output row (the stored
 * code times the scale is the weight); they must be NULL otherwise.
 * x_perm, expert_offsets, perm_slot from moe_permute; topk_gate [T*K] from
 * moe_route; out_slots [T*K, d] slot dtype. Accumulation is fp32; h is held
 * in the activation dtype. Workspace: MOE_WS_FFN bytes. */
int moe_expert_ffn(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                   const int32_t* perm_slot, const float* topk_gate,
                   const void* w1, const void* w3, const void* w2,
                   const float* s1, const float* s3, const float* s2,
                   void* out_slots, void* ws, size_t ws_bytes, void* stream);

/* ---- moe_expert_gate_up / moe_expert_down --------------------------------
 * The two halves of moe_expert_ffn, for callers that hold the intermediate
 * activations themselves (and to time each grouped GEMM on its own):
 *   moe_expert_gate_up: h[p, :] = SiLU(W1_e x_perm[p]) * (W3_e x_perm[p])
 *   moe_expert_down:    out_slots[perm_slot[p], :] = topk_gate[perm_slot[p]]
 *                                                    * (W2_e h[p])
 * for every row p of expert e. h [T*K, I] act dtype. Weights and scales as for
 * moe_expert_ffn (gate_up takes s1, s3; down takes s2). Workspace:
 * moe_workspace_size(cfg, MOE_WS_GEMM) bytes each. moe_expert_ffn is
 * exactly gate_up followed by down with h held in its workspace. */
int moe_expert_gate_up(const moe_config* cfg, const void* x_perm, const int32_t* expert_offsets,
                       const void* w1, const void* w3, const float* s1, const float* s3,
                       void* h, void* ws, size_t ws_bytes, void* stream);
int moe_expert_down(const moe_config* cfg, const void* h, const int32_t* expert_offsets,
                    const int32_t* perm_slot, const float* topk_gate, const void* w2,
                    const float* s2, void* out_slots, void* ws, size_t ws_bytes, void* stream);

/* ---- moe_shared_ffn -------------------------------------------------------
 * The always-on shared experts ([DSMoE] section 1; [COURSE] section 三) on
 * every token: y_shared[t] = sum_m W2s_m (SiLU(W1s_m x[t]) * (W3s_m x[t])).
 * The S experts are passed concatenated, which computes the same sum:
 * w1s, w3s [S*Is, d] (expert m = rows m*Is .. (m+1)*Is-1), w2s [d, S*Is]
 * (expert m = columns m*Is ..); MOE_LAYOUT_TILED: w1s and w2s packed with
 * groups = 1, w3s = NULL. fp8: s1s, s3s [S*Is] and s2s [d] row scales.
 * x [T, d] act dtype; y_shared [T, d] fp32. Requires num_shared > 0.
 * Workspace: MOE_WS_SHARED bytes. */
int moe_shared_ffn(const moe_config* cfg, const void* x, const void* w1s, const void* w3s,
                   const void* w2s, const float* s1s, const float* s3s, const float* s2s,
                   void* y_shared, void* ws, size_t ws_bytes, void* stream);

/* ---- moe_experts ----------------------------------------------------------
 * moe_expert_ffn and moe_shared_ffn together: one grouped gate/up launch and
 * one grouped down launch cover the shared experts' tiles and the routed
 * experts' tiles, so neither waits behind the other's tail. The routed rows
 * are read from x through perm_slot (row p of expert e is x[perm_slot[p] /
 * K]), so moe_permute need not write x_perm. Results are bit-identical to
 * moe_expert_ffn on the gathered rows followed by moe_shared_ffn.
 * x [T, d]; expert_offsets, perm_slot from moe_permute; topk_gate [T*K];
 * routed weights and scales as for moe_expert_ffn, shared ones as for
 * moe_shared_ffn (all NULL when num_shared == 0, y_shared too); out_slots
 * [T*K, d] slot dtype; y_shared [T, d] fp32. bf16 activations only
 * (MOE_ERR_DTYPE otherwise). Workspace: MOE_WS_EXPERTS bytes. */
int moe_experts(const moe_config* cfg, const void* x, const int32_t* expert_offsets,
                const int32_t* perm_slot, const float* topk_gate,
                const void* w1, const void* w3, const void* w2,
                const float* s1, const float* s3, const float* s2,
                const void* w1s, const void* w3s, const void* w2s,
                const float* s1s, const float* s3s, const float* s2s,
                void* out_slots, void* y_shared, void* ws, size_t ws_bytes, void* stream);

/* The two launches of moe_experts, for callers that hold the intermediate
 * activations themselves (and to time each grouped GEMM on its own):
 *   moe_experts_gate_up: h[p] = SiLU(W1_e x[perm_slot[p]/K]) * (W3_e ...) for
 *       the routed rows, hs[t] = SiLU(W1s x[t]) * (W3s x[t]) for the shared
 *       experts; h [T*K, I], hs [T, S*Is], both act dtype (hs NULL when
 *       num_shared == 0).
 *   moe_experts_down: out_slots[perm_slot[p]] = topk_gate[perm_slot[p]] *
 *       (W2_e h[p]) and y_shared[t] = W2s hs[t].
 * Arguments as for moe_experts. Workspace: MOE_WS_GEMM bytes each.
 * moe_experts is exactly gate_up followed by down with h, hs held in its
 * workspace. */
int moe_experts_gate_up(const moe_config* cfg, const void* x, const int32_t* expert_offsets,
                        const int32_t* perm_slot, const void* w1, const void* w3,
                        const float* s1, const float* s3, const void* w1s, const void* w3s,
                        const float* s1s, const float* s3s, void* h, void* hs,
                        void* ws, size_t ws_bytes, void* stream);
int moe_experts_down(const moe_config* cfg, const void* h, const void* hs,
                     const int32_t* expert_offsets, const int32_t* perm_slot,
                     const float* topk_gate, const void* w2, const float* s2, const void* w2s,
                     const float* s2s, void* out_slots, void* y_shared,
                     void* ws, size_t ws_bytes, void* stream);

/* ---- fine-grained fp8 experts ----------------------------------------------
 * The FP8 scheme of [DSMoE] section 4.3: weights quantised to OCP E4M3FN in
 * 128 x 128 blocks and activations in 1 x 128 tiles (one fp32 scale per
 * block / tile), products accumulated in fp32 with each 128-wide block of
 * the reduction multiplied by its two scales. Call sequence:
 *   moe_route (bf16 x) -> moe_permute (x_perm = NULL) -> moe_quantize_act
 *   -> moe_experts_fp8 (= moe_experts_fp8_gate_up + moe_experts_fp8_down)
 *   -> moe_combine
 * Requirements (else the status in brackets): bf16 activations and fp8
 * weights [MOE_ERR_DTYPE]; weight_layout MOE_LAYOUT_TILED, hidden, inter
 * and num_shared * shared_inter multiples of 128 [MOE_ERR_SHAPE], each at
 * most 8192 [MOE_ERR_UNSUPPORTED].
 *
 * moe_quantize_act: for each token t and tile j (channels 128j .. 128j+127):
 *   xs[t, j] = amax / 448 with amax = max |x[t, tile]| (fp32, rounded once;
 *   1 when amax = 0), xq[t, c] = the E4M3 code nearest to x[t, c] / xs[t, j]
 *   (fp32 division rounded once; ties to the even code; negative values
 *   that round to zero give the code 0x80). x [T, d] bf16, xq [T, d] codes
 *   (uint8), xs [T, d/128] fp32. Needs only act_dtype bf16 and d % 128 == 0.
 *
 * moe_experts_fp8: the routed and shared experts on the quantised tokens,
 * with the routed rows read through perm_slot like moe_experts:
 *   g = W1 x, u = W3 x (each 128-wide block of the reduction scaled by its
 *   weight-block and token-tile scales), h = SiLU(g) * u in fp32, h
 *   quantised in 1 x 128 tiles exactly as moe_quantize_act does, then
 *   W2 h the same way; routed rows times their gate go to out_slots [T*K, d]
 *   (slot dtype), the shared experts' sum to y_shared [T, d] (fp32).
 *   w13 / w13s: the MOE_PACK_GATE_UP tensors of W1, W3 (groups E / 1);
 *   w2 / w2s: the MOE_PACK_DOWN tensors; codes in both. Block scales (fp32):
 *   s1, s3 [E, I/128, d/128] of W1, W3 (block (i, j) covers rows 128i.. and
 *   columns 128j..), s2 [E, d/128, I/128] of W2; s1s, s3s [S*Is/128, d/128],
 *   s2s [d/128, S*Is/128] (all shared pointers NULL when num_shared == 0).
 *   Workspace: MOE_WS_EXPERTS_FP8 bytes (holds the quantised h).
 * moe_experts_fp8_gate_up / moe_experts_fp8_down: its two launches, with the
 *   quantised intermediate held by the caller: hq [T*K, I] codes and hs
 *   [T*K, I/128] fp32 (routed rows in expert order), hsq [T, S*Is] codes and
 *   hss [T, S*Is/128] (shared; NULL when num_shared == 0). Workspace:
 *   MOE_WS_GEMM bytes each. */
int moe_quantize_act(const moe_config* cfg, const void* x, void* xq, float* xs, void* stream);
int moe_experts_fp8(const moe_config* cfg, const void* xq, const float* xs,
                    const int32_t* expert_offsets, const int32_t* perm_slot,
                    const float* topk_gate, const void* w13, const void* w2,
                    const float* s1, const float* s3, const float* s2,
                    const void* w13s, const void* w2s, const float* s1s, const float* s3s,
                    const float* s2s, void* out_slots, void* y_shared,
                    void* ws, size_t ws_bytes, void* stream);
int moe_experts_fp8_gate_up(const moe_config* cfg, const void* xq, const float* xs,
                            const int32_t* expert_offsets, const int32_t* perm_slot,
                            const void* w13, const float* s1, const float* s3,
                            const void* w13s, const float* s1s, const float* s3s,
                            void* hq, float* hs, void* hsq, float* hss,
                            void* ws, size_t ws_bytes, void* stream);
int moe_experts_fp8_down(const moe_config* cfg, const void* hq, const float* hs,
                         const void* hsq, const float* hss, const int32_t* expert_offsets,
                         const int32_t* perm_slot, const float* topk_gate, const void* w2,
                         const float* s2, const void* w2s, const float* s2s, void* out_slots,
                         void* y_shared, void* ws, size_t ws_bytes, void* stream);

/* ---- moe_combine ----------------------------------------------------------
 * The layer output: shared experts plus the gate-weighted routed experts
 * ([DSMoE] section 1 and the weighted sum of section 3.1; no residual):
 *   y[t, :] = y_shared[t, :] + sum_{k=0..K-1} out_slots[t*K + k, :]
 * summed in fp32 in exactly this order (deterministic), rounded once to
 * cfg->out_dtype. y_shared may be NULL (then it counts as zero).
 * out_slots [T*K, d] slot dtype; y_shared [T, d] fp32; y [T, d] out_dtype. */
int moe_combine(const moe_config* cfg, const void* out_slots, const void* y_shared,
                void* y, void* stream);

/* ---- moe_rmsnorm / moe_combine_residual ------------------------------------
 * The steps either side of the layer ([DSMoE] section 4.1: an RMSNorm before
 * (and after) the MoE layer, eps 1e-6; section 2.1's eq. (12) adds the
 * layer's input to the expert sum). For a pre-norm layer:
 *   u = moe_rmsnorm(x)  ->  moe_route / moe_permute / moe_experts on u
 *   y = moe_combine_residual(out_slots, y_shared, x)
 * moe_rmsnorm: u[t, j] = x[t, j] / sqrt(mean_j' x[t, j']^2 + eps) * weight[j],
 *   computed in double precision
 *   (the sum of squares of bf16 inputs is then exact in any order, and every
 *   further step is one correctly rounded double operation) and rounded once
 *   to the activation dtype (round to nearest even). x, u [T, d] act dtype
 *   (u may be x); weight [d] fp32; eps > 0 and finite (the pages use 1e-6);
 *   d <= 16384 (bf16) or 8192 (fp32), else MOE_ERR_UNSUPPORTED.
 * moe_combine_residual: y[t] = residual[t] + y_shared[t] + sum_k
 *   out_slots[t*K + k], summed in fp32 in this order, rounded once to
 *   cfg->out_dtype. residual [T, d] act dtype; other arguments as for
 *   moe_combine (y_shared may be NULL). */
int moe_rmsnorm(const moe_config* cfg, const void* x, const float* weight, double eps, void* u,
                void* stream);
int moe_combine_residual(const moe_config* cfg, const void* out_slots, const void* y_shared,
                         const void* residual, void* y, void* stream);

/* ---- moe_sequence_loads ---------------------------------------------------
 * Per-sequence expert loads, the statistic behind a sequence-wise balance
 * check ([COURSE] section 五): the T tokens of the batch are taken as
 * consecutive sequences of seq_len tokens (the last may be shorter) and
 *   seq_load[q, e] = number of (t, k) with t in sequence q and topk_idx[t,k] == e
 * (ids outside [0, E) are not counted). topk_idx [T, K] int32 from moe_route;
 * seq_load [ceil(T / seq_len), E] int32, overwritten. seq_len >= 1.
 * Integer results are exact. */
int moe_sequence_loads(const moe_config* cfg, const int32_t* topk_idx, int32_t seq_len,
                       int32_t* seq_load, void* stream);

/* ---- moe_bias_update ------------------------------------------------------
 * Auxiliary-loss-free balance step of [DSMoE] section 2.2 ([COURSE] section
 * 五: applied after each batch, outside the gradient):
 *   bias[i] <- bias[i] - gamma * sign(load[i] - mean(load))
 * with mean(load) = sum(load)/E decided exactly in integers as
 * sign(load[i]*E - sum(load)); an expert exactly at the mean is unchanged.
 * The subtraction is one IEEE fp32 operation. load [E] int32, bias [E] fp32
 * in place; 1 <= num_experts <= 256; gamma finite and >= 0 (the pages use
 * 1e-3). */
int moe_bias_update(int32_t num_experts, const int32_t* load, float gamma, float* bias,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_H */
