/*
 * moe.h -- C ABI of the dropless mixture-of-experts expert layer for MI355X
 * (gfx950), library libmoe.so.
 *
 * The layer (page "NVIDIA Accelerates Dropless MoE Training in JAX Using
 * Transformer Engine", sections "What specialized optimizations are required
 * for dropless MoE?" with Figure 3, "Optimization 1: Grouped GEMM" and
 * "Optimization 2: Expert parallelism to integrate Dispatch and Combine"):
 *
 *   router top-K  ->  permute tokens into expert-contiguous rows (dispatch,
 *   local part)  ->  grouped GEMM of every expert's rows with its own gate/up
 *   weight, SwiGLU  ->  grouped GEMM with the down weight  ->  unpermute and
 *   combine by the routing weights.  Optionally the grouped GEMMs run on
 *   MXFP8 operands (E4M3 values, one E8M0 scale per 32 along K) produced by a
 *   group-aware quantiser.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers are DEVICE pointers (HBM) unless stated otherwise; the caller
 *    owns every buffer.  The library never allocates, frees, copies to the
 *    host or synchronises inside a call: each call only enqueues kernels on
 *    `stream` (a hipStream_t; NULL = the null stream) and returns.
 *  - Per-expert token counts (`group_sizes`) stay on the device; no entry
 *    point reads them on the host, and every launch grid depends only on host
 *    arguments, so each call may be captured in a hipGraph and replayed with
 *    new data (the page's requirement that kernels work when the shapes are
 *    not visible to the CPU, section "What specialized optimizations are
 *    required for dropless MoE?").
 *  - bf16 tensors are passed as uint16_t bit patterns, row-major.
 *  - Errors that the host can see (NULL required pointers, bad sizes,
 *    misalignment, too small workspace, unsupported combinations) return a
 *    status synchronously and enqueue nothing.  A launch failure returns
 *    MOE_ERR_HIP.  Errors in the DATA (an expert id outside [0,E), a
 *    negative group size, group sizes summing past the buffer) cannot be
 *    seen without a sync: kernels OR a MOE_FLAG_* bit into *err_flag (a
 *    device uint32; may be NULL) and clamp so that every access stays in
 *    bounds.  The caller polls the flag when it chooses.
 *  - Calls are thread-safe; calls on different streams may overlap.
 */
#ifndef DROPLESS_MOE_H
#define DROPLESS_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* NULL pointer, size out of range */
  MOE_ERR_UNSUPPORTED = 2, /* shape / dtype / layout combination not implemented */
  MOE_ERR_ALIGNMENT = 3,   /* a pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = 4,   /* workspace missing or too small */
  MOE_ERR_HIP = 5          /* the HIP runtime refused a launch */
} moe_status_t;

/* bits OR-ed into *err_flag by kernels */
#define MOE_FLAG_BAD_EXPERT_ID 0x1u  /* id outside [0,E): treated as E-1 */
#define MOE_FLAG_ROWS_OVER_CAP 0x2u  /* sum of group sizes > m_cap: rows past m_cap ignored */
#define MOE_FLAG_NEGATIVE_SIZE 0x4u  /* a group size < 0: treated as 0 */
#define MOE_FLAG_NAN_LOGIT     0x8u  /* NaN router logit: treated as -inf */

/* Version of this ABI (MOE_ABI_VERSION). */
int moe_abi_version(void);
/* Static text of a status code. */
const char* moe_status_string(int status);

/* ------------------------------------------------------------------------
 * Router top-K.  Blog intro: a learned router activates each token's Top-K
 * experts; ch. 1 of "AI Systems Performance Engineering", §4.1 worked
 * example: softmax = exponentials of (score - row max) over their sum.
 *
 * logits    fp32 [T, E]   router scores (bias already added)
 * topk_ids  int32 [T, K]  out: the K highest-scoring experts, in descending
 *                         score order; equal scores go to the lower index
 * topk_w    fp32 [T, K]   out: renormalize != 0: exp(l_k - max) / sum over
 *                         the K picks (they sum to 1); renormalize == 0: the
 *                         softmax over all E experts at the picks
 * Limits: 1 <= K <= min(E, 32), E <= 256, T >= 0.
 * ------------------------------------------------------------------------ */
moe_status_t moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t K, int32_t renormalize,
                            int32_t* topk_ids, float* topk_w, uint32_t* err_flag, void* stream);

/* ------------------------------------------------------------------------
 * Permute (dispatch, local part; blog section "Optimization 2": tokens are
 * reordered by expert).  A stable counting sort of the T*K (token, expert)
 * pairs, pair i = t*K + k:
 *   group_sizes[e]    = number of pairs routed to e                int32 [E]
 *   group_offsets[e]  = exclusive prefix sum; [E] = T*K            int32 [E+1]
 *   perm_dst[i]       = row of pair i in expert-contiguous order    int32 [T*K]
 *   perm_src[r]       = pair held by row r (inverse of perm_dst)    int32 [T*K]
 *   x_perm[r, :]      = x[perm_src[r] / K, :]                       bf16 [T*K, d]
 * Rows of one expert keep ascending token order.  The result does not
 * depend on thread timing (no atomics decide an order).  x / x_perm may both
 * be NULL to build the maps only.  ws: moe_permute_workspace_bytes(T,E,K)
 * bytes, 256-byte aligned, contents need not be initialised.
 * Limits: E <= 256, K <= 32, d % 8 == 0 when x is given.
 * ------------------------------------------------------------------------ */
size_t moe_permute_workspace_bytes(int64_t T, int32_t E, int32_t K);
moe_status_t moe_permute(const uint16_t* x, const int32_t* topk_ids, int64_t T, int32_t d, int32_t E, int32_t K,
                         int32_t* group_sizes, int32_t* group_offsets, int32_t* perm_src, int32_t* perm_dst,
                         uint16_t* x_perm, void* ws, size_t ws_bytes, uint32_t* err_flag, void* stream);

/* For callers that cannot allocate (code under hipGraph capture, tight
 * serving loops, harnesses that forbid hipMalloc): moe_permute with the
 * workspace taken from the library's own device memory, a static array of
 * MOE_PERMUTE_NOALLOC_SCRATCH_BYTES per GPU held until the process ends, so
 * the call allocates nothing and needs no ws argument.  Arguments, outputs
 * and limits as moe_permute; additionally moe_permute_workspace_bytes(T, E,
 * K) must not exceed MOE_PERMUTE_NOALLOC_SCRATCH_BYTES (8 MiB: T*K up to
 * 2^20 pairs with E = 256, about 2^21 with E = 8), else MOE_ERR_WORKSPACE is
 * returned and
 * nothing is enqueued.  The first call on a device looks up the array's
 * address there (MOE_ERR_HIP if that fails).  All calls on one GPU share the
 * array: calls that overlap on one GPU (several streams, or several graphs
 * replayed concurrently) race and give undefined results; calls ordered on
 * one stream do not. */
#define MOE_PERMUTE_NOALLOC_SCRATCH_BYTES ((size_t)8 << 20)
moe_status_t moe_permute_noalloc(const uint16_t* x, const int32_t* topk_ids, int64_t T, int32_t d, int32_t E,
                                 int32_t K, int32_t* group_sizes, int32_t* group_offsets, int32_t* perm_src,
                                 int32_t* perm_dst, uint16_t* x_perm, uint32_t* err_flag, void* stream);

/* Permute with MXFP8 output (the page's planned quantisation fused into the
 * dispatch, section "Optimization 1"): the same maps as moe_permute, and
 * instead of bf16 rows the E4M3 codes x_q uint8 [T*K, d] and E8M0 scales
 * x_scale uint8 [T*K, d/32] that mxfp8_group_quantize (axis 0) would produce
 * from moe_permute's x_perm, bit for bit; each token row is read and
 * quantised once.  x, x_q 16-byte aligned; d % 32 == 0; ws as moe_permute. */
moe_status_t moe_permute_mxfp8(const uint16_t* x, const int32_t* topk_ids, int64_t T, int32_t d, int32_t E,
                               int32_t K, int32_t* group_sizes, int32_t* group_offsets, int32_t* perm_src,
                               int32_t* perm_dst, uint8_t* x_q, uint8_t* x_scale, void* ws, size_t ws_bytes,
                               uint32_t* err_flag, void* stream);

/* ------------------------------------------------------------------------
 * Fused router (blog section "Optimization 2: Expert parallelism to
 * integrate Dispatch and Combine": the router runs as fused kernels right
 * before the dispatch; intro: a learned router picks each token's Top-K
 * experts).  One kernel computes
 *   logits[t, e] = sum_k x[t, k] * w_router[e, k]  (+ bias[e])   fp32 accumulation
 * and from them the same selection and weights as moe_route_topk (equal
 * logits go to the lower index; renormalize as there), and, when ws is
 * given, the dispatch histogram that moe_permute_routed consumes.
 *
 * x         bf16 [T, d]   tokens, 16-byte aligned
 * w_router  bf16 [E, d]   router weight, 16-byte aligned
 * bias      fp32 [E]      added to every token's logits; NULL: none
 * topk_ids  int32 [T, K], topk_w fp32 [T, K]   out, as moe_route_topk
 * logits    fp32 [T, E]   out if not NULL (16-byte aligned): the logits the
 *                         selection was made on (NaN already turned -inf)
 * ws        NULL, or moe_route_fused_workspace_bytes(T, E, K) bytes,
 *           256-byte aligned: receives each (token, expert) pair's rank among
 *           the earlier pairs of its token block with the same expert, and
 *           every block's per-expert counts.  Pass it unchanged to
 *           moe_permute_routed (same T, E, K).
 * Errors: MOE_FLAG_NAN_LOGIT in *err_flag for a NaN logit (taken as -inf).
 * Limits: 1 <= K <= min(E, 32), E <= 256, d % 32 == 0, d >= 32, T*K < 2^31.
 * ------------------------------------------------------------------------ */
size_t moe_route_fused_workspace_bytes(int64_t T, int32_t E, int32_t K);
moe_status_t moe_route_fused(const uint16_t* x, const uint16_t* w_router, const float* bias, int64_t T, int32_t d,
                             int32_t E, int32_t K, int32_t renormalize, int32_t* topk_ids, float* topk_w,
                             float* logits, void* ws, size_t ws_bytes, uint32_t* err_flag, void* stream);

/* Permute from the fused router's histogram: the outputs of moe_permute
 * (same definitions, bit for bit) for the ids moe_route_fused wrote, with
 * that call's ws (the rank pass is skipped; the ws contents are consumed:
 * pass a fresh moe_route_fused result each time).  Limits as moe_permute. */
moe_status_t moe_permute_routed(const uint16_t* x, const int32_t* topk_ids, int64_t T, int32_t d, int32_t E,
                                int32_t K, int32_t* group_sizes, int32_t* group_offsets, int32_t* perm_src,
                                int32_t* perm_dst, uint16_t* x_perm, void* ws, size_t ws_bytes, uint32_t* err_flag,
                                void* stream);

/* ------------------------------------------------------------------------
 * Grouped GEMM (blog section "Optimization 1: Grouped GEMM": all experts in
 * one call, each with its true token count, only rows with valid tokens
 * computed; counts on the device).  Group g owns rows [o_g, o_g + s_g) of the
 * ragged operand, o_g = s_0 + ... + s_{g-1}, s_g = group_sizes[g].
 *
 * ragged = MOE_RAGGED_M (forward and data gradient):
 *   C[r, n] = sum_k A[r, k] * Bop_g[k, n]   for rows r of group g
 *   A  [m_cap, K] (K contiguous);  B_NK: B [G, N, K] (Bop_g = B[g]^T);
 *   B_KN: B [G, K, N] (Bop_g = B[g]);  B_PACKED: B[g]^T of B_NK stored in
 *   the tile-stage layout written by moe_pack_weights (bf16) or
 *   moe_pack_weights_mxfp8 for the same G, N, K and epilogue.  Output
 *   C [m_cap, N] (out_dtype).
 *   epilogue MOE_EPI_SWIGLU (B_NK, bf16 only): N = 2f; with acc = A*Bop,
 *   C [m_cap, f] = bf16(silu(acc[:, j]) * acc[:, f + j]) (rows [0,f) of B[g]
 *   are the gate projection, rows [f,2f) the up projection: the prefused
 *   weight of the blog's MaxText config) and, if C_aux is not NULL,
 *   C_aux [m_cap, 2f] = bf16(acc) (the pre-activations, for the backward).
 *   Rows r >= sum(s_g) are not written.
 *   epilogue MOE_EPI_SWIGLU_BWD (B_KN, bf16 only: the data gradient of the
 *   down projection fused with SwiGLU's backward, so that dh is never
 *   written and read back; blog section "Optimization 2", data read and
 *   written to memory multiple times): N = f; with dh = bf16(A*Bop) and the
 *   forward's pre-activations C_aux [m_cap, 2f] = [g | u] (required, read
 *   only), C [m_cap, 2f] = [dg | du], dg = bf16(dh u s (1 + g (1 - s))),
 *   du = bf16(dh g s), s = 1 / (1 + e^-g), as moe_swiglu_backward computes
 *   them from the stored dh.  N <= 2^21.  Rows r >= sum(s_g) are not
 *   written.
 * ragged = MOE_RAGGED_K (weight gradient; contraction over a group's rows):
 *   C[g] [M, N] = sum over rows r of group g of A[r, m] * B[r, n];
 *   A [m_cap, M], B [m_cap, N] (both row-major).  Empty groups get zeros.
 *   Its workgroups take tiles from counters in the library's own device
 *   memory (64 slots handed out in turn, each call tagged with its own
 *   epoch: counts left in a slot by another call, one that ended part-way
 *   included, count as zero, and the call's last workgroup presets the slot
 *   for the slot's next call when it finishes), so up to 64 such calls may
 *   be in flight on one GPU at once; a captured call keeps its slot and
 *   epoch on every replay, so one graph must not be replayed on two streams
 *   concurrently.  A call of more than 2^22 output tiles (G ceil(M/256)
 *   ceil(N/256); an output that fits in memory has fewer) returns
 *   MOE_ERR_INVALID_ARG.  Each tile is computed by one
 *   workgroup in a fixed order: results are bitwise reproducible.
 *   dtype = MOE_DTYPE_MXFP8 (the group-aware MXFP8 weight gradient): A and
 *   B are the outputs of mxfp8_quantize_transposed (grouped) for the same
 *   group_sizes and m_cap: codes A [M, K], B [N, K] with scales A_scale
 *   [M, K/32], B_scale [N, K/32], where K is that call's k_cap; output bf16.
 *   The same 64 queue slots apply (a separate set).
 * dtype = MOE_DTYPE_MXFP8 (RAGGED_M, B_NK or B_PACKED): A, B are E4M3 codes
 *   with E8M0 scales A_scale [m_cap, K/32], B_scale [G, N, K/32] (value =
 *   code * 2^(scale - 127)); accumulation fp32, output bf16.  With
 *   B_PACKED, B comes from moe_pack_weights_mxfp8 (codes and scales
 *   together) and B_scale is ignored.
 *   epilogue MOE_EPI_SWIGLU_MXFP8 (MXFP8 only; the page's planned
 *   quantisation fused with the GEMM, section "Optimization 1"): as
 *   MOE_EPI_SWIGLU, and the bf16 h is then quantised exactly as
 *   mxfp8_group_quantize (axis 0) would quantise it: C receives the E4M3
 *   codes uint8 [m_cap, f], C_aux (required) the E8M0 scales uint8
 *   [m_cap, f/32]; f % 32 == 0; packed weights are those packed for
 *   MOE_EPI_SWIGLU.  Rows r >= sum(s_g) are not written.
 * ws: optional.  grouped_gemm_workspace_bytes(desc) is 0 except for bf16
 *   and MXFP8 RAGGED_M calls, where it is one fp32 256 x 256 tile per
 *   compute unit (64 MiB on MI355X).  Given that many bytes (256-byte
 *   aligned), a call of at least 64 K stages (K >= 2048 in bf16, K >= 4096
 *   in MXFP8) whose tiles fill at most three rounds of the grid even
 *   if every group ends in a partial tile (G + ceil(m_cap / 256) row tiles
 *   times the column tiles <= 3 x the workgroups) splits the tiles of its
 *   last round along K when that round holds at most half as many tiles as
 *   the grid has workgroups: each tile's K stages are cut into 2-4 equal
 *   ranges on different workgroups, whose fp32 partial sums meet in ws and
 *   are added in range order by the one that arrives last (the work of a
 *   short last round is shared instead of leaving most of the GPU idle;
 *   blog section "Optimization 1", full utilisation with irregular expert
 *   shapes).  The partition depends only on the group sizes, the grid and
 *   K, so results stay bitwise reproducible (and within a rounding of the
 *   unsplit sums); with ws NULL or smaller, nothing is split.  A call's
 *   arrival counters are library words handed out in 64 slots as for the
 *   weight gradients; calls in flight together must not share ws.
 * Limits: G <= 1024; N <= 2^22 (else MOE_ERR_UNSUPPORTED);
 *   bf16: K % 64 == 0 (RAGGED_M), N % 8 == 0, M % 8 == 0;
 *   MXFP8: K % 128 == 0 (RAGGED_M), K % 64 == 0 and K >= m_cap + 63 G
 *   (RAGGED_K).  A, B, C 16-byte aligned; scales 4-byte aligned.
 * dtype = MOE_DTYPE_MXFP4 (RAGGED_M, B_NK, bf16 out; the gfx950 analog of
 *   the blog's planned 4-bit format, closing of "Optimization 1"): A and B
 *   are E2M1 codes, two per byte (element 2i in the low nibble of byte i):
 *   A [m_cap, K/2], B [G, N, K/2]; A_scale [K/128, m_cap, 4] and
 *   B_scale [K/128, G*N, 4] are E8M0 scales of the 32-blocks along K,
 *   stage-major (the word of row r and 128-code stage t holds blocks 4t..4t+3),
 *   as mxfp4_quantize writes them.  Element value = code value * 2^(scale-127).
 *   epilogue MOE_EPI_NONE or MOE_EPI_SWIGLU (B rows [0,f) gate, [f,2f) up).
 *   K % 128 == 0, N % 8 == 0 (N/2 % 8 for SwiGLU); C_aux must be NULL.
 * ------------------------------------------------------------------------ */
#define MOE_DTYPE_BF16 0
#define MOE_DTYPE_MXFP8 1
#define MOE_DTYPE_MXFP4 2
#define MOE_RAGGED_M 0
#define MOE_RAGGED_K 1
#define MOE_B_NK 0
#define MOE_B_KN 1
#define MOE_B_PACKED 2
#define MOE_EPI_NONE 0
#define MOE_EPI_SWIGLU 1
#define MOE_EPI_SWIGLU_MXFP8 2
#define MOE_EPI_SWIGLU_BWD 3
#define MOE_OUT_BF16 0
#define MOE_OUT_F32 1

typedef struct moe_gg_desc {
  int32_t dtype;     /* MOE_DTYPE_* */
  int32_t ragged;    /* MOE_RAGGED_M | MOE_RAGGED_K */
  int32_t b_layout;  /* MOE_B_NK | MOE_B_KN | MOE_B_PACKED (RAGGED_M) */
  int32_t epilogue;  /* MOE_EPI_NONE | MOE_EPI_SWIGLU */
  int32_t out_dtype; /* MOE_OUT_BF16 | MOE_OUT_F32 */
  int32_t G;         /* number of groups */
  int32_t M;         /* RAGGED_K: rows of each C[g]; ignored for RAGGED_M */
  int32_t N;         /* output columns (before the SwiGLU epilogue halves them) */
  int32_t K;         /* RAGGED_M: contraction length; ignored for RAGGED_K */
  int64_t m_cap;     /* rows of the ragged operand(s); sum(group_sizes) <= m_cap */
} moe_gg_desc;

size_t grouped_gemm_workspace_bytes(const moe_gg_desc* desc);
moe_status_t grouped_gemm(const moe_gg_desc* desc, const void* A, const uint8_t* A_scale, const void* B,
                          const uint8_t* B_scale, const int32_t* group_sizes, void* C, void* C_aux, void* ws,
                          size_t ws_bytes, uint32_t* err_flag, void* stream);

/* Weight packing for the bf16 forward GEMM (the expert weights of the blog's
 * grouped GEMM, section "Optimization 1", are fixed between optimiser
 * steps, so their storage order is free): W bf16 [G, N, K] (the B_NK
 * operand; for epilogue MOE_EPI_SWIGLU the fused [gate; up] weight with
 * N = 2f) is rewritten into out, moe_pack_weights_bytes(G, N, K, epilogue)
 * bytes, 16-byte aligned, owned by the caller.  Every weight tile of every
 * K-step becomes one contiguous block in the order the GEMM loads it;
 * padding rows are zero.  The result is valid only as B of grouped_gemm with
 * b_layout MOE_B_PACKED and the same G, N, K and epilogue.  Limits as for
 * grouped_gemm (K % 64 == 0, N % 8 == 0, SwiGLU: (N/2) % 8 == 0). */
size_t moe_pack_weights_bytes(int32_t G, int32_t N, int32_t K, int32_t epilogue);
moe_status_t moe_pack_weights(const uint16_t* w, int32_t G, int32_t N, int32_t K, int32_t epilogue, void* out,
                              size_t out_bytes, void* stream);

/* The same for MXFP8 weights (blog: MXFP8 expert matmuls, section
 * "Optimization 1"; weights quantised once): codes q uint8 [G, N, K]
 * (16-byte aligned) and E8M0 scales uint8 [G, N, K/32] (2-byte aligned), as
 * written by mxfp8_group_quantize, are rewritten together into out
 * (moe_pack_weights_mxfp8_bytes(G, N, K, epilogue) bytes, 16-byte aligned,
 * caller-owned): per weight tile and 64-deep K-step the codes in load order,
 * then the scale bytes of that step.  Valid only as B of an MXFP8
 * grouped_gemm with b_layout MOE_B_PACKED and the same G, N, K, epilogue.
 * K % 128 == 0, N % 8 == 0 (SwiGLU: (N/2) % 8 == 0); 0 bytes = unsupported. */
size_t moe_pack_weights_mxfp8_bytes(int32_t G, int32_t N, int32_t K, int32_t epilogue);
moe_status_t moe_pack_weights_mxfp8(const uint8_t* q, const uint8_t* scale, int32_t G, int32_t N, int32_t K,
                                    int32_t epilogue, void* out, size_t out_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Unpermute and combine (blog Figure 3: restore the original token order;
 * ch. 1 §2.3.2 dispatch/combine table: the expert outputs of a token are
 * merged by a weighted sum):
 *   y[t, :] = bf16( sum_{k ascending} w[t,k] * y_perm[perm_dst[t*K+k], :] )
 * accumulated in fp32.  topk_w == NULL means every weight is 1 (the plain
 * sum used to fold the data gradient back to tokens).
 * y_perm bf16 [>= T*K, d], perm_dst int32 [T*K], y bf16 [T, d]; d % 8 == 0.
 * ------------------------------------------------------------------------ */
moe_status_t moe_unpermute_combine(const uint16_t* y_perm, const float* topk_w, const int32_t* perm_dst,
                                   int64_t T, int32_t d, int32_t K, uint16_t* y, void* stream);

/* Backward of the combine.  The combine accumulates each token's per-expert
 * results weighted by its routing weights (blog section "Optimization 2:
 * Expert parallelism to integrate Dispatch and Combine", the Combine stage);
 * the pages train this layer (blog title and intro) but give no backward, so
 * this is the gradient of that weighted sum with the routing held fixed:
 *   dy_perm[perm_dst[t*K+k], :] = bf16(w[t,k] * dy[t, :])
 *   d_topk_w[t,k] = sum_j dy[t,j] * y_perm[perm_dst[t*K+k], j] (fp32),
 * the second being what a router's own backward would take in.
 * dy bf16 [T,d], y_perm bf16 [T*K,d], dy_perm bf16 [T*K,d], d_topk_w fp32 [T,K];
 * d % 8 == 0; dy, y_perm, dy_perm 16-byte aligned.  Each row of dy_perm is
 * written by exactly one pair, so the result is bitwise reproducible.
 * dy_perm == NULL computes d_topk_w only (the MXFP8 backward takes dy_perm
 * from mxfp8_quantize_gathered instead, already quantised). */
moe_status_t moe_combine_backward(const uint16_t* dy, const uint16_t* y_perm, const float* topk_w,
                                  const int32_t* perm_dst, int64_t T, int32_t d, int32_t K, uint16_t* dy_perm,
                                  float* d_topk_w, void* stream);

/* The same backward with dy_perm delivered only as MXFP8 along its rows:
 * q_rows uint8 [T*K, d] and scale_rows uint8 [T*K, d/32] equal, bit for bit,
 * mxfp8_group_quantize(axis 0) of the bf16 dy_perm that moe_combine_backward
 * writes (that quantisation fused with its producer, blog section
 * "Optimization 1": each dy row is read once for its K weighted copies);
 * d_topk_w as there.  The transposed codes of dy_perm come from
 * mxfp8_quantize_gathered with topk_w.  d % 32 == 0; dy, y_perm 16-byte
 * aligned, q_rows 8-byte aligned. */
moe_status_t moe_combine_backward_mxfp8(const uint16_t* dy, const uint16_t* y_perm, const float* topk_w,
                                        const int32_t* perm_dst, int64_t T, int32_t d, int32_t K, uint8_t* q_rows,
                                        uint8_t* scale_rows, float* d_topk_w, void* stream);

/* Backward of SwiGLU.  The expert MLP's two input projections are the
 * blog's moe_mlpwi_0 / moe_mlpwi_1 (gate and up, fused into one weight by
 * prefuse_moe_weights), whose activations the DeepSeek-V3 training config
 * keeps for the backward pass (section "Performance reproduction for
 * DeepSeek V3", custom_remat_config; section "JAX host offloading": saved
 * intermediate activations).  From those stored pre-activations
 * gu = [g | u] bf16 [m_cap, 2f] and dh bf16 [m_cap, f], with s = sigmoid(g):
 *   dgu[:, j] = bf16(dh*u*s*(1 + g*(1-s))),  dgu[:, f+j] = bf16(dh*g*s)
 * (the derivative of silu(g)*u), fp32 arithmetic.  Rows >= sum(group_sizes)
 * are skipped (group_sizes may be NULL: all m_cap rows); negative sizes
 * count as 0.  f % 8 == 0; gu, dh, dgu 16-byte aligned. */
moe_status_t moe_swiglu_backward(const uint16_t* gu, const uint16_t* dh, int64_t m_cap, int32_t f,
                                 const int32_t* group_sizes, int32_t G, uint16_t* dgu, void* stream);

/* ------------------------------------------------------------------------
 * Group-aware MXFP8 quantisation (blog: "group-aware MXFP8 quantization" and
 * MXFP8 block scaling for expert matmuls, section "Optimization 1"; ch. 1
 * §1.1 low-precision scaling: one scale per block of 32).  Scale rule (OCP
 * MX v1.0): per block, e = floor(log2(amax)) - 8 clamped to [-127, 127],
 * scale byte = e + 127 (amax == 0 gives byte 0); codes = E4M3FN
 * round-to-nearest-even of clamp(v * 2^-e, -448, 448), sign kept on zero.
 * A block holding a NaN or an infinity gets scale byte 0xFF (the E8M0 NaN:
 * every element of the block decodes to NaN) and codes 0x7F with each
 * value's sign bit (E4M3FN's NaN; the format has no infinity).  The same
 * rule holds for every entry point that writes MXFP8 codes.
 *
 * axis 0: blocks of 32 along each row. x bf16 [rows, cols] -> q [rows, cols],
 *   scale [rows, cols/32].  If group_sizes != NULL only rows < sum(sizes)
 *   are written.  cols % 32 == 0.
 * axis 1: blocks of 32 down each column, restarting at every group's first
 *   row (a group's last block may be short).  The block starting at row
 *   o_g + 32*b has scale row P_g + b, P_g = sum_{h<g} ceil(s_h/32); scale is
 *   [rows/32 + G, cols] (rows past the used ones are not written).
 *   group_sizes required.  cols % 8 == 0.
 * ------------------------------------------------------------------------ */
moe_status_t mxfp8_group_quantize(const uint16_t* x, int64_t rows, int32_t cols, int32_t axis,
                                  const int32_t* group_sizes, int32_t G, uint8_t* q, uint8_t* scale,
                                  uint32_t* err_flag, void* stream);

/* MXFP4 quantisation for the MXFP4 grouped GEMM (OCP MX E2M1 elements; the
 * blog's planned 4-bit format, closing of "Optimization 1").  Per row, per 32
 * consecutive columns: scale 2^e, e = floor(log2 amax) - 2 clamped to
 * [-127, 127] (byte e + 127); codes = round-to-nearest-even of x / 2^e on
 * {0, 0.5, 1, 1.5, 2, 3, 4, 6}, saturating, sign kept (also of zero).  A
 * block holding a NaN or an infinity gets scale byte 0xFF (E8M0 NaN) and
 * codes 7 with each value's sign bit (E2M1 has no NaN: its largest code).
 * x bf16 [rows, cols] (16-byte aligned); codes [rows, cols/2] (16-byte
 * aligned, element 2i in the low nibble of byte i); scales stage-major
 * [cols/128, rows, 4].  cols % 128 == 0.  Weights [G, N, K] quantise as
 * rows = G*N. */
moe_status_t mxfp4_quantize(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                            void* stream);

/* Transposed group-aware MXFP8 quantisation, for the operands of the MXFP8
 * backward whose contraction runs down their rows (the weight gradients sum
 * over a group's tokens; the data gradients contract the weights over their
 * output axis): blocks of 32 run down each column as in axis 1 above,
 * restarting at every group's first row, with the same scale rule, and each
 * column's codes are stored contiguously, so the grouped GEMM reads them as
 * K-contiguous rows (blog: group-aware MXFP8 quantisation, section "What
 * specialized optimizations are required for dropless MoE?").
 * group_sizes != NULL (activations, x bf16 [rows, cols], rows = m_cap):
 *   group g's rows occupy positions [K_g, K_g + s_g) of every row of
 *   qT uint8 [cols, k_cap], K_g = sum_{h<g} 64 * ceil(s_h / 64): groups
 *   start 64-aligned, and positions up to K_g + 64 * ceil(s_g / 64) hold
 *   zero codes (a block with no rows of the group has scale byte 0).  The
 *   block at positions [K_g + 32 b, +32) has its scale at scaleT [cols,
 *   k_cap / 32], column (K_g + 32 b) / 32.  Positions past the last group's
 *   are not written.  k_cap % 64 == 0, k_cap >= rows + 63 G.
 * group_sizes == NULL (weights, x bf16 [G, rows, cols], one group per
 *   batch): qT [G, cols, rows], scaleT [G, cols, rows / 32]; rows % 64 == 0;
 *   k_cap ignored.
 * q_rows, scale_rows (both or neither; cols % 32 == 0, q_rows 16-byte
 *   aligned): also the axis-0 quantisation of the same rows, from the same
 *   read of x, exactly as mxfp8_group_quantize (axis 0) writes it: q_rows
 *   [rows, cols] (batched: [G, rows, cols]), scale_rows [rows, cols / 32];
 *   grouped, only rows < sum(group_sizes) are written.
 * cols % 8 == 0; x, qT 16-byte aligned, scaleT 2-byte aligned.  The data errors of the grouped
 * kernels (negative sizes, sizes past rows) raise err_flag. */
moe_status_t mxfp8_quantize_transposed(const uint16_t* x, int64_t rows, int32_t cols, const int32_t* group_sizes,
                                       int32_t G, int64_t k_cap, uint8_t* qT, uint8_t* scaleT, uint8_t* q_rows,
                                       uint8_t* scale_rows, uint32_t* err_flag, void* stream);

/* Quantisation fused with the dispatch: mxfp8_quantize_transposed (grouped,
 * rows = T*K) of the permuted rows, read straight from their tokens, so that
 * the bf16 permuted copy is never written and read back (blog section
 * "Optimization 2: Expert parallelism to integrate Dispatch and Combine": an
 * unfused chain reads and writes the data several times; "Optimization 1":
 * group-aware MXFP8 quantisation).  Row r of the quantised operand is
 *   topk_w == NULL:  x[perm_src[r] / K, :]                (moe_permute's x_perm)
 *   topk_w != NULL:  bf16(topk_w[perm_src[r]] * x[perm_src[r] / K, :])
 *                    (moe_combine_backward's dy_perm for dy = x),
 * and every output equals, bit for bit, that of mxfp8_quantize_transposed on
 * that bf16 operand with the same group_sizes, G, k_cap, q_rows, scale_rows.
 * x bf16 [T, cols]; perm_src int32 [T*K] as moe_permute writes it (a pair
 * index outside [0, T*K) is clamped into it, never read past x or topk_w);
 * topk_w fp32 [T*K] or NULL; K in [1, 32]; group_sizes required (sum of the
 * sizes = T*K); outputs and alignment as mxfp8_quantize_transposed. */
moe_status_t mxfp8_quantize_gathered(const uint16_t* x, const int32_t* perm_src, const float* topk_w, int64_t T,
                                     int32_t K, int32_t cols, const int32_t* group_sizes, int32_t G, int64_t k_cap,
                                     uint8_t* qT, uint8_t* scaleT, uint8_t* q_rows, uint8_t* scale_rows,
                                     uint32_t* err_flag, void* stream);

/* The SwiGLU backward of moe_swiglu_backward with its output dgu [m_cap, 2f]
 * delivered only as MXFP8, both layouts, as mxfp8_quantize_transposed
 * (grouped, with q_rows and scale_rows) would quantise the bf16 dgu that
 * moe_swiglu_backward writes - bit for bit - without dgu ever being stored
 * in bf16 (the blog's planned quantisation fused with its producer, section
 * "Optimization 1").  Arguments as those two calls; all outputs required;
 * f % 16 == 0. */
moe_status_t moe_swiglu_backward_mxfp8(const uint16_t* gu, const uint16_t* dh, int64_t m_cap, int32_t f,
                                       const int32_t* group_sizes, int32_t G, int64_t k_cap, uint8_t* qT,
                                       uint8_t* scaleT, uint8_t* q_rows, uint8_t* scale_rows, uint32_t* err_flag,
                                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DROPLESS_MOE_H */
