/*
 * oracle.c -- plain CPU oracle for the dropless MoE expert layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  It shares no code, header,
 * table or constant with the device library under dropless_moe_expert_amd/.
 *
 * Everything here is the plain definition, written as loops:
 *   - floating point is accumulated in fp64 and rounded once to the storage
 *     type the method stores (bf16 tensors, fp32 routing weights);
 *   - integer results (routing ids, counts, offsets, permutation maps, MXFP8
 *     codes and scales) are exact.
 *
 * Sources (titles of the pages; section / figure / table on that page):
 *   [BLOG]  "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
 *           Engine": intro (learned Top-K router); "How is dropless MoE
 *           different from capacity-based MoE?" (every token processed by each
 *           expert it selected, nothing dropped or padded); "What specialized
 *           optimizations are required for dropless MoE?" and Figure 3 (router,
 *           dispatch, two grouped GEMMs, combine back to original order);
 *           "Optimization 1: Grouped GEMM" (one call, per-group true counts,
 *           only valid rows computed; MXFP8 block scaling); "Optimization 2"
 *           (dispatch = local reordering; combine = accumulate per-expert
 *           results); MaxText config (moe_mlpwi_0 / moe_mlpwi_1 / moe_mlpwo,
 *           prefuse_moe_weights).
 *   [CH1]   "AI Systems Performance Engineering", ch. 1 (第一章：介绍与 AI 系统概览):
 *           §1.1 data-precision table (bf16 = 1+8+7, E4M3 = 1+4+3), the
 *           floating-point storage example (exponent bias 2^(n-1)-1), the
 *           low-precision scaling figure (MXFP8: one scale per block of 32);
 *           §2.3.1/§2.3.2 (router picks a few experts per token, outputs are
 *           merged by a weighted sum); §4.1 softmax worked example
 *           (max-subtracted exponentials divided by their sum).
 *
 * Readings where the pages are silent (each is listed in the design notes):
 *   - gating = softmax over all experts, then the K largest are kept and their
 *     weights renormalised to sum to one; ties go to the lower expert index;
 *     ids are listed in selection order (descending logit);
 *   - permuted order is a stable counting sort: expert-major, and within an
 *     expert ascending token index (pair index t*K+k);
 *   - expert FFN = SwiGLU: h = silu(g) * u with g from the first f rows of the
 *     fused input projection and u from the next f rows; silu(g) = g/(1+e^-g);
 *     g and u are NOT rounded before the activation, h is stored as bf16;
 *   - MXFP8 scale/code rule from the OCP Microscaling (MX) v1.0 spec (the
 *     pages give only "one scale per 32"): shared exponent
 *     floor(log2(amax)) - 8, clamped to [-127,127], E8M0 byte = exp + 127,
 *     amax == 0 -> byte 0 and all codes +0; codes = E4M3FN round-to-nearest-
 *     even of the scaled value after clamping to +-448; sign kept on zero.
 */
#include <math.h>
#include <stdlib.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* bf16: 1 sign, 8 exponent (bias 127), 7 stored mantissa bits [CH1 §1.1].   */
/* ------------------------------------------------------------------------- */

double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
}

/* Round a double to the nearest bf16, ties to even, overflow to infinity. */
uint16_t oracle_f64_to_bf16(double v)
{
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int ex;
    frexp(a, &ex);              /* a = m * 2^ex, m in [0.5, 1) */
    int e = ex - 1;             /* a in [2^e, 2^(e+1)) */
    int qexp = (e < -126) ? (-126 - 7) : (e - 7);   /* value of one mantissa step */
    double q = rint(ldexp(a, -qexp));                /* default mode: ties-to-even */
    double r = ldexp(q, qexp);
    /* largest finite bf16 is (2 - 2^-7) * 2^127; anything that rounds above is inf */
    if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
    float rf = (float)r;        /* exact: r is a bf16 value */
    uint32_t bits;
    memcpy(&bits, &rf, 4);
    return sign | (uint16_t)((bits >> 16) & 0x7FFF);
}

void oracle_bf16_round_array(const double* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16(in[i]);
}

/* ------------------------------------------------------------------------- */
/* E4M3 (FN variant): 1 sign, 4 exponent (bias 2^(4-1)-1 = 7), 3 mantissa.    */
/* Largest finite 448 = 1.75 * 2^8, smallest subnormal 2^-9, no infinity,     */
/* only 0x7F / 0xFF are NaN.                                                  */
/* ------------------------------------------------------------------------- */

double oracle_e4m3_to_f64(uint8_t c)
{
    int s = c >> 7, ef = (c >> 3) & 0xF, m = c & 7;
    if (ef == 15 && m == 7) return NAN;
    double v = (ef == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, ef - 7);
    return s ? -v : v;
}

/* Saturating round-to-nearest-even encode of an (already scaled) value.
   NaN and +-infinity become E4M3FN's NaN with the value's sign (the format
   has no infinity; only finite values saturate at 448). */
uint8_t oracle_f64_to_e4m3(double x)
{
    uint8_t sign = signbit(x) ? 0x80 : 0;
    if (!isfinite(x)) return sign | 0x7F;
    double a = fabs(x);
    if (a >= 448.0) a = 448.0;                       /* clamp before rounding */
    if (a == 0.0) return sign;
    int ex;
    frexp(a, &ex);
    int e = ex - 1;
    int qexp = (e < -6) ? -9 : (e - 3);              /* one mantissa step */
    double q = rint(ldexp(a, -qexp));
    double r = ldexp(q, qexp);                       /* rounded magnitude */
    if (r == 0.0) return sign;
    if (r < ldexp(1.0, -6)) {                        /* subnormal: exponent field 0 */
        return sign | (uint8_t)(int)ldexp(r, 9);
    }
    frexp(r, &ex);
    e = ex - 1;
    int mant = (int)ldexp(r, 3 - e) - 8;             /* r = (8 + mant) * 2^(e-3) */
    return sign | (uint8_t)(((e + 7) << 3) | mant);
}

/* ------------------------------------------------------------------------- */
/* S0: router scores.  [BLOG] intro: a learned router scores every expert for  */
/* each token; section "Optimization 2": fused router kernels produce them     */
/* right before the dispatch.  The score is the linear map of the token:       */
/*   logits[t, e] = sum_k x[t, k] * w[e, k]  (+ bias[e]),  in fp64.            */
/* ------------------------------------------------------------------------- */

void oracle_route_logits(const uint16_t* x, const uint16_t* w, const float* bias, int64_t T, int32_t d,
                         int32_t E, double* logits)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int k = 0; k < d; ++k)
                acc += oracle_bf16_to_f64(x[t * d + k]) * oracle_bf16_to_f64(w[(int64_t)e * d + k]);
            logits[t * E + e] = acc + (bias ? (double)bias[e] : 0.0);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* S1: router top-K with softmax gating.                                      */
/* [BLOG] intro: a learned router activates the Top-K experts of each token.  */
/* [CH1 §4.1]: softmax = exp of (logit - row max), divided by the row sum.    */
/* ------------------------------------------------------------------------- */

void oracle_route_topk(const float* logits, int64_t T, int32_t E, int32_t K, int32_t renormalize,
                       int32_t* ids, float* w)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float* l = logits + t * E;
        unsigned char taken[1024];
        memset(taken, 0, sizeof(taken));
        /* K rounds of argmax over the experts not yet taken. Strictly greater
           replaces the best, so among equal logits the lowest index wins. */
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e;
            }
            taken[best] = 1;
            ids[t * K + k] = best;
        }
        double m = (double)l[ids[t * K]];            /* first pick holds the row max */
        double denom = 0.0;
        if (renormalize) {
            for (int k = 0; k < K; ++k) denom += exp((double)l[ids[t * K + k]] - m);
        } else {
            for (int e = 0; e < E; ++e) denom += exp((double)l[e] - m);
        }
        for (int k = 0; k < K; ++k)
            w[t * K + k] = (float)(exp((double)l[ids[t * K + k]] - m) / denom);
    }
}

/* ------------------------------------------------------------------------- */
/* S2: dispatch, local part = reorder (token, expert) pairs expert by expert. */
/* [BLOG] "Optimization 2": tokens are permuted to their experts; combine     */
/* later restores the original order (Figure 3).                              */
/* ------------------------------------------------------------------------- */

void oracle_permute(const int32_t* ids, int64_t T, int32_t E, int32_t K,
                    int32_t* group_sizes, int32_t* group_offsets,
                    int32_t* perm_src, int32_t* perm_dst)
{
    int64_t M = T * K;
    for (int e = 0; e < E; ++e) group_sizes[e] = 0;
    for (int64_t i = 0; i < M; ++i) group_sizes[ids[i]] += 1;
    group_offsets[0] = 0;
    for (int e = 0; e < E; ++e) group_offsets[e + 1] = group_offsets[e] + group_sizes[e];
    int32_t fill[1024];
    for (int e = 0; e < E; ++e) fill[e] = 0;
    for (int64_t i = 0; i < M; ++i) {            /* i = t*K + k, ascending */
        int e = ids[i];
        int32_t r = group_offsets[e] + fill[e]++;
        perm_src[r] = (int32_t)i;
        perm_dst[i] = r;
    }
}

/* x_perm[r] = x[perm_src[r] / K]: the row copy of the dispatch. */
void oracle_gather_rows(const uint16_t* x, const int32_t* perm_src, int64_t M, int32_t d, int32_t K,
                        uint16_t* x_perm)
{
    for (int64_t r = 0; r < M; ++r)
        memcpy(x_perm + r * d, x + (int64_t)(perm_src[r] / K) * d, sizeof(uint16_t) * (size_t)d);
}

/* ------------------------------------------------------------------------- */
/* Grouped GEMM, ragged along rows: group e owns rows [o_e, o_e + s_e) of A   */
/* and multiplies them by its own weight B[e] (N x Kd, contraction index       */
/* last).  [BLOG] "Optimization 1": one call, each expert with its true       */
/* token count, only rows with valid tokens computed.                         */
/* The row list selects which rows to compute (NULL = all rows of all groups).*/
/* ------------------------------------------------------------------------- */

static int group_of_row(const int32_t* sizes, int32_t G, int64_t r, int64_t* base)
{
    int64_t o = 0;
    for (int e = 0; e < G; ++e) {
        if (r < o + sizes[e]) { *base = o; return e; }
        o += sizes[e];
    }
    return -1;
}

/* Plain row-ragged GEMM: C[r, n] = bf16(sum_i A[r,i] * B[e][n,i]). */
void oracle_grouped_gemm_rows(const uint16_t* A, const uint16_t* B, const int32_t* sizes, int32_t G,
                              int32_t N, int32_t Kd, const int64_t* rows, int64_t nrows, uint16_t* C)
{
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t q = 0; q < nrows; ++q) {
        int64_t r = rows[q], base;
        int e = group_of_row(sizes, G, r, &base);
        if (e < 0) continue;
        const uint16_t* a = A + r * Kd;
        const uint16_t* b = B + (int64_t)e * N * Kd;
        for (int n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int i = 0; i < Kd; ++i)
                acc += oracle_bf16_to_f64(a[i]) * oracle_bf16_to_f64(b[(int64_t)n * Kd + i]);
            C[q * N + n] = oracle_f64_to_bf16(acc);
        }
    }
}

/* Gate/up projection followed by SwiGLU.  B[e] is the prefused [2f, Kd]
   weight: rows [0,f) are the gate projection (moe_mlpwi_0), rows [f,2f) the
   up projection (moe_mlpwi_1).  h[r,j] = bf16(silu(g) * u).  When gu_out is
   non-NULL the two pre-activations are also stored, as bf16, in [2f] rows. */
void oracle_gemm_swiglu_rows(const uint16_t* A, const uint16_t* B, const int32_t* sizes, int32_t G,
                             int32_t f, int32_t Kd, const int64_t* rows, int64_t nrows,
                             uint16_t* H, uint16_t* gu_out)
{
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t q = 0; q < nrows; ++q) {
        int64_t r = rows[q], base;
        int e = group_of_row(sizes, G, r, &base);
        if (e < 0) continue;
        const uint16_t* a = A + r * Kd;
        const uint16_t* b = B + (int64_t)e * 2 * f * Kd;
        for (int j = 0; j < f; ++j) {
            double g = 0.0, u = 0.0;
            for (int i = 0; i < Kd; ++i) {
                double av = oracle_bf16_to_f64(a[i]);
                g += av * oracle_bf16_to_f64(b[(int64_t)j * Kd + i]);
                u += av * oracle_bf16_to_f64(b[(int64_t)(f + j) * Kd + i]);
            }
            double silu = g / (1.0 + exp(-g));
            H[q * f + j] = oracle_f64_to_bf16(silu * u);
            if (gu_out) {
                gu_out[q * 2 * f + j] = oracle_f64_to_bf16(g);
                gu_out[q * 2 * f + f + j] = oracle_f64_to_bf16(u);
            }
        }
    }
}

/* ------------------------------------------------------------------------- */
/* S6: combine = weighted sum of a token's K expert outputs, back in token    */
/* order.  [CH1 §2.3.2] dispatch/combine table and figure (weighted sum);     */
/* [BLOG] Figure 3 (restore original order).  w == NULL means weight 1.       */
/* ------------------------------------------------------------------------- */

void oracle_unpermute_combine(const uint16_t* y_perm, const float* w, const int32_t* perm_dst,
                              int64_t T, int32_t d, int32_t K, uint16_t* y)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int j = 0; j < d; ++j) {
            double acc = 0.0;
            for (int k = 0; k < K; ++k) {
                double wk = w ? (double)w[t * K + k] : 1.0;
                acc += wk * oracle_bf16_to_f64(y_perm[(int64_t)perm_dst[t * K + k] * d + j]);
            }
            y[t * d + j] = oracle_f64_to_bf16(acc);
        }
    }
}

/* ------------------------------------------------------------------------- */
/* S4: MXFP8 quantisation, blocks of 32 consecutive elements along the         */
/* contraction axis [CH1 §1.1 low-precision scaling figure; BLOG "Optimization */
/* 1" MXFP8 block scaling].  Rule: OCP MX v1.0 (see header).                   */
/* ------------------------------------------------------------------------- */

/* E8M0 scale byte -> its value: 2^(s-127); 0xFF is NaN (OCP MX v1.0). */
double oracle_e8m0_to_f64(uint8_t s)
{
    return s == 0xFF ? NAN : ldexp(1.0, (int)s - 127);
}

/* One block.  A block holding a NaN or an infinity has no finite shared
   exponent: its scale is the E8M0 NaN (0xFF), which makes every element of
   the block NaN, and each code is the element format's NaN with the value's
   sign. */
static void mx_block(const double* v, int n, uint8_t* codes, uint8_t* scale)
{
    for (int i = 0; i < n; ++i) {
        if (!isfinite(v[i])) {
            *scale = 0xFF;
            for (int j = 0; j < n; ++j) codes[j] = oracle_f64_to_e4m3(signbit(v[j]) ? -NAN : NAN);
            return;
        }
    }
    double amax = 0.0;
    for (int i = 0; i < n; ++i) if (fabs(v[i]) > amax) amax = fabs(v[i]);
    if (amax == 0.0) {
        *scale = 0;
        for (int i = 0; i < n; ++i) codes[i] = signbit(v[i]) ? 0x80 : 0x00;
        return;
    }
    int ex;
    frexp(amax, &ex);
    int e = (ex - 1) - 8;                 /* floor(log2 amax) - emax(E4M3) */
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    *scale = (uint8_t)(e + 127);
    for (int i = 0; i < n; ++i) codes[i] = oracle_f64_to_e4m3(ldexp(v[i], -e));
}

/* axis 0: each row is cut into blocks of 32 along the columns.
   q[rows, cols] codes, s[rows, cols/32] scales. */
void oracle_mxfp8_quantize_rows(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* q, uint8_t* s)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double v[32];
        for (int b = 0; b < cols / 32; ++b) {
            for (int i = 0; i < 32; ++i) v[i] = oracle_bf16_to_f64(x[r * cols + b * 32 + i]);
            mx_block(v, 32, q + r * cols + b * 32, s + r * (cols / 32) + b);
        }
    }
}

/* axis 1, group-aware: blocks of 32 run down each column and restart at every
   group's first row; a group's last block may be short (its missing elements
   count as zero for amax).  Scale row of the block starting at row o_e + 32*b
   is P_e + b, where P_e = sum over earlier groups of ceil(s/32).
   q[rows, cols], s[sum_e ceil(s_e/32), cols]. */
void oracle_mxfp8_quantize_cols_grouped(const uint16_t* x, int64_t rows, int32_t cols,
                                        const int32_t* sizes, int32_t G, uint8_t* q, uint8_t* s)
{
    (void)rows;
    int64_t o = 0, P = 0;
    for (int e = 0; e < G; ++e) {
        int64_t nb = (sizes[e] + 31) / 32;
        for (int64_t b = 0; b < nb; ++b) {
            int64_t r0 = o + 32 * b;
            int n = (int)((sizes[e] - 32 * b) < 32 ? (sizes[e] - 32 * b) : 32);
            for (int c = 0; c < cols; ++c) {
                double v[32];
                uint8_t codes[32];
                for (int i = 0; i < n; ++i) v[i] = oracle_bf16_to_f64(x[(r0 + i) * cols + c]);
                mx_block(v, n, codes, s + (P + b) * cols + c);
                for (int i = 0; i < n; ++i) q[(r0 + i) * cols + c] = codes[i];
            }
        }
        o += sizes[e];
        P += nb;
    }
}

/* MXFP8 grouped GEMM: dequantise exactly (code value * 2^(scale-127)), then
   the plain row-ragged GEMM.  A codes [M, Kd] with scales [M, Kd/32]; B codes
   [G, N, Kd] with scales [G, N, Kd/32]. Output bf16. Epilogue 1 = SwiGLU
   (N = 2f, output [f]). */
void oracle_mx_grouped_gemm_rows(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq, const uint8_t* Bs,
                                 const int32_t* sizes, int32_t G, int32_t N, int32_t Kd, int32_t swiglu,
                                 const int64_t* rows, int64_t nrows, uint16_t* C)
{
    int32_t nb = Kd / 32;
    int32_t nout = swiglu ? N / 2 : N;
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t q = 0; q < nrows; ++q) {
        int64_t r = rows[q], base;
        int e = group_of_row(sizes, G, r, &base);
        if (e < 0) continue;
        double* av = (double*)malloc(sizeof(double) * (size_t)Kd);
        for (int i = 0; i < Kd; ++i)
            av[i] = oracle_e4m3_to_f64(Aq[r * Kd + i]) * oracle_e8m0_to_f64(As[r * nb + i / 32]);
        const uint8_t* bq = Bq + (int64_t)e * N * Kd;
        const uint8_t* bs = Bs + (int64_t)e * N * nb;
        double acc2[2];
        for (int n = 0; n < nout; ++n) {
            for (int h = 0; h < (swiglu ? 2 : 1); ++h) {
                int64_t col = n + (int64_t)h * nout;
                double acc = 0.0;
                for (int i = 0; i < Kd; ++i)
                    acc += av[i] * oracle_e4m3_to_f64(bq[col * Kd + i]) * oracle_e8m0_to_f64(bs[col * nb + i / 32]);
                acc2[h] = acc;
            }
            if (swiglu) {
                double g = acc2[0], u = acc2[1];
                C[q * nout + n] = oracle_f64_to_bf16(g / (1.0 + exp(-g)) * u);
            } else {
                C[q * nout + n] = oracle_f64_to_bf16(acc2[0]);
            }
        }
        free(av);
    }
}

/* ------------------------------------------------------------------------- */
/* MXFP4: E2M1 elements with an E8M0 scale per 32 (the gfx950 analog of the  */
/* page's planned NVFP4, [BLOG] "Optimization 1" closing plans; MX element   */
/* formats per the OCP MX v1.0 specification).                               */
/* E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit; no Inf/NaN.      */
/* ------------------------------------------------------------------------- */

double oracle_e2m1_to_f64(uint8_t c)
{
    int s = (c >> 3) & 1, ex = (c >> 1) & 3, m = c & 1;
    double mag = ex == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, ex - 1);
    return s ? -mag : mag;
}

/* round to nearest representable magnitude, ties to the even code (mantissa
   bit 0), saturating at 6; the sign is kept (also for a zero result).  E2M1
   has no infinity or NaN: infinities saturate like any value past 6, and NaN
   takes the same largest-magnitude code with its sign. */
uint8_t oracle_f64_to_e2m1(double v)
{
    uint8_t sign = signbit(v) ? 8 : 0;
    double a = fabs(v);
    if (isnan(a) || a >= 6.0) return sign | 7;   /* saturation: 6 is the largest magnitude */
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(oracle_e2m1_to_f64((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0)) { bd = d; best = c; }
    }
    return sign | (uint8_t)best;
}

/* one 32-block: scale 2^e with e = floor(log2 amax) - 2 (2 = largest E2M1
   exponent), clamped to [-127, 127]; codes one per byte */
static void mx4_block(const double* v, int n, uint8_t* codes, uint8_t* scale)
{
    for (int i = 0; i < n; ++i) {             /* NaN or infinity: NaN scale, as mx_block */
        if (!isfinite(v[i])) {
            *scale = 0xFF;
            for (int j = 0; j < n; ++j) codes[j] = oracle_f64_to_e2m1(signbit(v[j]) ? -NAN : NAN);
            return;
        }
    }
    double amax = 0.0;
    for (int i = 0; i < n; ++i) if (fabs(v[i]) > amax) amax = fabs(v[i]);
    if (amax == 0.0) {
        *scale = 0;
        for (int i = 0; i < n; ++i) codes[i] = signbit(v[i]) ? 8 : 0;
        return;
    }
    int ex;
    frexp(amax, &ex);
    int e = (ex - 1) - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    *scale = (uint8_t)(e + 127);
    for (int i = 0; i < n; ++i) codes[i] = oracle_f64_to_e2m1(ldexp(v[i], -e));
}

/* q[rows, cols]: one code per byte; s[rows, cols/32] */
void oracle_mxfp4_quantize_rows(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* q, uint8_t* s)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        double v[32];
        for (int b = 0; b < cols / 32; ++b) {
            for (int i = 0; i < 32; ++i) v[i] = oracle_bf16_to_f64(x[r * cols + b * 32 + i]);
            mx4_block(v, 32, q + r * cols + b * 32, s + r * (cols / 32) + b);
        }
    }
}

/* MXFP4 grouped GEMM on the listed rows of A: dequantise exactly, fp64
   contraction, bf16 output; swiglu: h = silu(g) * u over B rows [0, N/2) and
   [N/2, N) of each expert.  Codes one per byte: A [M, K], B [G, N, K];
   scales [M, K/32], [G, N, K/32]. */
void oracle_mx4_grouped_gemm_rows(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq, const uint8_t* Bs,
                                  const int32_t* sizes, int32_t G, int32_t N, int32_t Kd, int32_t swiglu,
                                  const int64_t* rows, int64_t nrows, uint16_t* C)
{
    int32_t nb = Kd / 32;
    int32_t nout = swiglu ? N / 2 : N;
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t q = 0; q < nrows; ++q) {
        int64_t r = rows[q], base;
        int e = group_of_row(sizes, G, r, &base);
        if (e < 0) continue;
        double* av = (double*)malloc(sizeof(double) * (size_t)Kd);
        for (int i = 0; i < Kd; ++i)
            av[i] = oracle_e2m1_to_f64(Aq[r * Kd + i]) * oracle_e8m0_to_f64(As[r * nb + i / 32]);
        const uint8_t* bq = Bq + (int64_t)e * N * Kd;
        const uint8_t* bs = Bs + (int64_t)e * N * nb;
        double acc2[2];
        for (int n = 0; n < nout; ++n) {
            for (int h = 0; h < (swiglu ? 2 : 1); ++h) {
                int64_t col = n + (int64_t)h * nout;
                double acc = 0.0;
                for (int i = 0; i < Kd; ++i)
                    acc += av[i] * oracle_e2m1_to_f64(bq[col * Kd + i]) * oracle_e8m0_to_f64(bs[col * nb + i / 32]);
                acc2[h] = acc;
            }
            if (swiglu) {
                double g = acc2[0], u = acc2[1];
                C[q * nout + n] = oracle_f64_to_bf16(g / (1.0 + exp(-g)) * u);
            } else {
                C[q * nout + n] = oracle_f64_to_bf16(acc2[0]);
            }
        }
        free(av);
    }
}

/* MXFP8 weight gradient [BLOG "What specialized optimizations are required  */
/* for dropless MoE?": group-aware MXFP8 quantisation; "Optimization 1":     */
/* MXFP8 block scaling].  Both operands quantised along their rows by the     */
/* group-aware axis-1 rule above (codes [rows, P] and [rows, Q], scales       */
/* [sum_e ceil(s_e/32), P] and [.., Q]); dequantise exactly, then the plain   */
/* ragged contraction: C[e][p, q] = bf16(sum_{r in e} a[r, p] * b[r, q]).      */
void oracle_mx_grouped_wgrad(const uint8_t* Aq, const uint8_t* As, const uint8_t* Bq, const uint8_t* Bs,
                             const int32_t* sizes, int32_t G, int32_t P, int32_t Q, uint16_t* C)
{
    int64_t o = 0, pb = 0;
    for (int e = 0; e < G; ++e) {
        int64_t s = sizes[e];
        uint16_t* out = C + (int64_t)e * P * Q;
        #pragma omp parallel for schedule(static)
        for (int p = 0; p < P; ++p) {
            for (int q = 0; q < Q; ++q) {
                double acc = 0.0;
                for (int64_t i = 0; i < s; ++i) {
                    int64_t r = o + i, blk = pb + i / 32;
                    double a = oracle_e4m3_to_f64(Aq[r * P + p]) * oracle_e8m0_to_f64(As[blk * P + p]);
                    double b = oracle_e4m3_to_f64(Bq[r * Q + q]) * oracle_e8m0_to_f64(Bs[blk * Q + q]);
                    acc += a * b;
                }
                out[(int64_t)p * Q + q] = oracle_f64_to_bf16(acc);
            }
        }
        o += s;
        pb += (s + 31) / 32;
    }
}

/* ------------------------------------------------------------------------- */
/* S7: backward of the layer (training).  Derivatives of the forward above;   */
/* each result is accumulated in fp64 and stored as bf16 (dw as fp32).        */
/* ------------------------------------------------------------------------- */

/* Combine backward.  dy_perm[perm_dst[t,k]] = bf16(w[t,k] * dy[t]) and
   dw[t,k] = <dy[t], y_perm[perm_dst[t,k]]>. */
void oracle_combine_backward(const uint16_t* dy, const uint16_t* y_perm, const float* w,
                             const int32_t* perm_dst, int64_t T, int32_t d, int32_t K,
                             uint16_t* dy_perm, float* dw)
{
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int k = 0; k < K; ++k) {
            int64_t r = perm_dst[t * K + k];
            double dot = 0.0;
            for (int j = 0; j < d; ++j) {
                double g = oracle_bf16_to_f64(dy[t * d + j]);
                dot += g * oracle_bf16_to_f64(y_perm[r * d + j]);
                dy_perm[r * d + j] = oracle_f64_to_bf16((double)w[t * K + k] * g);
            }
            dw[t * K + k] = (float)dot;
        }
    }
}

/* SwiGLU backward from the stored pre-activations gu = [g | u] (bf16):
   with s = sigmoid(g): dg = dh*u*s*(1 + g*(1-s)), du = dh*g*s. */
void oracle_swiglu_backward(const uint16_t* gu, const uint16_t* dh, int64_t M, int32_t f, uint16_t* dgu)
{
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < M; ++r) {
        for (int j = 0; j < f; ++j) {
            double g = oracle_bf16_to_f64(gu[r * 2 * f + j]);
            double u = oracle_bf16_to_f64(gu[r * 2 * f + f + j]);
            double d = oracle_bf16_to_f64(dh[r * f + j]);
            double s = 1.0 / (1.0 + exp(-g));
            dgu[r * 2 * f + j] = oracle_f64_to_bf16(d * u * s * (1.0 + g * (1.0 - s)));
            dgu[r * 2 * f + f + j] = oracle_f64_to_bf16(d * g * s);
        }
    }
}

/* Data gradient of a row-ragged GEMM C = A * B[e]^T (B[e] is [N, Kd]):
   dA[r, i] = bf16(sum_n dC[r, n] * B[e][n, i]).  Rows selected as above. */
void oracle_grouped_dgrad_rows(const uint16_t* dC, const uint16_t* B, const int32_t* sizes, int32_t G,
                               int32_t N, int32_t Kd, const int64_t* rows, int64_t nrows, uint16_t* dA)
{
    #pragma omp parallel for schedule(dynamic, 4)
    for (int64_t q = 0; q < nrows; ++q) {
        int64_t r = rows[q], base;
        int e = group_of_row(sizes, G, r, &base);
        if (e < 0) continue;
        const uint16_t* b = B + (int64_t)e * N * Kd;
        for (int i = 0; i < Kd; ++i) {
            double acc = 0.0;
            for (int n = 0; n < N; ++n)
                acc += oracle_bf16_to_f64(dC[r * N + n]) * oracle_bf16_to_f64(b[(int64_t)n * Kd + i]);
            dA[q * Kd + i] = oracle_f64_to_bf16(acc);
        }
    }
}

/* Weight gradient of the same GEMM, contracted over each group's rows (a
   ragged contraction): dB[e][n, i] = bf16(sum_{r in group e} dC[r, n] * A[r, i]).
   Empty groups give exact zeros.  Groups selected by the list (NULL = all). */
void oracle_grouped_wgrad(const uint16_t* dC, const uint16_t* A, const int32_t* sizes, int32_t G,
                          int32_t N, int32_t Kd, const int32_t* groups, int32_t ngroups, uint16_t* dB)
{
    int64_t offs[1025];
    offs[0] = 0;
    for (int e = 0; e < G; ++e) offs[e + 1] = offs[e] + sizes[e];
    int32_t ng = groups ? ngroups : G;
    for (int32_t q = 0; q < ng; ++q) {
        int e = groups ? groups[q] : q;
        uint16_t* out = dB + (int64_t)q * N * Kd;
        #pragma omp parallel for schedule(static)
        for (int n = 0; n < N; ++n) {
            for (int i = 0; i < Kd; ++i) {
                double acc = 0.0;
                for (int64_t r = offs[e]; r < offs[e + 1]; ++r)
                    acc += oracle_bf16_to_f64(dC[r * N + n]) * oracle_bf16_to_f64(A[r * Kd + i]);
                out[(int64_t)n * Kd + i] = oracle_f64_to_bf16(acc);
            }
        }
    }
}
