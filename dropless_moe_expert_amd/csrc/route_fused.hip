// Fused router: the logits product, top-K with softmax gating and the
// dispatch histogram in one kernel.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine": intro (a learned router picks each token's Top-K experts) and
// section "Optimization 2: Expert parallelism to integrate Dispatch and
// Combine" (the router runs as fused kernels right before the dispatch).
// "AI Systems Performance Engineering" ch. 1, §4.1: softmax weights are
// exp(score - max) over their sum.
//
// One workgroup (4 wavefronts) per block of TW tokens:
//  1. logits [TW, E] = x[t0 : t0 + TW] W_r^T on bf16 MFMA (16x16x32, fp32
//     accumulation), in one of two ways:
//     E > 32: rows of x and of W_r stream through an LDS ring of NS stages of
//     KC = 32 NSUB k-values, filled by direct-to-LDS loads issued NS - 1
//     stages ahead.  A stage holds NSUB / 2 pairs of 32-k steps as 128-byte
//     rows, so each load instruction reads whole cache lines (8 rows x 128
//     bytes); every stage issues the same number of loads (pairs past d
//     re-read the last one), so one vmcnt count per stage distance is exact.
//     A wavefront owns a (16 TM tokens) x (16 TN experts) block of the logits
//     and, with SK > 1, every SK-th 32-k step.
//     E <= 32: the wavefronts split the contraction and stream their
//     fragments straight into registers (route_fused_reg_kernel).
//  2. The partial logit blocks meet in LDS; one pass sums them in block
//     order, adds the bias, turns NaN into -inf (flag) and writes the optional
//     fp32 logits.
//  3. Top-K: a group of 4-16 lanes per token reads the token's logits from
//     LDS and selects as moe_route_topk does (route_select.h), hence the same
//     ids for the same logits.
//  4. Weights: exp(l_k - l_max) over their sum (renormalised) or over the sum
//     across all E experts, as moe_route_topk computes them.
//  5. Dispatch histogram: the block's pairs (t, k), in pair order, form one
//     chunk of moe_permute's counting sort: each pair's rank among the
//     chunk's earlier pairs with the same expert, and the chunk's per-expert
//     counts, in the workspace layout moe_permute_routed reads.
#include "common.h"
#include "route_select.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace moe {
namespace router {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int wave_idx() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}

// 16-byte slot of chunk c (0..7) in LDS row r (128-byte rows): c ^ ((r >> 1) & 7).
// A fragment read (16 rows, one chunk) then touches rows of both parities at
// eight distinct slots each: the 16 lanes of a quarter-wave hit 256 distinct bytes.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

template <int NB>
__device__ __forceinline__ void wait_stages(int q) {
  if (q <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (q == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NB) : "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NB) : "memory");
}

template <int TM, int TN, int WM, int WN, int SK, int NSUB, int NS>
struct Cfg {
  static constexpr int TW = WM * 16 * TM;          // tokens per workgroup
  static constexpr int EP = WN * 16 * TN;          // experts, padded
  static constexpr int ROWS = TW + EP;             // LDS rows per pair of steps (x rows, then W_r rows)
  static constexpr int PAIR_B = ROWS * 128;        // one pair of 32-k steps: 128-byte rows
  static constexpr int NP = NSUB / 2;              // pairs per stage
  static constexpr int KC = 32 * NSUB;
  static constexpr int STAGE_B = NP * PAIR_B;
  static constexpr int NJ = ROWS / 8;              // 1-KB load blocks (8 rows) per pair
  static constexpr int NB = NP * NJ / 4;           // load blocks per wavefront and stage
  static constexpr int LS = EP + 4;                // logits row stride (floats), as in Epi
  static_assert(WM * WN * SK == 4, "four wavefronts");
  static_assert(NSUB % 2 == 0 && (NP * NJ) % 4 == 0 && NSUB % SK == 0, "tiling");
  static_assert(NS >= 2 && NS <= 4, "the stage wait covers up to two stages ahead");
};

// Epilogue shared by both kernels: on entry LG = lds holds SK partial logit
// blocks [SK][TW][EP + 4] (fp32) written by the caller, and BIAS the bias.
template <int TW, int EP, int SK, int KL>
struct Epi {
  static constexpr int LS = EP + 4;                // logits row stride (floats)
  static constexpr int LG_B = SK * TW * LS * 4;
  static constexpr int ID_B = TW * 32 * 4;
  static constexpr int BYTES = LG_B + ID_B + 256 * 4;
  // top-K: a group of LPT lanes per token, VPL logits per lane (route_select.h)
  static constexpr int LPT = EP <= 32 ? 4 : EP <= 128 ? 8 : 16;
  static constexpr int VPL = EP / LPT;
  static constexpr int SLOTS = (KL + LPT - 1) / LPT;
  static_assert(VPL <= 16 && VPL % 4 == 0, "whole 16-byte chunks of logits per lane");
};

template <int TW, int EP, int SK, int KL>
__device__ __forceinline__ void finish_block(uint8_t* lds, const float* BIAS, int64_t t0, int tvalid, int E, int K,
                                             int renorm, int32_t* __restrict__ ids, float* __restrict__ wout,
                                             float* __restrict__ logits, int32_t* __restrict__ local_rank,
                                             int32_t* __restrict__ chunk_counts, uint32_t* flag) {
  using P = Epi<TW, EP, SK, KL>;
  constexpr int LS = P::LS, LG_B = P::LG_B, ID_B = P::ID_B;
  const int tid = threadIdx.x, lane = tid & 63, w = wave_idx();
  float* LG = reinterpret_cast<float*>(lds);
  int32_t* IDL = reinterpret_cast<int32_t*>(lds + LG_B);
  int32_t* running = reinterpret_cast<int32_t*>(lds + LG_B + ID_B);
  __syncthreads();
  bool nan_seen = false;
  for (int u = tid; u < TW * (EP / 4); u += 256) {
    const int tok = u / (EP / 4), e4 = (u % (EP / 4)) * 4;
    f32x4_t v = *reinterpret_cast<const f32x4_t*>(LG + tok * LS + e4);
#pragma unroll
    for (int q = 1; q < SK; ++q) {
      const f32x4_t p = *reinterpret_cast<const f32x4_t*>(LG + (q * TW + tok) * LS + e4);
      v[0] += p[0]; v[1] += p[1]; v[2] += p[2]; v[3] += p[3];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e4 + j;
      if (e < E) {
        float l = v[j] + BIAS[e];
        if (l != l) { nan_seen = true; l = -INFINITY; }
        v[j] = l;
      } else {
        v[j] = -INFINITY;
      }
    }
    *reinterpret_cast<f32x4_t*>(LG + tok * LS + e4) = v;
    if (logits && tok < tvalid && e4 < E) {
      float* dst = logits + (t0 + tok) * E + e4;
      if ((E & 3) == 0) {
        *reinterpret_cast<f32x4_t*>(dst) = v;
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (e4 + j < E) dst[j] = v[j];
      }
    }
  }
  if (__any(nan_seen) && lane == 0) raise_flag(flag, MOE_FLAG_NAN_LOGIT);
  __syncthreads();

  // ------------------------------------------------- 3-4. top-K and weights
  // A group of LPT lanes per token, as moe_route_topk (route_select.h): the
  // same ids and weights for the same logits.  Lane sub of the group reads
  // its chunks of 4 logits from the token's LDS row (padded experts hold
  // -inf and are absent to the selection).
  {
    using G = topk::Group<P::LPT, P::VPL>;
    constexpr int TPW = 64 / P::LPT;   // tokens per wavefront and pass
    const int sub = lane % P::LPT;
#pragma unroll 1
    for (int base = 0; base < TW; base += 4 * TPW) {
      const int t = base + w * TPW + lane / P::LPT;
      if (t >= TW) break;   // whole groups of lanes leave together
      float v[P::VPL];
      const float* row = LG + t * LS;
#pragma unroll
      for (int c = 0; c < P::VPL / 4; ++c) {
        const f32x4_t q = *reinterpret_cast<const f32x4_t*>(row + G::expert(sub, 4 * c));
        v[4 * c] = q[0]; v[4 * c + 1] = q[1]; v[4 * c + 2] = q[2]; v[4 * c + 3] = q[3];
      }
      int pk[P::SLOTS], pi[P::SLOTS], kmax;
      G::template select<P::SLOTS>(v, E, K, sub, pk, pi, kmax);
      float a[P::SLOTS];
      const float part = G::template weights<P::SLOTS>(v, E, K, renorm, sub, pk, kmax, a);
      if (t < tvalid) {
        const int64_t o = (t0 + t) * K;
#pragma unroll
        for (int q = 0; q < P::SLOTS; ++q) {
          const int k = q * P::LPT + sub;
          if (k < K) {
            ids[o + k] = pi[q];
            wout[o + k] = a[q] / part;
            IDL[t * K + k] = pi[q];
          }
        }
      }
    }
  }
  if (local_rank == nullptr) return;
  __syncthreads();

  // --------------------------------------------------- 5. dispatch histogram
  if (w == 0) {
    for (int e = lane; e < E; e += 64) running[e] = 0;
    const int npairs = tvalid * K;
    for (int base = 0; base < npairs; base += 64) {
      const int i = base + lane;
      const bool valid = i < npairs;
      const int e = valid ? IDL[i] : 0;
      uint64_t same = __ballot(valid);
#pragma unroll
      for (int bit = 0; bit < 8; ++bit) {
        const uint64_t ones = __ballot(valid && ((e >> bit) & 1));
        same &= ((e >> bit) & 1) ? ones : ~ones;
      }
      const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      const int before = __popcll(same & below);
      const int total = __popcll(same);
      const int r = valid ? running[e] + before : 0;
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // every lane has read running[] before the updates
      if (valid) {
        local_rank[t0 * K + i] = r;
        if (before == total - 1) running[e] += total;   // the class's highest lane
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    for (int e = lane; e < E; e += 64) chunk_counts[(int64_t)blockIdx.x * E + e] = running[e];
  }
}

template <int TM, int TN, int WM, int WN, int SK, int NSUB, int NS, int KL>
__global__ __launch_bounds__(256) void route_fused_lds_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          const float* __restrict__ bias, int64_t T, int d, int E,
                                                          int K, int renorm, int32_t* __restrict__ ids,
                                                          float* __restrict__ wout, float* __restrict__ logits,
                                                          int32_t* __restrict__ local_rank,
                                                          int32_t* __restrict__ chunk_counts, uint32_t* flag) {
  using C = Cfg<TM, TN, WM, WN, SK, NSUB, NS>;
  constexpr int TW = C::TW, EP = C::EP, LS = C::LS, NB = C::NB;
  constexpr int EPI_B = Epi<TW, EP, SK, KL>::BYTES;
  constexpr int LDS_B = (NS * C::STAGE_B > EPI_B) ? NS * C::STAGE_B : EPI_B;
  __shared__ __align__(1024) uint8_t lds[LDS_B];
  __shared__ float BIAS[256];

  const int tid = threadIdx.x, lane = tid & 63, w = wave_idx();
  const int64_t t0 = (int64_t)blockIdx.x * TW;
  const int tvalid = (int)min<int64_t>(TW, T - t0);   // >= 1
  const float bias_r = (bias != nullptr && tid < E) ? bias[tid] : 0.f;   // lands during the k loop

  // ---------------------------------------------------------------- 1. logits
  const int ks = w % SK, wn = (w / SK) % WN, wm = w / (SK * WN);
  const uint8_t* xb = uniform_ptr(reinterpret_cast<const uint8_t*>(x + t0 * d));
  const uint8_t* wb = uniform_ptr(reinterpret_cast<const uint8_t*>(wr));
  // load slot i of wavefront w: block b = 4i + w = (pair p, 8-row block j);
  // lane l fills slot l & 7 of row 8j + l / 8 with chunk (l & 7) ^ swz(row)
  uint32_t voff[NB], lds_of[NB], hi_adj[NB];
  int pair_of[NB];
  bool is_x[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int b = 4 * i + w, p = b / C::NJ, j = b % C::NJ;
    const int r = 8 * j + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    pair_of[i] = p;
    lds_of[i] = (uint32_t)(p * C::PAIR_B + j * 1024);
    is_x[i] = 8 * j < TW;
    const int grow = is_x[i] ? min(r, tvalid - 1) : min(r - TW, E - 1);
    voff[i] = (uint32_t)grow * (uint32_t)d * 2u + (uint32_t)c * 16u;
    hi_adj[i] = c >= 4 ? 64u : 0u;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)lds;
  const int nst = (d + C::KC - 1) / C::KC;
  // the last pair starts at last_pair; when only its first step exists
  // (d % 64 == 32) its upper 64 bytes re-read the lower ones
  const int last_pair = ((d - 1) / 64) * 64;
  const bool half_pair = (d - last_pair) == 32;
  auto issue = [&](int st) {
    const int buf = st % NS, k0 = st * C::KC;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int kb = min(k0 + 64 * pair_of[i], last_pair);
      const uint8_t* base = uniform_ptr((is_x[i] ? xb : wb) + (int64_t)kb * 2);
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)(buf * C::STAGE_B) + lds_of[i]);
      const uint32_t vo = (half_pair && kb == last_pair) ? voff[i] - hi_adj[i] : voff[i];
      asm volatile(
          "s_mov_b32 m0, %0\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dwordx4 %1, %2"
          :
          : "s"(m0), "v"(vo), "s"(base)
          : "memory", "m0");
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int st = 0; st < NS - 1 && st < nst; ++st) issue(st);
  for (int st = 0; st < nst; ++st) {
    wait_stages<NB>(min(nst - 1, st + NS - 2) - st);
    asm volatile("s_barrier" ::: "memory");
    if (st + NS - 1 < nst) issue(st + NS - 1);
    const uint8_t* sb = lds + (st % NS) * C::STAGE_B;
    const int k0 = st * C::KC;
#pragma unroll
    for (int s = 0; s < NSUB; ++s) {
      if (s % SK != ks || k0 + 32 * s >= d) continue;
      // step s: pair s / 2, chunks 4 (s & 1) .. + 3 of each 128-byte row
      const uint8_t* pr = sb + (s >> 1) * C::PAIR_B;
      const int cc = 4 * (s & 1) + (lane >> 4);
      bf16x8_t xf[TM], wf[TN];
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        const int r = wm * 16 * TM + 16 * a + (lane & 15);
        xf[a] = *reinterpret_cast<const bf16x8_t*>(pr + r * 128 + ((cc ^ swz(r)) << 4));
      }
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int r = TW + wn * 16 * TN + 16 * b + (lane & 15);
        wf[b] = *reinterpret_cast<const bf16x8_t*>(pr + r * 128 + ((cc ^ swz(r)) << 4));
      }
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[b], xf[a], acc[a][b], 0, 0, 0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // ------------------------------------------------- 2. partial logits -> LDS
  float* LG = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      // lane: token (lane & 15) of block a, experts 4 (lane >> 4) .. + 3 of block b
      const int tok = wm * 16 * TM + 16 * a + (lane & 15);
      const int e = wn * 16 * TN + 16 * b + 4 * (lane >> 4);
      *reinterpret_cast<f32x4_t*>(LG + (ks * TW + tok) * LS + e) = acc[a][b];
    }
  BIAS[tid] = bias_r;
  finish_block<TW, EP, SK, KL>(lds, BIAS, t0, tvalid, E, K, renorm, ids, wout, logits, local_rank, chunk_counts,
                               flag);
}

// Small E: the four wavefronts split the contraction instead (wavefront w owns
// the whole TW x E block for the 64-k pairs of steps q = w, w + 4, ...), so no
// operand is shared and each wavefront streams its x and W_r fragments from
// global memory straight into registers, two steps in flight; a pair's two
// loads cover whole 128-byte lines of every row.  With few experts the W_r
// share of the traffic is small and this avoids the LDS round trip.
typedef const __attribute__((address_space(1))) bf16x8_t gbf16x8_t;

template <int TM, int TN>
struct Frags {
  bf16x8_t x[TM], w[TN];
  __device__ __forceinline__ void load(const uint8_t* xb, const uint8_t* wb, const uint32_t (&xo)[TM],
                                       const uint32_t (&wo)[TN], uint32_t kbytes) {
#pragma unroll
    for (int a = 0; a < TM; ++a) x[a] = *(gbf16x8_t*)(xb + xo[a] + kbytes);
#pragma unroll
    for (int b = 0; b < TN; ++b) w[b] = *(gbf16x8_t*)(wb + wo[b] + kbytes);
  }
  __device__ __forceinline__ void mma(f32x4_t (&acc)[TM][TN]) const {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b) acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[b], x[a], acc[a][b], 0, 0, 0);
  }
};

template <int TM, int TN, int KL>
__global__ __launch_bounds__(256) void route_fused_reg_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ wr,
                                                              const float* __restrict__ bias, int64_t T, int d, int E,
                                                              int K, int renorm, int32_t* __restrict__ ids,
                                                              float* __restrict__ wout, float* __restrict__ logits,
                                                              int32_t* __restrict__ local_rank,
                                                              int32_t* __restrict__ chunk_counts, uint32_t* flag) {
  constexpr int TW = 16 * TM, EP = 16 * TN, LS = EP + 4;
  __shared__ __align__(16) uint8_t lds[Epi<TW, EP, 4, KL>::BYTES];
  __shared__ float BIAS[256];
  const int tid = threadIdx.x, lane = tid & 63, w = wave_idx();
  const int64_t t0 = (int64_t)blockIdx.x * TW;
  const int tvalid = (int)min<int64_t>(TW, T - t0);   // >= 1
  const float bias_r = (bias != nullptr && tid < E) ? bias[tid] : 0.f;

  const uint8_t* xb = uniform_ptr(reinterpret_cast<const uint8_t*>(x + t0 * d));
  const uint8_t* wb = uniform_ptr(reinterpret_cast<const uint8_t*>(wr));
  uint32_t xo[TM], wo[TN];   // byte offsets of this lane's rows (rows past the end re-read the last one)
#pragma unroll
  for (int a = 0; a < TM; ++a)
    xo[a] = (uint32_t)min(16 * a + (lane & 15), tvalid - 1) * (uint32_t)d * 2u + (uint32_t)(lane >> 4) * 16u;
#pragma unroll
  for (int b = 0; b < TN; ++b)
    wo[b] = (uint32_t)min(16 * b + (lane & 15), E - 1) * (uint32_t)d * 2u + (uint32_t)(lane >> 4) * 16u;
  f32x4_t acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // the loop body is branch-free (the last prefetch re-reads the last pair)
  // so that the compiler's vmcnt waits keep the next pair in flight; the
  // sched_barrier fences stop the scheduler from sinking loads to their use
  const int nsteps = d / 32;
  const int npairs = nsteps / 2;
  const int cnt = (w < npairs) ? (npairs - w + 3) / 4 : 0;
  Frags<TM, TN> fa, fb;
  if (cnt > 0) {
    fa.load(xb, wb, xo, wo, (uint32_t)w * 128u);
    fb.load(xb, wb, xo, wo, (uint32_t)w * 128u + 64u);
    for (int j = 0; j < cnt; ++j) {
      const uint32_t next = (uint32_t)(w + 4 * min(j + 1, cnt - 1)) * 128u;
      __builtin_amdgcn_sched_barrier(0);
      fa.mma(acc);
      __builtin_amdgcn_sched_barrier(0);
      fa.load(xb, wb, xo, wo, next);
      __builtin_amdgcn_sched_barrier(0);
      fb.mma(acc);
      __builtin_amdgcn_sched_barrier(0);
      fb.load(xb, wb, xo, wo, next + 64u);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if ((nsteps & 1) && w == (npairs & 3)) {   // an unpaired last step (d % 64 == 32)
    fa.load(xb, wb, xo, wo, (uint32_t)(nsteps - 1) * 64u);
    fa.mma(acc);
  }
  float* LG = reinterpret_cast<float*>(lds);
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const int tok = 16 * a + (lane & 15);
      const int e = 16 * b + 4 * (lane >> 4);
      *reinterpret_cast<f32x4_t*>(LG + (w * TW + tok) * LS + e) = acc[a][b];
    }
  BIAS[tid] = bias_r;
  finish_block<TW, EP, 4, KL>(lds, BIAS, t0, tvalid, E, K, renorm, ids, wout, logits, local_rank, chunk_counts, flag);
}

}  // namespace router
}  // namespace moe

namespace {
template <int TM, int TN, int WM, int WN, int SK, int NSUB, int NS>
moe_status_t launch_lds(const uint16_t* x, const uint16_t* wr, const float* bias, int64_t T, int d, int E, int K,
                        int renorm, int32_t* ids, float* w, float* logits, int32_t* lr, int32_t* cc, uint32_t* flag,
                        hipStream_t s) {
  constexpr int TW = moe::router::Cfg<TM, TN, WM, WN, SK, NSUB, NS>::TW;
  const dim3 grid((unsigned)((T + TW - 1) / TW)), block(256);
  if (K <= 2) {
    hipLaunchKernelGGL((moe::router::route_fused_lds_kernel<TM, TN, WM, WN, SK, NSUB, NS, 2>), grid, block, 0, s, x,
                       wr, bias, T, d, E, K, renorm, ids, w, logits, lr, cc, flag);
  } else if (K <= 8) {
    hipLaunchKernelGGL((moe::router::route_fused_lds_kernel<TM, TN, WM, WN, SK, NSUB, NS, 8>), grid, block, 0, s, x,
                       wr, bias, T, d, E, K, renorm, ids, w, logits, lr, cc, flag);
  } else {
    hipLaunchKernelGGL((moe::router::route_fused_lds_kernel<TM, TN, WM, WN, SK, NSUB, NS, 32>), grid, block, 0, s, x,
                       wr, bias, T, d, E, K, renorm, ids, w, logits, lr, cc, flag);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

template <int TM, int TN>
moe_status_t launch_reg(const uint16_t* x, const uint16_t* wr, const float* bias, int64_t T, int d, int E, int K,
                        int renorm, int32_t* ids, float* w, float* logits, int32_t* lr, int32_t* cc, uint32_t* flag,
                        hipStream_t s) {
  const dim3 grid((unsigned)((T + 16 * TM - 1) / (16 * TM))), block(256);
  if (K <= 2) {
    hipLaunchKernelGGL((moe::router::route_fused_reg_kernel<TM, TN, 2>), grid, block, 0, s, x, wr, bias, T, d, E, K,
                       renorm, ids, w, logits, lr, cc, flag);
  } else if (K <= 8) {
    hipLaunchKernelGGL((moe::router::route_fused_reg_kernel<TM, TN, 8>), grid, block, 0, s, x, wr, bias, T, d, E, K,
                       renorm, ids, w, logits, lr, cc, flag);
  } else {
    hipLaunchKernelGGL((moe::router::route_fused_reg_kernel<TM, TN, 32>), grid, block, 0, s, x, wr, bias, T, d, E, K,
                       renorm, ids, w, logits, lr, cc, flag);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
}  // namespace

// tokens per workgroup (= tokens per dispatch-histogram chunk) for E experts
extern "C" int moe_route_fused_tokens(int32_t E) { return E <= 32 ? 16 : E <= 64 ? 32 : 64; }

extern "C" moe_status_t moe_route_fused_launch(const uint16_t* x, const uint16_t* wr, const float* bias, int64_t T,
                                               int32_t d, int32_t E, int32_t K, int32_t renorm, int32_t* ids,
                                               float* w, float* logits, int32_t* local_rank, int32_t* chunk_counts,
                                               uint32_t* flag, hipStream_t s) {
  if (T == 0) return MOE_OK;
  if (E <= 32) return launch_reg<1, 2>(x, wr, bias, T, d, E, K, renorm, ids, w, logits, local_rank, chunk_counts, flag, s);
  if (E <= 64)
    return launch_lds<2, 2, 1, 2, 2, 4, 3>(x, wr, bias, T, d, E, K, renorm, ids, w, logits, local_rank, chunk_counts,
                                           flag, s);
  if (E <= 128)
    return launch_lds<2, 4, 2, 2, 1, 4, 3>(x, wr, bias, T, d, E, K, renorm, ids, w, logits, local_rank, chunk_counts,
                                           flag, s);
  return launch_lds<2, 8, 2, 2, 1, 2, 3>(x, wr, bias, T, d, E, K, renorm, ids, w, logits, local_rank, chunk_counts,
                                         flag, s);
}
