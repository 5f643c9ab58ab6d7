// Grouped GEMM, ragged along rows, bf16, K-contiguous weights: the forward
// expert matmuls (gate/up with the SwiGLU epilogue, and down).
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", section "Optimization 1: Grouped GEMM": one call for all experts,
// each with its true token count, only regions with valid tokens computed,
// counts never copied to the host.
//
// gfx950 design:
//  * persistent workgroups (one per CU) walk the tiles of the device-side
//    group prefix; grid size depends on host arguments only;
//  * 256 x 256 output tile, 8 wavefronts = 2 per SIMD (wavefront tile
//    128 n x 64 m, 8 x 4 MFMA 16x16x32 bf16), so one wavefront's LDS waits
//    hide behind the other's MFMAs;
//  * K is staged 32 at a time (64-byte LDS rows, 16-byte slots swizzled by
//    (row >> 2) & 3 so a fragment read touches 16 distinct bank groups) in
//    four named LDS buffers, filled by direct-to-LDS loads issued three
//    stages ahead; each stage waits only for its own loads (vmcnt);
//  * tiles are ordered in blocks of 4 m-tiles x all n-tiles and consecutive
//    tiles run on one XCD, so the 32 tiles an XCD holds at a time share
//    4 activation panels and 8 weight panels in its L2.
#include "gg_common.h"

namespace moe {
namespace fwd {

constexpr int BM = 256, BN = 256;   // tile rows (m) and columns (n)
constexpr int ROWB = 64;            // LDS bytes per row and stage (32 bf16)
constexpr int WM = 4, WN = 2;       // wavefront grid (m x n)
constexpr int NWAVE = WM * WN, THREADS = NWAVE * 64;
constexpr int WTM = BM / WM, WTN = BN / WN;   // 64 x 128 per wavefront
constexpr int TM = WTM / 16, TN = WTN / 16;   // 4 x 8 MFMA subtiles
constexpr int XOFF = BN * ROWB;               // X (activation) rows follow the W rows in a stage
constexpr int STAGE = (BM + BN) * ROWB;       // 32 KB
constexpr int GM = 4;                         // m-tiles per tile-order block
constexpr int LPW = (BM + BN) / 16 / NWAVE;   // direct loads per wavefront and stage (4)

// Direct-to-LDS rows: one wavefront instruction fills 16 rows (1 KB).  Lane l
// writes slot l & 3 of row 16*blk + l/4, which holds chunk (l & 3) ^ (l >> 4)
// of that row (the swizzle (row >> 2) & 3 equals l >> 4 for these rows).
template <int R>
struct Rows {
  static constexpr int N = R / 16 / NWAVE;
  uint32_t off[N];
  template <typename RowFn>
  __device__ __forceinline__ void init(int64_t ld_bytes, RowFn grow) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const int chunk = (lane & 3) ^ (lane >> 4);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int row = (i * NWAVE + wave) * 16 + (lane >> 2);
      off[i] = (uint32_t)(grow(row) * ld_bytes + chunk * 16);
    }
  }
  // The loads are written as inline asm: the compiler then does not track
  // them as LDS writes and inserts no wait of its own before the fragment
  // reads of other stage buffers; completion is enforced by the explicit
  // vmcnt wait of each stage.  Its own vector-memory waits only grow more
  // conservative (loads complete in order).
  __device__ __forceinline__ void issue(uint8_t* lds, const uint8_t* base) const {
    const int wave = wave_id();
    const uint32_t l0 = (uint32_t)(uintptr_t)(lds_ptr_t)lds + wave * 1024;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      asm volatile(
          "s_mov_b32 m0, %0\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dwordx4 %1, %2"
          :
          : "s"(l0 + i * NWAVE * 1024), "v"(off[i]), "s"(base)
          : "memory", "m0");
    }
  }
};

__device__ __forceinline__ void compute(const uint8_t* buf, f32x4_t (&acc)[TN][TM]) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int wn = wave / WM, wm = wave % WM;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int slot = g4 ^ ((r16 >> 2) & 3);
  const uint8_t* lw = buf + (wn * WTN + r16) * ROWB + slot * 16;
  const uint8_t* lx = buf + XOFF + (wm * WTM + r16) * ROWB + slot * 16;
  bf16x8_t wf[TN], xf[TM];
#pragma unroll
  for (int j = 0; j < TM; ++j) xf[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(lx + j * 16 * ROWB));
#pragma unroll
  for (int i = 0; i < TN; ++i) wf[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(lw + i * 16 * ROWB));
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < TM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i], xf[j], acc[i][j], 0, 0, 0);
}

// Stores the wavefront's 128 x 64 block.  Plain: column n0 + wn*WTN + 16i + 4*g4.
// SwiGLU: subtiles i < TN/2 hold gate column j = n0 + wn*WTN/2 + 16i + 4*g4 and
// subtile i + TN/2 the up column of the same j.
template <int EPI, int OUT>
__device__ __forceinline__ void store(const GGArgs& a, f32x4_t (&acc)[TN][TM], int64_t m0, int rows, int n0,
                                      int ncols, int f) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int wn = wave / WM, wm = wave % WM;
  const int r16 = lane & 15, g4 = lane >> 4;
  if constexpr (EPI == MOE_EPI_SWIGLU) {
    const int jbase = n0 + wn * (WTN / 2) + g4 * 4;
    if (a.Caux) {
      const int64_t lda = 2 * (int64_t)f;
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        const int mr = wm * WTM + j * 16 + r16;
#pragma unroll
        for (int i = 0; i < TN / 2; ++i) {
          const int jc = jbase + i * 16;
          if (mr < rows && jc < f) {
            store_sub<MOE_OUT_BF16>(a.Caux, lda, m0 + mr, jc, acc[i][j]);
            store_sub<MOE_OUT_BF16>(a.Caux, lda, m0 + mr, f + jc, acc[i + TN / 2][j]);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int mr = wm * WTM + j * 16 + r16;
#pragma unroll
      for (int i = 0; i < TN / 2; ++i) {
        const int jc = jbase + i * 16;
        f32x4_t h;
#pragma unroll
        for (int q = 0; q < 4; ++q) h[q] = silu_f32(acc[i][j][q]) * acc[i + TN / 2][j][q];
        if (mr < rows && jc < f) store_sub<MOE_OUT_BF16>(a.C, f, m0 + mr, jc, h);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int mr = wm * WTM + j * 16 + r16;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int n = n0 + wn * WTN + i * 16 + g4 * 4;
        if (mr < rows && n < ncols) store_sub<OUT>(a.C, ncols, m0 + mr, n, acc[i][j]);
      }
    }
  }
}

template <int EPI, int OUT>
__global__ void __launch_bounds__(THREADS, 1) gg_fwd_kernel(GGArgs a) {
  __shared__ __align__(1024) uint8_t b0[STAGE];
  __shared__ __align__(1024) uint8_t b1[STAGE];
  __shared__ __align__(1024) uint8_t b2[STAGE];
  __shared__ __align__(1024) uint8_t b3[STAGE];
  __shared__ GroupInfo<THREADS> gi;

  build_groups<THREADS, BM, true>(a, gi);

  const int wid = worker_id();
  const int f = a.N / 2;
  const int64_t m_tiles = gi.tpre[a.G];
  const int64_t total = m_tiles * a.n_tiles;
  const int64_t lda_b = (int64_t)a.K * 2;
  const int nk = a.K / 32;

  for (int64_t tile = wid; tile < total; tile += gridDim.x) {
    // tile order: blocks of GM m-tiles; inside a block m varies fastest
    const int64_t blk = tile / ((int64_t)GM * a.n_tiles);
    const int rem = (int)(tile - blk * GM * a.n_tiles);
    const int gm = (int)min<int64_t>(GM, m_tiles - blk * GM);
    const int mt = (int)(blk * GM) + rem % gm, nt = rem / gm;
    const int g = find_group(gi.tpre, a.G, mt);
    const int64_t m0 = gi.roff[g] + (int64_t)(mt - gi.tpre[g]) * BM;
    const int rows = (int)min<int64_t>(BM, gi.roff[g + 1] - m0);
    const int n0 = (EPI == MOE_EPI_SWIGLU) ? nt * (BN / 2) : nt * BN;
    const int nrows_b = (EPI == MOE_EPI_SWIGLU) ? 2 * f : a.N;

    Rows<BM> xl;
    Rows<BN> wl;
    xl.init(lda_b, [&](int r) -> int64_t { return min(r, rows - 1); });
    wl.init(lda_b, [&](int r) -> int64_t {
      if constexpr (EPI == MOE_EPI_SWIGLU) {
        const int wn = r / WTN, q = r % WTN;
        const int jj = min(n0 + wn * (WTN / 2) + (q % (WTN / 2)), f - 1);
        return q < WTN / 2 ? jj : f + jj;
      } else {
        return min(n0 + r, a.N - 1);
      }
    });
    const uint8_t* xbase = a.A + m0 * lda_b;
    const uint8_t* wbase = a.B + (int64_t)g * nrows_b * lda_b;

    f32x4_t acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](uint8_t* buf, int kt) {
      wl.issue(buf, wbase + kt * ROWB);
      xl.issue(buf + XOFF, xbase + kt * ROWB);
    };
    // stage kt lives in cur; stage kt + 3 is loaded into nxt (the buffer of stage kt - 1)
    auto step = [&](uint8_t* cur, uint8_t* nxt, int kt) {
      const int after = min(2, nk - 1 - kt);   // stages issued after kt that may still be in flight
      if (after >= 2) {
        MOE_WAIT_VMCNT(2 * LPW);
      } else if (after == 1) {
        MOE_WAIT_VMCNT(LPW);
      } else {
        MOE_WAIT_VMCNT(0);
      }
      // a plain s_barrier: the loads were waited for above, and the memory
      // clobber keeps the compiler from moving LDS reads across it
      asm volatile("s_barrier" ::: "memory");
      if (kt + 3 < nk) issue(nxt, kt + 3);
      compute(cur, acc);
    };

    __syncthreads();  // every wavefront is done with the previous tile's buffers
    issue(b0, 0);
    if (nk > 1) issue(b1, 1);
    if (nk > 2) issue(b2, 2);
    for (int kt = 0; kt < nk; kt += 4) {
      step(b0, b3, kt);
      if (kt + 1 < nk) step(b1, b0, kt + 1);
      if (kt + 2 < nk) step(b2, b1, kt + 2);
      if (kt + 3 < nk) step(b3, b2, kt + 3);
    }
    store<EPI, OUT>(a, acc, m0, rows, n0, EPI == MOE_EPI_SWIGLU ? f : a.N, f);
  }
}

}  // namespace fwd

// bf16, ragged-M, B [G, N, K]: the forward kernels
moe_status_t launch_fwd(const GGArgs& a, int epilogue, int out_f32, hipStream_t s) {
  GGArgs b = a;
  const int ncols = epilogue == MOE_EPI_SWIGLU ? a.N / 2 : a.N;
  const int bn = epilogue == MOE_EPI_SWIGLU ? fwd::BN / 2 : fwd::BN;
  b.n_tiles = (ncols + bn - 1) / bn;
  const int64_t max_tiles = ((a.m_cap + fwd::BM - 1) / fwd::BM + a.G) * b.n_tiles;
  int64_t grid = moe_host::device_cu_count();
  if (max_tiles < grid) grid = max_tiles;
  if (grid <= 0) grid = 1;
  const dim3 g((unsigned)grid), t(fwd::THREADS);
  if (epilogue == MOE_EPI_SWIGLU) {
    hipLaunchKernelGGL((fwd::gg_fwd_kernel<MOE_EPI_SWIGLU, MOE_OUT_BF16>), g, t, 0, s, b);
  } else if (out_f32) {
    hipLaunchKernelGGL((fwd::gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_F32>), g, t, 0, s, b);
  } else {
    hipLaunchKernelGGL((fwd::gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_BF16>), g, t, 0, s, b);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
