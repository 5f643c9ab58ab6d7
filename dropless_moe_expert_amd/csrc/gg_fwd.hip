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
//    hide behind the other's MFMAs (measured alternatives, all slower: one
//    wavefront per SIMD with 128 x 128 blocks and the accumulators in the
//    accumulation registers; MFMA 32x32x16 instead of 16x16x32; issuing the
//    next tile's first stages before storing the current one);
//  * K is staged 32 at a time (64-byte LDS rows, 16-byte slots swizzled by
//    (row >> 1) & 3, free of bank conflicts for the fragment reads) in
//    five named LDS buffers (all 160 KB), filled by direct-to-LDS loads
//    issued four stages ahead of the stage being read: loads from the
//    L2 / MALL / HBM take microseconds under load, and LDS capacity is what
//    bounds the bytes in flight; each stage waits only for its own loads;
//  * the MFMA fragments of stage kt + 1 are read into registers while the
//    MFMAs of stage kt run, so LDS latency and the per-stage barrier stay
//    off the MFMA pipe;
//  * the group of a tile is found by a wavefront scan over the device
//    group sizes (no LDS table), which leaves all of LDS to the stages;
//  * tiles are ordered in blocks of 4 m-tiles x all n-tiles and consecutive
//    tiles run on one XCD, so the 32 tiles an XCD holds at a time share
//    4 activation panels and 8 weight panels in its L2.
#include <type_traits>

#include "gg_pipeline.h"

namespace moe {
namespace fwd {

constexpr int WM = 4;                         // wavefront grid 4 (m) x 2 (n)
constexpr int NWAVE = WM * WN, THREADS = NWAVE * 64;
constexpr int WTM = BM / WM;                  // 64 x 128 per wavefront
constexpr int TM = WTM / 16, TN = WTN / 16;   // 4 x 8 MFMA subtiles
constexpr int LPW = (BM + BN) / 16 / NWAVE;   // direct loads per wavefront and stage (4)

// MFMA fragments of one stage: 8 W (n) and 4 X (m) 16x32 slices per lane
struct Frags {
  bf16x8_t w[TN], x[TM];
};

// Wavefront position in the tile: wn = wave / WM, and the m-block wm is
// rotated by 2 for wn = 1, so the two wavefronts of a SIMD (waves w and
// w + 4 when wavefronts are dealt round-robin to the SIMDs) own m-blocks
// two apart.  In a group's last, partial m-tile the wavefronts whose rows
// are all past the group's end skip their MFMAs; with this placement every
// SIMD then keeps about the same share of the remaining work.
__device__ __forceinline__ void wave_pos(int& wn, int& wm) {
  const int wave = wave_id();
  wn = wave / WM;
  wm = (wave % WM + 2 * wn) % WM;
}

// reads the W fragments and the first ACT X fragments (ACT = 0: nothing)
template <int ACT>
__device__ __forceinline__ void read_frags(const uint8_t* buf, Frags& fr) {
  if constexpr (ACT > 0) {
    const int lane = threadIdx.x & 63;
    int wn, wm;
    wave_pos(wn, wm);
    const int r16 = lane & 15, g4 = lane >> 4;
    // rows base + 16 i + r16 with 16 | base: the swizzle depends on r16 only
    const int slot = g4 ^ swz64(r16);
    const uint8_t* lw = buf + (wn * WTN + r16) * ROWB + slot * 16;
    const uint8_t* lx = buf + XOFF + (wm * WTM + r16) * ROWB + slot * 16;
#pragma unroll
    for (int j = 0; j < ACT; ++j)
      fr.x[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(lx + j * 16 * ROWB));
#pragma unroll
    for (int i = 0; i < TN; ++i)
      fr.w[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(lw + i * 16 * ROWB));
  }
}

// MFMAs of the first ACT 16-row subtiles of the wavefront's 64 rows
template <int ACT>
__device__ __forceinline__ void mma(const Frags& fr, f32x4_t (&acc)[TN][TM]) {
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < ACT; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr.w[i], fr.x[j], acc[i][j], 0, 0, 0);
}

// Stores the wavefront's 128 x 64 block.  Plain: column n0 + wn*WTN + 16i + 4*g4.
// SwiGLU: subtiles i < TN/2 hold gate column j = n0 + wn*WTN/2 + 16i + 4*g4 and
// subtile i + TN/2 the up column of the same j.
template <int EPI, int OUT>
__device__ __forceinline__ void store(const GGArgs& a, f32x4_t (&acc)[TN][TM], int64_t m0, int rows, int n0,
                                      int ncols, int f) {
  const int lane = threadIdx.x & 63;
  int wn, wm;
  wave_pos(wn, wm);
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

// Packed weights: for expert g, n-tile nt and K-stage kt the 256 weight rows
// of the tile (in the order the tile uses them) are one contiguous 16 KB
// block at ((g * n_tiles + nt) * nk + kt) * 16 KB, already in the LDS slot
// order, so each direct load reads 1 KB of consecutive bytes.
template <int EPI, int OUT, bool PACKED>
__global__ void __launch_bounds__(THREADS, 1) gg_fwd_kernel(GGArgs a) {
  // five named 32 KB stage buffers (the whole 160 KB LDS): stage kt lives in
  // buffer kt % 5; loads run four stages ahead of the stage being read
  __shared__ __align__(1024) uint8_t b0[STAGE];
  __shared__ __align__(1024) uint8_t b1[STAGE];
  __shared__ __align__(1024) uint8_t b2[STAGE];
  __shared__ __align__(1024) uint8_t b3[STAGE];
  __shared__ __align__(1024) uint8_t b4[STAGE];

  if (blockIdx.x == 0 && threadIdx.x < 64) {
    // data errors, reported once: negative sizes, rows past m_cap
    bool neg = false;
    int64_t tot = 0;
    for (int c = 0; c < a.G; c += 64) {
      const int gi = c + (int)threadIdx.x;
      const int32_t v = gi < a.G ? a.sizes[gi] : 0;
      neg |= v < 0;
      tot += max(v, 0);
    }
    tot = wave_sum(tot);
    if (__any(neg) && threadIdx.x == 0) raise_flag(a.flag, MOE_FLAG_NEGATIVE_SIZE);
    if (tot > a.m_cap && threadIdx.x == 0) raise_flag(a.flag, MOE_FLAG_ROWS_OVER_CAP);
  }

  const int wid = worker_id();
  const int f = a.N / 2;
  int64_t m_tiles = 0;
  locate(a, -1, &m_tiles);
  const int64_t total = m_tiles * a.n_tiles;
  const int64_t lda_b = (int64_t)a.K * 2;
  const int nk = a.K / 32;

  for (int64_t tile = wid; tile < total; tile += gridDim.x) {
    // tile order: blocks of GM m-tiles; inside a block m varies fastest
    const int64_t blk = tile / ((int64_t)GM * a.n_tiles);
    const int rem = (int)(tile - blk * GM * a.n_tiles);
    const int gm = (int)min<int64_t>(GM, m_tiles - blk * GM);
    const int64_t mt = blk * GM + rem % gm;
    const int nt = rem / gm;
    const TileGroup tg = locate(a, mt, nullptr);
    const int g = tg.g;
    const int64_t m0 = tg.row0 + (mt - tg.tile0) * BM;
    const int rows = (int)min<int64_t>(BM, tg.row1 - m0);
    const int n0 = (EPI == MOE_EPI_SWIGLU) ? nt * (BN / 2) : nt * BN;
    const int nrows_b = (EPI == MOE_EPI_SWIGLU) ? 2 * f : a.N;

    Rows<BM, NWAVE> xl;
    Rows<BN, NWAVE> wl;
    xl.init(lda_b, [&](int r) -> int64_t { return min(r, rows - 1); });
    if (!PACKED) wl.init(lda_b, [&](int r) -> int64_t {
      if constexpr (EPI == MOE_EPI_SWIGLU) {
        const int wn = r / WTN, q = r % WTN;
        const int jj = min(n0 + wn * (WTN / 2) + (q % (WTN / 2)), f - 1);
        return q < WTN / 2 ? jj : f + jj;
      } else {
        return min(n0 + r, a.N - 1);
      }
    });
    const uint8_t* xbase = a.A + m0 * lda_b;
    const uint8_t* wbase = PACKED ? a.B + ((int64_t)g * a.n_tiles + nt) * nk * (BN * ROWB)
                                  : a.B + (int64_t)g * nrows_b * lda_b;
    const int wstride = PACKED ? BN * ROWB : ROWB;   // bytes from one stage's weight block to the next
    if constexpr (PACKED) {
      const int wave = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < Rows<BN, NWAVE>::N; ++i) wl.off[i] = (uint32_t)(((i * NWAVE + wave) * 64 + lane) * 16);
    }

    f32x4_t acc[TN][TM];
#pragma unroll
    for (int i = 0; i < TN; ++i)
#pragma unroll
      for (int j = 0; j < TM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    auto issue = [&](uint8_t* buf, int kt) {
      wl.issue(buf, wbase + (int64_t)kt * wstride);
      xl.issue(buf + XOFF, xbase + kt * ROWB);
    };
    // wait until stage s has landed, given that stages up to s + 3 may have been issued
    auto wait_stage = [&](int s) {
      const int after = min(3, nk - 1 - s);
      if (after >= 3) {
        MOE_WAIT_VMCNT(3 * LPW);
      } else if (after == 2) {
        MOE_WAIT_VMCNT(2 * LPW);
      } else if (after == 1) {
        MOE_WAIT_VMCNT(LPW);
      } else {
        MOE_WAIT_VMCNT(0);
      }
      // every wavefront's fragment reads of the previous stage are done too
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt unconstrained
      asm volatile("s_barrier" ::: "memory");
    };
    // wavefronts whose 64 rows extend past the tile's valid rows skip the
    // MFMAs (and fragment reads) of the missing 16-row subtiles
    int wn_, wm_;
    wave_pos(wn_, wm_);
    const int act = min(TM, max(0, (rows - wm_ * WTM + 15) / 16));
    auto run = [&](auto act_c) {
      constexpr int ACT = decltype(act_c)::value;
      Frags fa, fb;
      // Step kt: the fragments of stage kt are in `cur`; stage kt + 1 (in nbuf)
      // is waited for, published by the barrier and read into `nxt` while the
      // MFMAs of stage kt run; stage kt's buffer (kbuf, now free) receives
      // stage kt + 5.  The fast form has no guards: conditional code around
      // the fragment reads makes the compiler wait for them (lgkmcnt(0)) at
      // the join, which would serialise LDS latency into the MFMA stream.
      auto step_fast = [&](Frags& cur, Frags& nxt, uint8_t* kbuf, uint8_t* nbuf, int kt) {
        MOE_WAIT_VMCNT(3 * LPW);
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): previous fragment reads done
        asm volatile("s_barrier" ::: "memory");
        issue(kbuf, kt + 5);
        read_frags<ACT>(nbuf, nxt);
        mma<ACT>(cur, acc);
      };
      auto step = [&](Frags& cur, Frags& nxt, uint8_t* kbuf, uint8_t* nbuf, int kt) {
        if (kt + 1 < nk) wait_stage(kt + 1);
        if (kt + 5 < nk) issue(kbuf, kt + 5);
        if (kt + 1 < nk) read_frags<ACT>(nbuf, nxt);
        mma<ACT>(cur, acc);
      };

      __syncthreads();  // every wavefront is done with the previous tile's buffers
      issue(b0, 0);
      if (nk > 1) issue(b1, 1);
      if (nk > 2) issue(b2, 2);
      if (nk > 3) issue(b3, 3);
      if (nk > 4) issue(b4, 4);
      {
        // stage 0 landed: stages 1..4 may still be in flight
        const int after = min(4, nk - 1);
        if (after >= 4) {
          MOE_WAIT_VMCNT(4 * LPW);
        } else if (after == 3) {
          MOE_WAIT_VMCNT(3 * LPW);
        } else if (after == 2) {
          MOE_WAIT_VMCNT(2 * LPW);
        } else if (after == 1) {
          MOE_WAIT_VMCNT(LPW);
        } else {
          MOE_WAIT_VMCNT(0);
        }
        asm volatile("s_barrier" ::: "memory");
      }
      read_frags<ACT>(b0, fa);
      int kt = 0;
      // groups of ten steps while every step of the group still issues a stage (kt + 14 < nk)
      for (; kt + 15 <= nk; kt += 10) {
        step_fast(fa, fb, b0, b1, kt);
        step_fast(fb, fa, b1, b2, kt + 1);
        step_fast(fa, fb, b2, b3, kt + 2);
        step_fast(fb, fa, b3, b4, kt + 3);
        step_fast(fa, fb, b4, b0, kt + 4);
        step_fast(fb, fa, b0, b1, kt + 5);
        step_fast(fa, fb, b1, b2, kt + 6);
        step_fast(fb, fa, b2, b3, kt + 7);
        step_fast(fa, fb, b3, b4, kt + 8);
        step_fast(fb, fa, b4, b0, kt + 9);
      }
      // the last (at most 14) steps, guarded; kt is a multiple of 10 here
      if (kt < nk) step(fa, fb, b0, b1, kt);
      if (kt + 1 < nk) step(fb, fa, b1, b2, kt + 1);
      if (kt + 2 < nk) step(fa, fb, b2, b3, kt + 2);
      if (kt + 3 < nk) step(fb, fa, b3, b4, kt + 3);
      if (kt + 4 < nk) step(fa, fb, b4, b0, kt + 4);
      if (kt + 5 < nk) step(fb, fa, b0, b1, kt + 5);
      if (kt + 6 < nk) step(fa, fb, b1, b2, kt + 6);
      if (kt + 7 < nk) step(fb, fa, b2, b3, kt + 7);
      if (kt + 8 < nk) step(fa, fb, b3, b4, kt + 8);
      if (kt + 9 < nk) step(fb, fa, b4, b0, kt + 9);
      if (kt + 10 < nk) step(fa, fb, b0, b1, kt + 10);
      if (kt + 11 < nk) step(fb, fa, b1, b2, kt + 11);
      if (kt + 12 < nk) step(fa, fb, b2, b3, kt + 12);
      if (kt + 13 < nk) step(fb, fa, b3, b4, kt + 13);
    };
    if (act == TM) {
      run(std::integral_constant<int, TM>());
    } else if (act == 3) {
      run(std::integral_constant<int, 3>());
    } else if (act == 2) {
      run(std::integral_constant<int, 2>());
    } else if (act == 1) {
      run(std::integral_constant<int, 1>());
    } else {
      run(std::integral_constant<int, 0>());
    }
    store<EPI, OUT>(a, acc, m0, rows, n0, EPI == MOE_EPI_SWIGLU ? f : a.N, f);
  }
}

// Packs W [G, rows_b, K] (rows_b = N, or 2f for SwiGLU) into the tile-stage
// blocks the PACKED kernel reads; rows past the weight's end are zero.
template <int EPI>
__global__ __launch_bounds__(256) void pack_weights_kernel(const uint16_t* __restrict__ w, int G, int N, int K,
                                                           int n_tiles, uint4* __restrict__ out) {
  const int nk = K / 32;
  const int64_t chunks = (int64_t)G * n_tiles * nk * BN * 4;   // 16-byte chunks
  const int f = N / 2;
  const int nrows_b = (EPI == MOE_EPI_SWIGLU) ? 2 * f : N;
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks; c += (int64_t)gridDim.x * blockDim.x) {
    const int slot = (int)(c & 3);
    const int r = (int)((c >> 2) % BN);
    const int64_t blk = (c >> 2) / BN;
    const int kt = (int)(blk % nk);
    const int64_t gn = blk / nk;
    const int nt = (int)(gn % n_tiles), g = (int)(gn / n_tiles);
    const int chunk = slot ^ swz64(r);
    int row;
    bool valid;
    if constexpr (EPI == MOE_EPI_SWIGLU) {
      const int n0 = nt * (BN / 2), wn = r / WTN, q = r % WTN;
      const int jj = n0 + wn * (WTN / 2) + (q % (WTN / 2));
      valid = jj < f;
      row = q < WTN / 2 ? jj : f + jj;
    } else {
      row = nt * BN + r;
      valid = row < N;
    }
    uint4 v = make_uint4(0, 0, 0, 0);
    if (valid) v = *reinterpret_cast<const uint4*>(w + ((int64_t)g * nrows_b + row) * K + kt * 32 + chunk * 8);
    out[c] = v;
  }
}

}  // namespace fwd

size_t packed_weight_bytes(int G, int N, int K, int epilogue) {
  const int ncols = epilogue == MOE_EPI_SWIGLU ? N / 2 : N;
  const int bn = epilogue == MOE_EPI_SWIGLU ? fwd::BN / 2 : fwd::BN;
  const int64_t n_tiles = (ncols + bn - 1) / bn;
  return (size_t)G * n_tiles * (K / 32) * fwd::BN * fwd::ROWB;
}

moe_status_t launch_pack_weights(const uint16_t* w, int G, int N, int K, int epilogue, void* out, hipStream_t s) {
  const int ncols = epilogue == MOE_EPI_SWIGLU ? N / 2 : N;
  const int bn = epilogue == MOE_EPI_SWIGLU ? fwd::BN / 2 : fwd::BN;
  const int n_tiles = (ncols + bn - 1) / bn;
  const int64_t chunks = (int64_t)G * n_tiles * (K / 32) * fwd::BN * 4;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((chunks + 255) / 256, (int64_t)moe_host::device_cu_count() * 16));
  if (epilogue == MOE_EPI_SWIGLU) {
    hipLaunchKernelGGL((fwd::pack_weights_kernel<MOE_EPI_SWIGLU>), dim3((unsigned)blocks), dim3(256), 0, s, w, G, N, K,
                       n_tiles, reinterpret_cast<uint4*>(out));
  } else {
    hipLaunchKernelGGL((fwd::pack_weights_kernel<MOE_EPI_NONE>), dim3((unsigned)blocks), dim3(256), 0, s, w, G, N, K,
                       n_tiles, reinterpret_cast<uint4*>(out));
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// bf16, ragged-M, B [G, N, K]: the forward kernels
moe_status_t launch_fwd(const GGArgs& a, int epilogue, int out_f32, int packed, hipStream_t s) {
  GGArgs b = a;
  const int ncols = epilogue == MOE_EPI_SWIGLU ? a.N / 2 : a.N;
  const int bn = epilogue == MOE_EPI_SWIGLU ? fwd::BN / 2 : fwd::BN;
  b.n_tiles = (ncols + bn - 1) / bn;
  const int64_t max_tiles = ((a.m_cap + fwd::BM - 1) / fwd::BM + a.G) * b.n_tiles;
  int64_t grid = moe_host::device_cu_count();
  if (max_tiles < grid) grid = max_tiles;
  if (grid <= 0) grid = 1;
  const dim3 g((unsigned)grid), t(fwd::THREADS);
  if (packed) {
    if (epilogue == MOE_EPI_SWIGLU) {
      hipLaunchKernelGGL((fwd::gg_fwd_kernel<MOE_EPI_SWIGLU, MOE_OUT_BF16, true>), g, t, 0, s, b);
    } else if (out_f32) {
      hipLaunchKernelGGL((fwd::gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_F32, true>), g, t, 0, s, b);
    } else {
      hipLaunchKernelGGL((fwd::gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_BF16, true>), g, t, 0, s, b);
    }
  } else if (epilogue == MOE_EPI_SWIGLU) {
    hipLaunchKernelGGL((fwd::gg_fwd_kernel<MOE_EPI_SWIGLU, MOE_OUT_BF16, false>), g, t, 0, s, b);
  } else if (out_f32) {
    hipLaunchKernelGGL((fwd::gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_F32, false>), g, t, 0, s, b);
  } else {
    hipLaunchKernelGGL((fwd::gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_BF16, false>), g, t, 0, s, b);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
