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
//  * 256 x 256 output tile, 8 wavefronts = 2 per SIMD, each owning 128 n x
//    64 m as 8 x 4 MFMA 16x16x32 bf16 accumulators; in a group's last,
//    partial tile a wavefront reads and multiplies only its 16-row subtiles
//    that hold valid rows (ACT of 4), and the two wavefronts of a SIMD own
//    row blocks two apart to share what is left.  Measured: dealing the
//    valid subtiles evenly to all wavefronts instead is 1.3 % slower, since
//    every wavefront then also reads the weight fragments (on a
//    power-limited chip, bytes moved cost as much as balance gains);
//  * ping-pong schedule: each K-stage is a memory phase (issue the loads of a
//    later stage, read this stage's fragments from LDS into registers) and a
//    compute phase (the stage's MFMAs from registers), separated by
//    workgroup barriers; the second wavefront of every SIMD runs one phase
//    behind the first, so one of the two issues MFMAs while the other waits
//    on LDS, and each needs a single set of fragment registers;
//  * K is staged 32 at a time (64-byte LDS rows, 16-byte slots swizzled by
//    (row >> 1) & 3, free of bank conflicts for the fragment reads) in
//    five named LDS buffers (all 160 KB), filled by direct-to-LDS loads
//    issued four stages ahead of the stage being read: loads from the
//    L2 / MALL / HBM take microseconds under load, and LDS capacity is what
//    bounds the bytes in flight; each stage waits only for its own loads;
//  * the group of a tile is found by a wavefront scan over the device
//    group sizes (no LDS table), which leaves all of LDS to the stages;
//  * tiles go group by group in blocks of about sqrt(32) m-tiles x all
//    n-tiles, and consecutive tiles run on one XCD, so the 32 tiles an XCD
//    holds at a time share a few activation and weight panels in its L2
//    and never mix two experts' weights.
// Measured on random operands, MI355X sustains about 70 % of its nominal
// bf16 MFMA rate for this fragment pattern even with no memory traffic
// (power-limited clocks); every byte moved lowers that further.
#include <atomic>
#include <type_traits>

#include "gg_pipeline.h"

namespace moe {
namespace fwd {

constexpr int WM = 4;                         // wavefront grid 4 (m) x 2 (n)
constexpr int NWAVE = WM * WN, THREADS = NWAVE * 64;
constexpr int WTM = BM / WM;                  // 64 x 128 per wavefront
constexpr int TM = WTM / 16, TN = WTN / 16;   // 4 x 8 MFMA subtiles
constexpr int LPW = (BM + BN) / 16 / NWAVE;   // direct loads per wavefront and stage (4)
static_assert(KRows<NWAVE>::N == Rows<BN, NWAVE>::N, "a K-outer weight stage takes as many loads as a row stage");

// weight (B) layouts of the kernel
enum { BL_NK = 0, BL_PACKED = 1, BL_KN = 2 };
// kernel-internal epilogue: SwiGLU that also stores the pre-activations
// (C_aux != NULL); its own instantiation keeps the h-only SwiGLU kernel lean
constexpr int EPI_SWIGLU_AUX = 7;
static_assert(EPI_SWIGLU_AUX != MOE_EPI_NONE && EPI_SWIGLU_AUX != MOE_EPI_SWIGLU &&
                  EPI_SWIGLU_AUX != MOE_EPI_SWIGLU_MXFP8 && EPI_SWIGLU_AUX != MOE_EPI_SWIGLU_BWD,
              "a kernel-internal epilogue value");
constexpr bool is_swiglu(int epi) { return epi == MOE_EPI_SWIGLU || epi == EPI_SWIGLU_AUX; }

// MFMA fragments of one stage: 8 W (n) and up to 4 X (m) 16x32 slices per lane
struct Frags {
  bf16x8_t w[TN], x[TM];
};

// Wavefront position in the tile: n-block wn = wave / WM (128 columns) and
// row slot wm, rotated by 2 for wn = 1 so that the two wavefronts of a SIMD
// (waves w and w + 4: wavefronts are dealt round-robin to the SIMDs) hold
// slots two apart.
__device__ __forceinline__ void wave_pos(int& wn, int& wm) {
  const int wave = wave_id();
  wn = wave / WM;
  wm = (wave % WM + 2 * wn) % WM;
}

// Row slot wm owns tile rows xrow0 = 64 * wm + [0, 64), of which the first
// act 16-row subtiles hold valid rows (0..4).
__device__ __forceinline__ void slot_rows(int rows, int wm, int& act, int& xrow0) {
  xrow0 = WTM * wm;
  act = min(TM, max(0, (rows - xrow0 + 15) / 16));
}

// reads the stage's W fragments and the wavefront's ACT X fragments (rows
// xrow0 + [0, 16 * ACT)); ACT = 0: nothing
template <int ACT, int BL>
__device__ __forceinline__ void read_frags(const uint8_t* buf, Frags& fr, int xrow0, const uint32_t (&koff)[TN]) {
  if constexpr (ACT == 0) return;
  const int lane = threadIdx.x & 63;
  int wn, wm;
  wave_pos(wn, wm);
  const int r16 = lane & 15, g4 = lane >> 4;
  // rows base + 16 i + r16 with 16 | base: the swizzle depends on r16 only
  const int slot = g4 ^ swz64(r16);
  const uint8_t* lw = buf + (wn * WTN + r16) * ROWB + slot * 16;
  const uint8_t* lx = buf + XOFF + (xrow0 + r16) * ROWB + slot * 16;
#pragma unroll
  for (int j = 0; j < ACT; ++j)
    fr.x[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(lx + j * 16 * ROWB));
  if constexpr (BL == BL_KN) {
#pragma unroll
    for (int i = 0; i < TN; ++i) fr.w[i] = kfrag_read(buf, koff[i]);
  } else {
#pragma unroll
    for (int i = 0; i < TN; ++i)
      fr.w[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4*>(lw + i * 16 * ROWB));
  }
}

// MFMAs of the wavefront's ACT 16-row subtiles, in serpentine order: the row
// subtile runs forwards for even weight fragments and backwards for odd ones,
// so consecutive MFMAs share an operand across the turn (measured 2-3 % faster
// than restarting each row on random operands, where the rate is power-bound)
template <int ACT>
__device__ __forceinline__ void mma(const Frags& fr, f32x4_t (&acc)[TN][TM]) {
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int jj = 0; jj < ACT; ++jj) {
      const int j = (i & 1) ? ACT - 1 - jj : jj;
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fr.w[i], fr.x[j], acc[i][j], 0, 0, 0);
    }
}

// Stores the wavefront's 128 x (16 * ACT) block (rows xrow0 + ...).  Plain: column n0 + wn*WTN + 16i + 4*g4.
// SwiGLU: subtiles i < TN/2 hold gate column j = n0 + wn*WTN/2 + 16i + 4*g4 and
// subtile i + TN/2 the up column of the same j.
template <int EPI, int OUT, int ACT>
__device__ __forceinline__ void store(const GGArgs& a, f32x4_t (&acc)[TN][TM], int64_t m0, int rows, int n0,
                                      int ncols, int f, int xrow0) {
  const int lane = threadIdx.x & 63;
  int wn, wm;
  wave_pos(wn, wm);
  const int r16 = lane & 15, g4 = lane >> 4;
  if constexpr (is_swiglu(EPI)) {
    const int jbase = n0 + wn * (WTN / 2) + g4 * 4;
    if (EPI == EPI_SWIGLU_AUX) {
      const int64_t lda = 2 * (int64_t)f;
#pragma unroll
      for (int j = 0; j < ACT; ++j) {
        const int mr = xrow0 + j * 16 + r16;
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
    for (int j = 0; j < ACT; ++j) {
      const int mr = xrow0 + j * 16 + r16;
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
    for (int j = 0; j < ACT; ++j) {
      const int mr = xrow0 + j * 16 + r16;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int n = n0 + wn * WTN + i * 16 + g4 * 4;
        if (mr < rows && n < ncols) store_sub<OUT>(a.C, ncols, m0 + mr, n, acc[i][j]);
      }
    }
  }
}

// Staged epilogue for bf16 outputs: every wavefront writes its rows
// xrow0 + [0, 64) of the tile into the stage buffer of its row slot (free once
// the K loop has waited for its last loads), 16-byte units XOR-swizzled by
// row so that the 16 rows one store instruction touches fall on distinct
// banks; after a barrier the workgroup copies whole tile rows out with
// 16-byte stores (the direct epilogue writes 32-byte pieces of 16 rows per
// instruction), each thread's LDS reads four at a time ahead of their
// stores.  ST_PLAIN: C [., ncols], the tile's 256 columns from n0 (512-byte
// rows); ST_H: SwiGLU's h, C [., f], 128 columns from n0 (256 bytes);
// ST_AUX: the pre-activations C_aux [., 2f], the tile's 128 gate columns
// from n0 then its 128 up columns from f + n0 (512 bytes).
// ST_BWD: the data gradient dh (staged as ST_PLAIN) leaves as SwiGLU's
// backward, C [., 2f] = [dg | du] from the forward's pre-activations in
// C_aux [., 2f] (read).
enum { ST_PLAIN = 0, ST_H = 1, ST_AUX = 2, ST_BWD = 3 };

// hp: ST_H takes h already rounded and packed (hp[i][j] for acc[i][j] and
// acc[i + TN/2][j]) instead of forming it from acc
template <int MODE, int ACT>
__device__ __forceinline__ void store_staged(const GGArgs& a, f32x4_t (&acc)[TN][TM], int64_t m0, int rows, int n0,
                                             int ncols, int f, int xrow0, uint8_t* s0, uint8_t* s1, uint8_t* s2,
                                             uint8_t* s3, const uint2 (*hp)[TM] = nullptr) {
  auto buf = [&](int i) { return i == 0 ? s0 : i == 1 ? s1 : i == 2 ? s2 : s3; };
  constexpr int RB = MODE == ST_H ? 256 : 512;   // bytes per staged row
  constexpr int UR = RB / 16;                    // 16-byte units per row
  const int lane = threadIdx.x & 63;
  int wn, wm;
  wave_pos(wn, wm);
  const int r16 = lane & 15, g4 = lane >> 4;
  uint8_t* sb = buf(xrow0 / WTM);
  auto put = [&](int rl, int col, uint2 w) {
    const int u = col >> 3, half = (col >> 2) & 1;
    *reinterpret_cast<uint2*>(sb + rl * RB + ((u ^ (rl % UR)) << 4) + half * 8) = w;
  };
  auto pack4 = [](const f32x4_t& v) { return make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])); };
#pragma unroll
  for (int j = 0; j < ACT; ++j) {
    const int rl = j * 16 + r16;   // row within the slot
    if constexpr (MODE == ST_PLAIN || MODE == ST_BWD) {
#pragma unroll
      for (int i = 0; i < TN; ++i) put(rl, wn * WTN + i * 16 + g4 * 4, pack4(acc[i][j]));
    } else {
#pragma unroll
      for (int i = 0; i < TN / 2; ++i) {
        const int col = wn * (WTN / 2) + i * 16 + g4 * 4;
        if constexpr (MODE == ST_H) {
          if (hp) {
            put(rl, col, hp[i][j]);
          } else {
            f32x4_t h;
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = silu_f32(acc[i][j][q]) * acc[i + TN / 2][j][q];
            put(rl, col, pack4(h));
          }
        } else {
          put(rl, col, pack4(acc[i][j]));                  // gate
          put(rl, BN / 2 + col, pack4(acc[i + TN / 2][j]));  // up
        }
      }
    }
  }
  __syncthreads();
  constexpr int NPT = BM * UR / THREADS;   // 16-byte pieces per thread
  constexpr int NB = 4;
  static_assert(BM * UR % THREADS == 0 && NPT % NB == 0, "whole batches");
  if constexpr (MODE == ST_BWD) {
    // SwiGLU backward of each 8-column piece of dh: its gate and up pieces
    // (C_aux, row pitch 2f) come in one batch ahead, so a batch's loads are
    // in flight while the batch before it is formed and stored; dg and du
    // go to C (row pitch 2f) at the piece's column and f + that column
    const int64_t ld2 = 2 * (int64_t)ncols;   // ncols = f
    const uint8_t* const gbase = a.Caux + m0 * ld2 * 2;
    uint8_t* const cbase = a.C + m0 * ld2 * 2;
    auto piece = [&](int k, int& row, int& col) {
      const int c = threadIdx.x + k * THREADS;
      row = c / UR;
      col = n0 + 8 * (c - row * UR);
    };
    uint4 gv0[NB], uv0[NB], gv1[NB], uv1[NB];
    auto load = [&](int k0, uint4 (&gv)[NB], uint4 (&uv)[NB]) {
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        int row, col;
        piece(k0 + k, row, col);
        if (row < rows && col < ncols) {
          const uint32_t o = (uint32_t)(row * ld2 + col) * 2u;
          gv[k] = *reinterpret_cast<const uint4*>(gbase + o);
          uv[k] = *reinterpret_cast<const uint4*>(gbase + o + (uint32_t)ncols * 2u);
        }
      }
    };
    // batch k0 (its gate and up pieces in gv, uv): issue the next batch's
    // loads into (gn, un), then form and store this one
    auto batch = [&](int k0, const uint4 (&gv)[NB], const uint4 (&uv)[NB], uint4 (&gn)[NB], uint4 (&un)[NB]) {
      uint4 v[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        const int c = threadIdx.x + (k0 + k) * THREADS;
        const int row = c / UR, u = c - row * UR;
        const int rl = row % WTM;
        v[k] = *reinterpret_cast<const uint4*>(buf(row / WTM) + rl * RB + ((u ^ (rl % UR)) << 4));
      }
      if (k0 + NB < NPT) load(k0 + NB, gn, un);
#pragma unroll
      for (int k = 0; k < NB; ++k) {
        int row, col;
        piece(k0 + k, row, col);
        if (row < rows && col < ncols) {
          float g[8], uu[8], dh[8], dg[8], du[8];
          unpack8(gv[k], g);
          unpack8(uv[k], uu);
          unpack8(v[k], dh);   // dh as stored: rounded to bf16
#pragma unroll
          for (int e = 0; e < 8; ++e) swiglu_grad(g[e], uu[e], dh[e], dg[e], du[e]);
          const uint32_t o = (uint32_t)(row * ld2 + col) * 2u;
          *reinterpret_cast<uint4*>(cbase + o) = pack8(dg);
          *reinterpret_cast<uint4*>(cbase + o + (uint32_t)ncols * 2u) = pack8(du);
        }
      }
    };
    static_assert(NPT % (2 * NB) == 0, "whole pairs of batches");
    load(0, gv0, uv0);
#pragma unroll 1
    for (int k0 = 0; k0 < NPT; k0 += 2 * NB) {
      batch(k0, gv0, uv0, gv1, uv1);
      batch(k0 + NB, gv1, uv1, gv0, uv0);
    }
    return;
  }
  // the tile's rows start at a uniform base; a piece is a 32-bit offset
  // from it (256 rows of at most 2^22 bf16 columns)
  const int ld = MODE == ST_PLAIN ? ncols : MODE == ST_H ? f : 2 * f;
  uint8_t* const cbase = (MODE == ST_AUX ? a.Caux : a.C) + m0 * (int64_t)ld * 2;
#pragma unroll 1
  for (int k0 = 0; k0 < NPT; k0 += NB) {   // rolled: per-piece addresses stay local to the epilogue
    uint4 v[NB];
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int c = threadIdx.x + (k0 + k) * THREADS;
      const int row = c / UR, u = c - row * UR;
      const int rl = row % WTM;
      v[k] = *reinterpret_cast<const uint4*>(buf(row / WTM) + rl * RB + ((u ^ (rl % UR)) << 4));
    }
#pragma unroll
    for (int k = 0; k < NB; ++k) {
      const int c = threadIdx.x + (k0 + k) * THREADS;
      const int row = c / UR, u = c - row * UR;
      int col, lim;
      if constexpr (MODE == ST_AUX) {
        const int uh = u % (UR / 2);
        col = (u < UR / 2 ? 0 : f) + n0 + 8 * uh;
        lim = (u < UR / 2 ? 0 : f) + f;
      } else {
        col = n0 + 8 * u;
        lim = MODE == ST_PLAIN ? ncols : f;
      }
      if (row < rows && col < lim) *reinterpret_cast<uint4*>(cbase + (uint32_t)(row * ld + col) * 2u) = v[k];
    }
  }
}

// ------------------------------------------------------------------ split tail
// (split_tail and its counters: gg_pipeline.h)
__device__ SplitSlots g_split_sched = initial_split_slots();

// Unit tail_unit (tile tail_unit / S, split tail_unit % S) has its partial
// sums in acc.  Returns true, with acc holding the tile's full sums, to the
// unit that completes the tile; false to the others.  box: one int of LDS
// that no wavefront reads or writes once it has left its K loop.
template <int ACT>
__device__ __forceinline__ bool split_reduce(const GGArgs& a, const SplitTail& sp, int64_t tail_unit,
                                             f32x4_t (&acc)[TN][TM], int32_t* box) {
  constexpr int SLOT = BM * BN;   // floats per unit
  const int t = threadIdx.x;
  const int64_t tile_tail = tail_unit / sp.S;
  float* const mine = a.part + tail_unit * SLOT;
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < ACT; ++j)
      *reinterpret_cast<f32x4_t*>(mine + ((i * TM + j) * THREADS + t) * 4) = acc[i][j];
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // this thread's partials are visible to the device
  __syncthreads();                                      // every thread's, and every wavefront has left its K loop
  if (t == 0) {
    DeviceWord w{g_split_sched.w[a.sched_slot] + tile_tail};
    box[0] = (int32_t)tq::take(w, a.sched_epoch) == sp.S - 1;
  }
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(box[0])) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the other units' partials
  const float* const first = a.part + tile_tail * sp.S * SLOT;
#pragma unroll
  for (int i = 0; i < TN; ++i)
#pragma unroll
    for (int j = 0; j < ACT; ++j) {
      const int64_t off = ((i * TM + j) * THREADS + t) * 4;
      f32x4_t v = *reinterpret_cast<const f32x4_t*>(first + off);
      for (int q = 1; q < sp.S; ++q) v += *reinterpret_cast<const f32x4_t*>(first + q * SLOT + off);
      acc[i][j] = v;
    }
  return true;
}

// Weight layouts (BL): BL_NK reads B [G, N, K] rows (K contiguous); BL_PACKED
// reads the tile-stage blocks of moe_pack_weights: for expert g, n-tile nt
// and K-stage kt the 256 weight rows of the tile (in the order the tile uses
// them) are one contiguous 16 KB block at ((g * n_tiles + nt) * nk + kt) *
// 16 KB, already in the LDS slot order, so each direct load reads 1 KB of
// consecutive bytes; BL_KN reads B [G, K, N] (the data gradient's weight)
// as K-outer stages, 32 rows of 256 columns, through LDS transpose reads.
template <int EPI, int OUT, int BL, bool SPLIT = false>
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
  const int64_t total = count_mtiles(a) * a.n_tiles;
  const int64_t lda_b = (int64_t)a.K * 2;
  const int nk_all = a.K / 32;
  uint32_t koff[TN];   // BL_KN: per-lane LDS offsets of the 8 weight fragments
  {
    int wn, wm;
    wave_pos(wn, wm);
#pragma unroll
    for (int i = 0; i < TN; ++i) koff[i] = BL == BL_KN ? kfrag_off(wn * WTN + 16 * i) : 0u;
  }

  // units: whole tiles, then (SPLIT) the split tail's stage ranges
  const SplitTail sp = SPLIT ? split_tail(total, (int)gridDim.x, nk_all) : SplitTail{total, total, 1};
  for (int64_t unit = wid; unit < sp.units; unit += gridDim.x) {
    int64_t tile = unit, tail_unit = -1;
    int kt0 = 0, nk = nk_all;   // the unit's first stage and stage count
    if constexpr (SPLIT) {
      if (unit >= sp.full) {
        tail_unit = unit - sp.full;
        tile = sp.full + tail_unit / sp.S;
        const int part = (int)(tail_unit % sp.S);
        kt0 = (int)((int64_t)part * nk_all / sp.S);
        nk = (int)((int64_t)(part + 1) * nk_all / sp.S) - kt0;
      }
    }
    const TileGroup tg = locate(a, tile);
    const int g = tg.g, nt = tg.nt;
    const int64_t m0 = tg.m0;
    const int rows = tg.rows;
    const int n0 = is_swiglu(EPI) ? nt * (BN / 2) : nt * BN;
    const int nrows_b = is_swiglu(EPI) ? 2 * f : a.N;

    Rows<BM, NWAVE> xl;
    Rows<BN, NWAVE> wl;
    KRows<NWAVE> kl;
    xl.init(lda_b, [&](int r) -> int64_t { return min(r, rows - 1); });
    if constexpr (BL == BL_KN) kl.init((int64_t)a.N * 2, n0, a.N);
    if constexpr (BL == BL_NK) wl.init(lda_b, [&](int r) -> int64_t {
      if constexpr (is_swiglu(EPI)) {
        const int wn = r / WTN, q = r % WTN;
        const int jj = min(n0 + wn * (WTN / 2) + (q % (WTN / 2)), f - 1);
        return q < WTN / 2 ? jj : f + jj;
      } else {
        return min(n0 + r, a.N - 1);
      }
    });
    // bytes from one stage's weight block to the next
    const int wstride = BL == BL_PACKED ? BN * ROWB : BL == BL_KN ? 32 * a.N * 2 : ROWB;
    // operands from the unit's first stage kt0 on
    const uint8_t* xbase = a.A + m0 * lda_b + (int64_t)kt0 * ROWB;
    const uint8_t* wbase = (BL == BL_PACKED ? a.B + ((int64_t)g * a.n_tiles + nt) * nk_all * (BN * ROWB)
                            : BL == BL_KN   ? a.B + (int64_t)g * a.K * a.N * 2
                                            : a.B + (int64_t)g * nrows_b * lda_b) +
                           (int64_t)kt0 * wstride;
    if constexpr (BL == BL_PACKED) {
      const int wave = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < Rows<BN, NWAVE>::N; ++i) wl.off[i] = (uint32_t)(((i * NWAVE + wave) * 64 + lane) * 16);
    }

    auto issue = [&](uint8_t* buf, int kt) {
      if constexpr (BL == BL_KN) {
        kl.issue(buf, wbase + (int64_t)kt * wstride);
      } else {
        wl.issue(buf, wbase + (int64_t)kt * wstride);
      }
      xl.issue(buf + XOFF, xbase + kt * ROWB);
    };
    // Waits until this wavefront's loads of stage s + 1 have landed (stages
    // up to min(s + 4, nk - 1) may have been issued) and its fragment reads
    // are done, then the workgroup barrier.  The scheduling fences keep the
    // compiler from moving MFMAs across the barrier.
    auto sync = [&](int s) {
      const int after = min(3, nk - 2 - s);
      __builtin_amdgcn_sched_barrier(0);
      if (after >= 3) {
        MOE_WAIT_VMCNT(3 * LPW);
      } else if (after == 2) {
        MOE_WAIT_VMCNT(2 * LPW);
      } else if (after == 1) {
        MOE_WAIT_VMCNT(LPW);
      } else {
        MOE_WAIT_VMCNT(0);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0), vmcnt/expcnt unconstrained
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    // the first wavefront of each SIMD is waves 0..3, the second 4..7
    const bool second = wave_id() >= NWAVE / 2;
    int wn_, wm_, act, xrow0;
    wave_pos(wn_, wm_);
    slot_rows(rows, wm_, act, xrow0);
    auto run = [&](auto act_c) {
      constexpr int ACT = decltype(act_c)::value;
      f32x4_t acc[TN][TM];
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      Frags fr;
      // Iteration s: memory phase (issue stage s + 4 into the buffer of
      // stage s - 1, which every wavefront finished reading before the last
      // barrier; read the fragments of stage s), barrier, compute phase,
      // barrier.  The second wavefronts start one barrier later, so their
      // memory phase runs beside the first wavefronts' compute phase and
      // the other way round; they skip the final barrier to even the count.
      auto iter = [&](uint8_t* sbuf, uint8_t* lbuf, int s) {
        if (s + 4 < nk) issue(lbuf, s + 4);
        read_frags<ACT, BL>(sbuf, fr, xrow0, koff);
        sync(s);
        mma<ACT>(fr, acc);
        if (!(second && s == nk - 1)) sync(s);
      };
      __syncthreads();  // every wavefront is done with the previous tile's buffers
      issue(b0, 0);
      if (nk > 1) issue(b1, 1);
      if (nk > 2) issue(b2, 2);
      if (nk > 3) issue(b3, 3);
      sync(-1);                 // stage 0 landed
      if (second) sync(-1);     // the half-step offset
      int s = 0;
      for (; s + 5 <= nk; s += 5) {
        iter(b0, b4, s);
        iter(b1, b0, s + 1);
        iter(b2, b1, s + 2);
        iter(b3, b2, s + 3);
        iter(b4, b3, s + 4);
      }
      if (s < nk) iter(b0, b4, s);
      if (s + 1 < nk) iter(b1, b0, s + 1);
      if (s + 2 < nk) iter(b2, b1, s + 2);
      if (s + 3 < nk) iter(b3, b2, s + 3);
      if constexpr (SPLIT) {
        // a split unit: partial sums to the workspace; the unit that
        // completes the tile adds them, in split order, and runs the epilogue
        if (tail_unit >= 0 && !split_reduce<ACT>(a, sp, tail_unit, acc, reinterpret_cast<int32_t*>(b4))) return;
      }
      if constexpr (OUT == MOE_OUT_BF16 && EPI == EPI_SWIGLU_AUX) {
        // h formed and packed first, so the accumulators are free once the
        // pre-activations are in LDS; then (once every thread has read
        // those out) h
        uint2 hp[TN / 2][TM];
#pragma unroll
        for (int j = 0; j < ACT; ++j)
#pragma unroll
          for (int i = 0; i < TN / 2; ++i) {
            f32x4_t h;
#pragma unroll
            for (int q = 0; q < 4; ++q) h[q] = silu_f32(acc[i][j][q]) * acc[i + TN / 2][j][q];
            hp[i][j] = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
          }
        store_staged<ST_AUX, ACT>(a, acc, m0, rows, n0, 0, f, xrow0, b0, b1, b2, b3);
        __syncthreads();
        store_staged<ST_H, ACT>(a, acc, m0, rows, n0, 0, f, xrow0, b0, b1, b2, b3, hp);
      } else if constexpr (OUT == MOE_OUT_BF16 && EPI == MOE_EPI_SWIGLU_BWD) {
        store_staged<ST_BWD, ACT>(a, acc, m0, rows, n0, a.N, f, xrow0, b0, b1, b2, b3);
      } else if constexpr (OUT == MOE_OUT_BF16) {
        store_staged<EPI == MOE_EPI_SWIGLU ? ST_H : ST_PLAIN, ACT>(a, acc, m0, rows, n0, a.N, f, xrow0, b0, b1, b2,
                                                                  b3);
      } else {
        store<EPI, OUT, ACT>(a, acc, m0, rows, n0, is_swiglu(EPI) ? f : a.N, f, xrow0);
      }
    };
    if (act == 4) {
      run(std::integral_constant<int, 4>());
    } else if (act == 3) {
      run(std::integral_constant<int, 3>());
    } else if (act == 2) {
      run(std::integral_constant<int, 2>());
    } else if (act == 1) {
      run(std::integral_constant<int, 1>());
    } else {
      run(std::integral_constant<int, 0>());
    }
  }
  if constexpr (SPLIT) {
    if (sp.S > 1) split_finish(a, g_split_sched.w[a.sched_slot], reinterpret_cast<int32_t*>(b4));
  }
}

// Weight gradient, ragged along the contraction: C[g] [P, Q] = sum over the
// rows r of group g of A[r, p] * B[r, q] with A [m_cap, P], B [m_cap, Q]
// (page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", section "Optimization 1: Grouped GEMM": every expert's matmul in
// one call, each over its true token count).  Both operands are K-outer
// stages (32 rows of 256 columns, transpose reads) on the same ping-pong
// schedule, in four 32 KB buffers (loads three stages ahead): the rest of LDS
// holds each workgroup's copy of the group row offsets and of the group order,
// largest group first, so the longest contractions start first.  A group's
// last stage re-reads its last row into the missing rows and zeroes those
// k-elements of the activation fragments.  Empty groups store zeros.
constexpr int WG_STAGES = 4;

// Tile queues of the weight-gradient kernel: one slot of tile_queue.h's
// words per launch (the host hands out epochs and slots in turn, so launches
// in flight together use different slots).
__device__ tq::Slots g_wgrad_sched = tq::initial_slots();

template <int OUT>
__global__ void __launch_bounds__(THREADS, 1) gg_wgrad_kernel(GGArgs a) {
  __shared__ __align__(1024) uint8_t b0[STAGE];
  __shared__ __align__(1024) uint8_t b1[STAGE];
  __shared__ __align__(1024) uint8_t b2[STAGE];
  __shared__ __align__(1024) uint8_t b3[STAGE];
  __shared__ GroupInfo<THREADS> gi;
  build_groups<THREADS>(a, gi);

  const int P = a.M, Q = a.N;
  const int per_group = a.p_tiles * a.n_tiles;
  const int64_t lda = (int64_t)P * 2, ldb = (int64_t)Q * 2;
  const int lane = threadIdx.x & 63;
  int wn, wm;
  wave_pos(wn, wm);
  uint32_t kw[TN], kx[TM];   // per-lane LDS offsets of the fragments
#pragma unroll
  for (int i = 0; i < TN; ++i) kw[i] = kfrag_off(wn * WTN + 16 * i);
#pragma unroll
  for (int j = 0; j < TM; ++j) kx[j] = XOFF + kfrag_off(wm * WTM + 16 * j);
  const bool second = wave_id() >= NWAVE / 2;

  // one tile: rem-th of the group of rank `rank` (groups ranked largest first)
  auto process = [&](int rank, int rem) {
    const int g = gi.tpre[rank];
    const int pt = rem / a.n_tiles, qt = rem - pt * a.n_tiles;
    const int p0 = pt * BM, q0 = qt * BN;
    const int64_t r0 = gi.roff[g];
    const int len = gi.roff[g + 1] - gi.roff[g];
    const int nk = (len + 31) / 32;
    const int rows = min(BM, P - p0);
    int act, xrow0;
    slot_rows(rows, wm, act, xrow0);

    KRows<NWAVE> al, bl;
    al.init(lda, p0, P);
    bl.init(ldb, q0, Q);
    const uint8_t* abase = a.A + r0 * lda;
    const uint8_t* bbase = a.B + r0 * ldb;
    auto issue = [&](uint8_t* buf, int kt) {
      const int kv = len - 32 * kt;
      if (kv >= 32) {
        bl.issue(buf, bbase + (int64_t)kt * 32 * ldb);
        al.issue(buf + XOFF, abase + (int64_t)kt * 32 * lda);
      } else {
        bl.issue_partial(buf, bbase + (int64_t)kt * 32 * ldb, kv, ldb);
        al.issue_partial(buf + XOFF, abase + (int64_t)kt * 32 * lda, kv, lda);
      }
    };
    auto sync = [&](int s) {
      const int after = min(WG_STAGES - 2, nk - 2 - s);
      __builtin_amdgcn_sched_barrier(0);
      if (after >= 2) {
        MOE_WAIT_VMCNT(2 * LPW);
      } else if (after == 1) {
        MOE_WAIT_VMCNT(LPW);
      } else {
        MOE_WAIT_VMCNT(0);
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    auto run = [&](auto act_c) {
      constexpr int ACT = decltype(act_c)::value;
      f32x4_t acc[TN][TM];
#pragma unroll
      for (int i = 0; i < TN; ++i)
#pragma unroll
        for (int j = 0; j < TM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      Frags fr;
      auto read = [&](const uint8_t* buf, int s) {
        if constexpr (ACT > 0) {
#pragma unroll
          for (int i = 0; i < TN; ++i) fr.w[i] = kfrag_read(buf, kw[i]);
#pragma unroll
          for (int j = 0; j < ACT; ++j) fr.x[j] = kfrag_read(buf, kx[j]);
          const int kv = len - 32 * s;
          if (kv < 32) {
            // k-elements past the group's rows: lane holds k = 8 (lane / 16) + e
            const int k0 = 8 * (lane >> 4);
#pragma unroll
            for (int j = 0; j < ACT; ++j) {
              s16x8_t v = __builtin_bit_cast(s16x8_t, fr.x[j]);
#pragma unroll
              for (int e = 0; e < 8; ++e) v[e] = (k0 + e < kv) ? v[e] : (short)0;
              fr.x[j] = __builtin_bit_cast(bf16x8_t, v);
            }
          }
        }
      };
      auto iter = [&](uint8_t* sbuf, uint8_t* lbuf, int s) {
        if (s + WG_STAGES - 1 < nk) issue(lbuf, s + WG_STAGES - 1);
        read(sbuf, s);
        sync(s);
        mma<ACT>(fr, acc);
        if (!(second && s == nk - 1)) sync(s);
      };
      __syncthreads();  // every wavefront is done with the previous tile's buffers
      if (nk > 0) {
        issue(b0, 0);
        if (nk > 1) issue(b1, 1);
        if (nk > 2) issue(b2, 2);
        sync(-1);
        if (second) sync(-1);
        int s = 0;
        for (; s + 4 <= nk; s += 4) {
          iter(b0, b3, s);
          iter(b1, b0, s + 1);
          iter(b2, b1, s + 2);
          iter(b3, b2, s + 3);
        }
        if (s < nk) iter(b0, b3, s);
        if (s + 1 < nk) iter(b1, b0, s + 1);
        if (s + 2 < nk) iter(b2, b1, s + 2);
      }
      GGArgs ag = a;
      ag.C = a.C + (int64_t)g * P * Q * (OUT == MOE_OUT_F32 ? 4 : 2);
      if constexpr (OUT == MOE_OUT_BF16) {
        store_staged<ST_PLAIN, ACT>(ag, acc, p0, rows, q0, Q, 0, xrow0, b0, b1, b2, b3);
      } else {
        store<MOE_EPI_NONE, OUT, ACT>(ag, acc, p0, rows, q0, Q, 0, xrow0);
      }
    };
    if (act == 4) {
      run(std::integral_constant<int, 4>());
    } else if (act == 3) {
      run(std::integral_constant<int, 3>());
    } else if (act == 2) {
      run(std::integral_constant<int, 2>());
    } else if (act == 1) {
      run(std::integral_constant<int, 1>());
    } else {
      run(std::integral_constant<int, 0>());
    }
  };

  // Dynamic tile queues (tq_walk): groups by size rank, largest first, each
  // group's tiles in a row; taking a tile is one atomic add.
  tq_walk(g_wgrad_sched.w[a.sched_slot], a.sched_epoch, a.sched_next, a.G, per_group, process);
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

// workspace of the bf16 ragged-M kernel's split tail: one fp32 tile per worker
size_t fwd_split_workspace_bytes() {
  return (size_t)moe_host::device_cu_count() * fwd::BM * fwd::BN * sizeof(float);
}

// bf16, ragged-M: the forward kernels (B [G, N, K] rows or packed) and the
// data gradient (B [G, K, N])
moe_status_t launch_fwd(const GGArgs& a, int epilogue, int out_f32, int b_layout, hipStream_t s) {
  static std::atomic<uint64_t> launches{0};
  GGArgs b = a;
  const int ncols = epilogue == MOE_EPI_SWIGLU ? a.N / 2 : a.N;
  const int bn = epilogue == MOE_EPI_SWIGLU ? fwd::BN / 2 : fwd::BN;
  b.n_tiles = (ncols + bn - 1) / bn;
  const int64_t max_tiles = ((a.m_cap + fwd::BM - 1) / fwd::BM + a.G) * b.n_tiles;
  int64_t grid = moe_host::device_cu_count();
  if (max_tiles < grid) grid = max_tiles;
  if (grid <= 0) grid = 1;
  const dim3 g((unsigned)grid), t(fwd::THREADS);
  using namespace fwd;
  // The split-tail instantiation (where a short last round is likely and
  // costs a large share of the call); other calls keep the plain kernel.
  if (use_split_tail(b.part != nullptr, max_tiles, grid, a.K / 32)) {
    const uint64_t n = launches.fetch_add(1u, std::memory_order_relaxed);
    b.sched_slot = tq::launch_slot(n);
    b.sched_epoch = tq::launch_epoch(n);
    b.sched_next = tq::slot_next_epoch(n);
    if (b_layout == MOE_B_KN) {
      if (epilogue == MOE_EPI_SWIGLU) return MOE_ERR_UNSUPPORTED;
      if (epilogue == MOE_EPI_SWIGLU_BWD) {
        hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_SWIGLU_BWD, MOE_OUT_BF16, BL_KN, true>), g, t, 0, s, b);
      } else if (out_f32) {
        hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_F32, BL_KN, true>), g, t, 0, s, b);
      } else {
        hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_BF16, BL_KN, true>), g, t, 0, s, b);
      }
    } else if (epilogue == MOE_EPI_SWIGLU && a.Caux) {
      if (b_layout == MOE_B_PACKED) {
        hipLaunchKernelGGL((gg_fwd_kernel<EPI_SWIGLU_AUX, MOE_OUT_BF16, BL_PACKED, true>), g, t, 0, s, b);
      } else {
        hipLaunchKernelGGL((gg_fwd_kernel<EPI_SWIGLU_AUX, MOE_OUT_BF16, BL_NK, true>), g, t, 0, s, b);
      }
    } else if (epilogue == MOE_EPI_SWIGLU) {
      if (b_layout == MOE_B_PACKED) {
        hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_SWIGLU, MOE_OUT_BF16, BL_PACKED, true>), g, t, 0, s, b);
      } else {
        hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_SWIGLU, MOE_OUT_BF16, BL_NK, true>), g, t, 0, s, b);
      }
    } else if (b_layout == MOE_B_PACKED) {
      if (out_f32) {
        hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_F32, BL_PACKED, true>), g, t, 0, s, b);
      } else {
        hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_BF16, BL_PACKED, true>), g, t, 0, s, b);
      }
    } else if (out_f32) {
      hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_F32, BL_NK, true>), g, t, 0, s, b);
    } else {
      hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_BF16, BL_NK, true>), g, t, 0, s, b);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  if (b_layout == MOE_B_KN) {
    if (epilogue == MOE_EPI_SWIGLU) return MOE_ERR_UNSUPPORTED;
    if (epilogue == MOE_EPI_SWIGLU_BWD) {
      hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_SWIGLU_BWD, MOE_OUT_BF16, BL_KN>), g, t, 0, s, b);
    } else if (out_f32) {
      hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_F32, BL_KN>), g, t, 0, s, b);
    } else {
      hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_BF16, BL_KN>), g, t, 0, s, b);
    }
  } else if (b_layout == MOE_B_PACKED) {
    if (epilogue == MOE_EPI_SWIGLU && a.Caux) {
      hipLaunchKernelGGL((gg_fwd_kernel<EPI_SWIGLU_AUX, MOE_OUT_BF16, BL_PACKED>), g, t, 0, s, b);
    } else if (epilogue == MOE_EPI_SWIGLU) {
      hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_SWIGLU, MOE_OUT_BF16, BL_PACKED>), g, t, 0, s, b);
    } else if (out_f32) {
      hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_F32, BL_PACKED>), g, t, 0, s, b);
    } else {
      hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_BF16, BL_PACKED>), g, t, 0, s, b);
    }
  } else if (epilogue == MOE_EPI_SWIGLU && a.Caux) {
    hipLaunchKernelGGL((gg_fwd_kernel<EPI_SWIGLU_AUX, MOE_OUT_BF16, BL_NK>), g, t, 0, s, b);
  } else if (epilogue == MOE_EPI_SWIGLU) {
    hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_SWIGLU, MOE_OUT_BF16, BL_NK>), g, t, 0, s, b);
  } else if (out_f32) {
    hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_F32, BL_NK>), g, t, 0, s, b);
  } else {
    hipLaunchKernelGGL((gg_fwd_kernel<MOE_EPI_NONE, MOE_OUT_BF16, BL_NK>), g, t, 0, s, b);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// bf16, ragged-K: the weight gradients
moe_status_t launch_wgrad(const GGArgs& a, int out_f32, hipStream_t s) {
  static std::atomic<uint64_t> launches{0};
  GGArgs b = a;
  b.n_tiles = (a.N + fwd::BN - 1) / fwd::BN;
  b.p_tiles = (a.M + fwd::BM - 1) / fwd::BM;
  const int64_t max_tiles = (int64_t)a.G * b.n_tiles * b.p_tiles;
  if (max_tiles > tq::kMaxTiles) return MOE_ERR_INVALID_ARG;   // the queue counts' range
  const uint64_t n = launches.fetch_add(1u, std::memory_order_relaxed);
  b.sched_slot = tq::launch_slot(n);
  b.sched_epoch = tq::launch_epoch(n);
  b.sched_next = tq::slot_next_epoch(n);
  int64_t grid = moe_host::device_cu_count();
  if (max_tiles < grid) grid = max_tiles;
  if (grid <= 0) grid = 1;
  const dim3 g((unsigned)grid), t(fwd::THREADS);
  if (out_f32) {
    hipLaunchKernelGGL((fwd::gg_wgrad_kernel<MOE_OUT_F32>), g, t, 0, s, b);
  } else {
    hipLaunchKernelGGL((fwd::gg_wgrad_kernel<MOE_OUT_BF16>), g, t, 0, s, b);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
