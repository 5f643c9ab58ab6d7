// Shared pieces of the forward grouped-GEMM pipelines (bf16 and MXFP8):
// tile geometry, the direct-to-LDS row loader and the device-side lookup of
// a tile's expert group.
#pragma once
#include "gg_common.h"

// The direct-to-LDS loads below are inline asm that sets M0 (the LDS
// destination) right before each load and lists M0 as clobbered.  Code the
// compiler generates for these kernels does not use M0 (checked in the
// generated assembly: every M0 write is one of these pairs), so its warning
// that a reserved register in a clobber list is not preserved is moot.
#pragma clang diagnostic ignored "-Winline-asm"

namespace moe {
namespace fwd {

constexpr int BM = 256, BN = 256;   // tile rows (m) and columns (n)
constexpr int ROWB = 64;            // LDS bytes per row and stage (32 bf16)
constexpr int WN = 2, WTN = BN / WN;          // two wavefront columns of 128 n each
constexpr int XOFF = BN * ROWB;               // X (activation) rows follow the W rows in a stage
constexpr int STAGE = (BM + BN) * ROWB;       // 32 KB

// 16-byte slot swizzles of a 64-byte LDS row: slot = chunk ^ swz_row<SW>(row),
// chosen by measuring SQ_LDS_BANK_CONFLICT for each fragment read pattern:
//  SW = 0, bf16 reads (lane l: row l % 16, chunk l / 16): (row >> 1) & 3 is
//    free of conflicts on gfx950, (row >> 2) & 3 or no swizzle are not;
//  SW = 1, MXFP8 reads (lane l: row l % 32, chunk l / 32 or 2 + l / 32):
//    (row >> 2) & 3 is free of conflicts, (row >> 1) & 3 is 2-way.
template <int SW>
__device__ __forceinline__ int swz_row(int row) {
  if constexpr (SW == 0) return (row >> 1) & 3;
  return (row >> 2) & 3;
}
__device__ __forceinline__ int swz64(int row) { return swz_row<0>(row); }

// Direct-to-LDS rows: one wavefront instruction fills 16 rows (1 KB).  Lane l
// writes slot l & 3 of row 16*blk + l/4, which holds chunk
// (l & 3) ^ swz_row<SW>(row) of that row.
template <int R, int NW, int SW = 0>
struct Rows {
  static constexpr int N = R / 16 / NW;
  uint32_t off[N];
  template <typename RowFn>
  __device__ __forceinline__ void init(int64_t ld_bytes, RowFn grow) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int row = (i * NW + wave) * 16 + (lane >> 2);
      const int chunk = (lane & 3) ^ swz_row<SW>(row);
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
          : "s"(l0 + i * NW * 1024), "v"(off[i]), "s"(base)
          : "memory", "m0");
    }
  }
};

// K-outer operands: element (k, n) at src[k * ld + n] (bf16), i.e. the
// contraction runs down the rows (the data-gradient weight [K, N] and both
// weight-gradient operands).  A stage holds 32 k-rows x 256 columns as
// 512-byte LDS rows; 16-byte slot s of row k holds the 8 columns of chunk
// s ^ kswz(k).  The swizzle gives the 8 rows that one half of a transpose
// read touches (rows 8g + r and 8(g+1) + r, r < 4) distinct 32-byte bank
// groups.  One direct load fills two rows (lane l: row l / 32, slot l % 32).
constexpr int KROWB = 512;
__device__ __forceinline__ int kswz(int k) { return ((k & 3) | (((k >> 3) & 1) << 2)) << 1; }

template <int NW>
struct KRows {
  static constexpr int N = 32 / 2 / NW;
  uint32_t off[N];
  // stage columns [n0, n0 + 256); chunks past the last column are clamped to
  // it (their products land in output columns that are never stored)
  __device__ __forceinline__ void init(int64_t ld_bytes, int n0, int ncols) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int k = 2 * (i * NW + wave) + (lane >> 5);
      const int c = (lane & 31) ^ kswz(k);
      const int col = min(n0 + 8 * c, ncols - 8);
      off[i] = (uint32_t)(k * ld_bytes + col * 2);
    }
  }
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
          : "s"(l0 + i * NW * 1024), "v"(off[i]), "s"(base)
          : "memory", "m0");
    }
  }
  // A stage with only kv < 32 valid rows: rows k >= kv re-read row kv - 1
  // (ld_bytes = the row pitch given to init), so no load leaves the operand.
  __device__ __forceinline__ void issue_partial(uint8_t* lds, const uint8_t* base, int kv, int64_t ld_bytes) const {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    const uint32_t l0 = (uint32_t)(uintptr_t)(lds_ptr_t)lds + wave * 1024;
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int k = 2 * (i * NW + wave) + (lane >> 5);
      const uint32_t o = off[i] - (uint32_t)((k - min(k, kv - 1)) * ld_bytes);
      asm volatile(
          "s_mov_b32 m0, %0\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dwordx4 %1, %2"
          :
          : "s"(l0 + i * NW * 1024), "v"(o), "s"(base)
          : "memory", "m0");
    }
  }
};

// MFMA fragment (16 columns x 32 k) of a K-outer stage at tile column nb
// (16 | nb): lane (g = l / 16, j = l % 16) receives k = 8g .. 8g + 7 of
// column nb + j.  ds_read_b64_tr_b16 hands lane j of each 16-lane block
// element (j % 4) of the 4-element rows addressed by lanes j / 4 + 4q,
// q = 0..3 (measured on gfx950), so lane j addresses row 8g + j / 4 at
// column nb + 4 (j % 4), and a second read covers rows + 4 (same swizzle).
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef short s16x8_t __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4_t* lds_s16x4_ptr;

__device__ __forceinline__ uint32_t kfrag_off(int nb) {
  const int lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15;
  const int k = 8 * g + (j >> 2);
  const int n = nb + 4 * (j & 3);
  return (uint32_t)(k * KROWB + (((n >> 3) ^ kswz(k)) << 4) + ((n >> 2) & 1) * 8);
}

__device__ __forceinline__ bf16x8_t kfrag_read(const uint8_t* buf, uint32_t off) {
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(buf + off));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(buf + off + 4 * KROWB));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Tile order of the ragged-M kernels, from the device group sizes (clamped
// to >= 0, and the rows to m_cap, as the other kernels do).  Tiles go group
// by group; a group's m m-tiles are cut into b = round(m / 5.66) blocks of
// near-equal size (at least one), and inside a block the m-tile varies
// fastest over all n-tiles.  The 32 consecutive tiles that run together on
// one XCD then share few operand panels in its L2 (per m-tile, a block of gm
// m-tiles costs about gm/32 activation panel reads per n-tile plus 1/gm
// weight panel reads: least at gm = sqrt(32)), and no block mixes the weights
// of two experts.
constexpr int kBlockTarget = 566;   // 100 x the m-tiles aimed at per block (sqrt(32))

struct TileGroup {
  int g;
  int nt;         // n-tile
  int64_t m0;     // first row of the tile
  int rows;       // valid rows in the tile (1..BM)
};

__device__ __forceinline__ int64_t wave_incl_scan(int64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int64_t u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

__device__ __forceinline__ int64_t wave_u64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// total number of m-tiles over all groups
__device__ __forceinline__ int64_t count_mtiles(const GGArgs& a) {
  const int lane = threadIdx.x & 63;
  int64_t rbase = 0, nt = 0;
  for (int c = 0; c < a.G; c += 64) {
    const int gi = c + lane;
    const int64_t s = gi < a.G ? (int64_t)max(a.sizes[gi], 0) : 0;
    const int64_t rincl = wave_incl_scan(s);
    const int64_t n = min(rbase + rincl, a.m_cap) - min(rbase + rincl - s, a.m_cap);
    nt += (n + BM - 1) / BM;
    rbase += __shfl(rincl, 63, 64);
  }
  return wave_u64(wave_sum(nt));
}

// tile number `tile` (0 <= tile < m-tiles * n_tiles) of the order above
__device__ __forceinline__ TileGroup locate(const GGArgs& a, int64_t tile) {
  const int lane = threadIdx.x & 63;
  int64_t rbase = 0, tbase = 0;
  TileGroup r{a.G - 1, 0, 0, 1};
  for (int c = 0; c < a.G; c += 64) {
    const int gi = c + lane;
    const int64_t s = gi < a.G ? (int64_t)max(a.sizes[gi], 0) : 0;
    const int64_t rincl = wave_incl_scan(s);
    const int64_t r0 = min(rbase + rincl - s, a.m_cap);
    const int64_t n = min(rbase + rincl, a.m_cap) - r0;
    const int64_t cnt = (n + BM - 1) / BM * a.n_tiles;
    const int64_t tincl = wave_incl_scan(cnt);
    const uint64_t hit = __ballot(gi < a.G && cnt > 0 && tbase + tincl > tile);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      const int64_t u = tile - (tbase + __shfl(tincl - cnt, l, 64));   // tile within the group
      const int64_t g0 = __shfl(r0, l, 64), gn = __shfl(n, l, 64);
      const int m = (int)((gn + BM - 1) / BM);
      const int b = max(1, (100 * m + kBlockTarget / 2) / kBlockTarget);   // round(m / 5.66)
      const int q = m / b, rr = m % b;                // rr blocks of q + 1 m-tiles, then q-tile blocks
      const int64_t big = (int64_t)rr * (q + 1) * a.n_tiles;
      int gm, mstart;
      int64_t v;
      if (u < big) {
        const int k = (int)(u / ((int64_t)(q + 1) * a.n_tiles));
        gm = q + 1;
        mstart = k * (q + 1);
        v = u - (int64_t)k * (q + 1) * a.n_tiles;
      } else {
        const int k = (int)((u - big) / ((int64_t)q * a.n_tiles));
        gm = q;
        mstart = rr * (q + 1) + k * q;
        v = u - big - (int64_t)k * q * a.n_tiles;
      }
      const int mloc = mstart + (int)(v % gm);
      r.g = c + l;
      r.nt = (int)(v / gm);
      r.m0 = g0 + (int64_t)mloc * BM;
      r.rows = (int)min<int64_t>(BM, gn - (int64_t)mloc * BM);
      break;
    }
    rbase += __shfl(rincl, 63, 64);
    tbase += __shfl(tincl, 63, 64);
  }
  // the results are wavefront-uniform: keep them in scalar registers
  r.g = __builtin_amdgcn_readfirstlane(r.g);
  r.nt = __builtin_amdgcn_readfirstlane(r.nt);
  r.m0 = wave_u64(r.m0);
  r.rows = __builtin_amdgcn_readfirstlane(r.rows);
  return r;
}

// ------------------------------------------------------------------ split tail
// The ragged-M kernels (bf16 and MXFP8) deal tiles to their workers in turn,
// so a last round of t tiles keeps only t of the grid's workers busy for a
// whole tile.  In a kernel's SPLIT instantiation (which the host picks for
// calls of at most three rounds of long-K tiles, where a short last round is
// likely and costly), when t is at most half the grid each of those tiles is
// instead
// cut along K into S = min(4, grid / t, stages / 16) equal stage ranges
// ("units"), the units of one tile on consecutive workers.  Every unit
// writes its fp32 partial sums to its own slot of the caller's workspace
// (each thread its accumulators, in register order) and counts itself in at
// the tile's counter; the unit that brings the count to S reads the S
// partials back and adds them in split order (so the result does not depend
// on which unit finishes last), then runs the tile's epilogue.  The
// partition depends only on the group sizes, the grid and K: results are
// bitwise reproducible.  Counters: one slot of kSplitWords words per call
// (64 slots handed out in turn; each kernel file holds its own array),
// epoch-tagged as the tile queues (tile_queue.h), reset for the slot's next
// call by the call's last workgroup (split_finish).
constexpr int kMaxSplit = 4, kMinSplitStages = 16;
constexpr int kSplitWords = 512 + 1;   // tail tiles (at most half a grid of <= 1024) + done count

struct SplitSlots {
  uint32_t w[tq::kSlots][kSplitWords];
};
constexpr SplitSlots initial_split_slots() {
  SplitSlots t{};
  for (int s = 0; s < tq::kSlots; ++s)
    for (int i = 0; i < kSplitWords; ++i) t.w[s][i] = tq::word(tq::launch_epoch((uint64_t)s), 0u);
  return t;
}
struct SplitTail {
  int64_t full;    // tiles of the whole rounds (units [0, full) are whole tiles)
  int64_t units;   // full + tail tiles x S
  int S;           // splits of each tail tile (1: none)
};

__device__ __forceinline__ SplitTail split_tail(int64_t total, int grid, int nk) {
  SplitTail r{total, total, 1};
  const int64_t tail = total % grid;
  if (tail == 0 || 2 * tail > grid || tail > kSplitWords - 1) return r;
  const int S = min(kMaxSplit, min(grid / (int)tail, nk / kMinSplitStages));
  if (S < 2) return r;
  r.full = total - tail;
  r.units = r.full + tail * S;
  r.S = S;
  return r;
}

// Once per workgroup of a call that split its tail, after its last unit:
// the last workgroup to arrive presets the slot's words (w) for the slot's
// next call.  box: one int of LDS no wavefront uses any more.
__device__ __forceinline__ void split_finish(const GGArgs& a, uint32_t* w, int32_t* box) {
  __syncthreads();
  if (threadIdx.x == 0) {
    DeviceWord done{w + (kSplitWords - 1)};
    box[0] = tq::finish(done, a.sched_epoch, gridDim.x);
  }
  __syncthreads();
  if (__builtin_amdgcn_readfirstlane(box[0]))
    for (int i = threadIdx.x; i < kSplitWords; i += blockDim.x) atomicExch(w + i, tq::word(a.sched_next, 0u));
}

// The host's choice of a SPLIT instantiation: given the workspace, for calls
// whose tiles fill at most three rounds even with every group's last tile
// partial, of at least 64 stages each.
inline bool use_split_tail(bool have_ws, int64_t max_tiles, int64_t grid, int stages) {
  return have_ws && max_tiles <= 3 * grid && stages >= 64;
}

}  // namespace fwd
}  // namespace moe
