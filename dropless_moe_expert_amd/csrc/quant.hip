// Group-aware MXFP8 quantisation: bf16 -> E4M3 codes + one E8M0 scale per
// block of 32.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine": group-aware MXFP8 quantisation is one of the building blocks
// (section "What specialized optimizations are required for dropless MoE?")
// and feeds MXFP8 block scaling of the expert matmuls (section "Optimization
// 1").  "AI Systems Performance Engineering" ch. 1, §1.1 low-precision
// scaling figure: each group of (usually) 32 values gets its own scale.
// Scale rule (OCP MX v1.0): e = floor(log2 amax) - 8 (8 = largest E4M3
// exponent) clamped to [-127, 127], byte = e + 127; codes are the E4M3FN
// round-to-nearest-even of v * 2^-e clamped to +-448.  A block holding a NaN
// or an infinity gets the E8M0 NaN scale and NaN codes (common.h).
//
// v * 2^-e is exact in fp32 (bf16 input times a power of two that keeps the
// result below 512); v_cvt_pk_fp8_f32 rounds to nearest even and keeps the
// sign of zero, so clamping first reproduces the rule exactly.
#include "common.h"

namespace moe {

// axis 0: 4 lanes per block of 32 (8 values each); rows < rows_valid
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(const uint16_t* __restrict__ x, int64_t rows, int cols,
                                                            const int32_t* __restrict__ group_sizes, int G,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ scale) {
  __shared__ int64_t s_rows;
  if (threadIdx.x < kWave) {
    const int64_t tot = group_sizes ? rows_in_use(group_sizes, G, rows) : rows;
    if (threadIdx.x == 0) s_rows = tot;
  }
  __syncthreads();
  const int64_t nrows = s_rows;
  const int nvec = cols / 8;  // 8-element pieces per row
  const int64_t total = nrows * nvec;
  // the grid-stride step is a multiple of 4, so the 4 lanes of one block
  // always move together and the shuffles stay within a block
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx - (threadIdx.x & 3) < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const bool live = idx < total;
    float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (live) unpack8(reinterpret_cast<const uint4*>(x)[idx], f);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = mx_absmax(amax, f[j]);
    amax = mx_absmax(amax, __shfl_xor(amax, 1, 64));
    amax = mx_absmax(amax, __shfl_xor(amax, 2, 64));
    const int e = mx_exponent(amax);
    if (live) {
      uint2 out;
      out.x = mx_codes4(f[0], f[1], f[2], f[3], e);
      out.y = mx_codes4(f[4], f[5], f[6], f[7], e);
      reinterpret_cast<uint2*>(q)[idx] = out;
      if ((idx & 3) == 0) scale[idx >> 2] = (uint8_t)(e + 127);
    }
  }
}

// axis 1: one thread per (block row p, 8-column piece); blocks restart at groups
__global__ __launch_bounds__(256) void mx_quant_cols_kernel(const uint16_t* __restrict__ x, int64_t rows, int cols,
                                                            const int32_t* __restrict__ group_sizes, int G,
                                                            uint8_t* __restrict__ q, uint8_t* __restrict__ scale,
                                                            uint32_t* flag) {
  extern __shared__ int64_t sh[];  // [0,G]: group row offsets; [G+1, 2G+2): block prefix
  int64_t* roff = sh;
  int64_t* boff = sh + G + 1;
  if (threadIdx.x == 0) {
    int64_t o = 0, p = 0;
    bool neg = false, over = false;
    for (int g = 0; g < G; ++g) {
      int64_t s = group_sizes[g];
      if (s < 0) { neg = true; s = 0; }
      if (o + s > rows) { over = true; s = rows - o; }
      roff[g] = o;
      boff[g] = p;
      o += s;
      p += (s + 31) / 32;
    }
    roff[G] = o;
    boff[G] = p;
    if (neg) raise_flag(flag, MOE_FLAG_NEGATIVE_SIZE);
    if (over) raise_flag(flag, MOE_FLAG_ROWS_OVER_CAP);
  }
  __syncthreads();
  const int64_t nblk = boff[G];
  const int npc = cols / 8;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < nblk * npc;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t p = idx / npc;
    const int c8 = (int)(idx - p * npc) * 8;
    // group of block p: last g with boff[g] <= p
    int lo = 0, hi = G - 1;
    while (lo < hi) {
      int mid = (lo + hi + 1) >> 1;
      if (boff[mid] <= p) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const int64_t r0 = roff[g] + (p - boff[g]) * 32;
    const int n = (int)min((int64_t)32, roff[g + 1] - r0);
    float amax[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int i = 0; i < n; ++i) {
      float f[8];
      unpack8(*reinterpret_cast<const uint4*>(x + (r0 + i) * cols + c8), f);
#pragma unroll
      for (int j = 0; j < 8; ++j) amax[j] = mx_absmax(amax[j], f[j]);
    }
    int e[8];
    uint2 sc;
    uint8_t* scb = reinterpret_cast<uint8_t*>(&sc);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      e[j] = mx_exponent(amax[j]);
      scb[j] = (uint8_t)(e[j] + 127);
    }
    *reinterpret_cast<uint2*>(scale + p * cols + c8) = sc;
    for (int i = 0; i < n; ++i) {
      float f[8];
      unpack8(*reinterpret_cast<const uint4*>(x + (r0 + i) * cols + c8), f);
      uint2 out;
      out.x = mx_codes4(f[0], f[1], f[2], f[3], e[0], e[1], e[2], e[3]);
      out.y = mx_codes4(f[4], f[5], f[6], f[7], e[4], e[5], e[6], e[7]);
      *reinterpret_cast<uint2*>(q + (r0 + i) * cols + c8) = out;
    }
  }
}

// Transposed axis 1, one workgroup per tile of 64 positions (two blocks) x
// 64 columns: the tile's rows are read as whole 128-byte row pieces into
// LDS, each (column, block) pair is quantised from there by one thread, the
// codes are assembled column-major in LDS and leave as 64-byte column rows of
// qT (four 16-byte pieces per column), the two scales of a column as one
// 2-byte word.  Grouped (group_sizes != NULL): positions in the 64-aligned
// padded layout (kpad = padded group starts); positions past a group's rows
// get zero codes, blocks with no rows scale 0.  Batched (NULL): G batches of
// `rows` rows, one group each.  With q0 != NULL the same tile also yields
// the row-wise (axis 0) codes and scales of its valid rows, by the threads
// the column blocks leave idle: one read of x for both layouts.
constexpr int QT_R = 64, QT_C = 64;
constexpr int QT_LD = QT_C + 2;   // bf16 per LDS row: the pad staggers the row reads over the banks
// bytes per column of the code tile: 128 codes and 16 of padding, so that
// 16-byte accesses by consecutive columns start 4 banks apart (at 128 bytes
// every column would start on the same bank)
constexpr int QT_CT = 2 * QT_R + 16;

// PRODUCER 0: the tile is read from x [rows, cols].  PRODUCER 1: the tile
// is the SwiGLU backward dgu [rows, cols = 2f] (bf16-rounded, as
// moe_swiglu_backward stores it), made from x = gu [rows, 2f] and dh
// [rows, f]: dgu never exists in bf16.
// the value of the neighbouring lane (t ^ 1), by DPP (quad_perm 1, 0, 3, 2)
__device__ __forceinline__ int dpp_swap1(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false); }

// a value equal in every lane, moved to scalar registers
__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// PRODUCER 3 (gather): row r of the tile source is row perm_src[r] / K of
// x [T, cols] (the permute's x_perm, never stored), times the routing weight
// w[perm_src[r]] and rounded to bf16 as moe_combine_backward rounds dy_perm
// when w != NULL.  The pair / K division is exact as a 64-bit multiply by
// magic = floor(2^40 / K) + 1 and a shift by 40 for pairs below 2^31 and
// K <= 32: the product exceeds pair / K by less than 2^-9 < 1 / K.
struct GatherArgs {
  const int32_t* src;   // perm_src [rows]
  const float* w;       // routing weights [rows] or NULL
  const float* wsrc;    // w, or (unweighted) src read as floats: the weight load is issued either way
  uint64_t magic;       // floor(2^40 / K) + 1
  uint32_t last;        // rows - 1: a pair index is clamped to it, so no value read from src leads outside x or w
};

// element h (0 or 1, known only at run time) of a two-element array
template <typename V>
__device__ __forceinline__ V sel(int h, const V (&a)[2]) { return h ? a[1] : a[0]; }

template <int PRODUCER, bool ROWS>
__global__ __launch_bounds__(256) void mx_quant_t_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ dh, int64_t rows, int cols,
                                                         const int32_t* __restrict__ group_sizes, int G,
                                                         int64_t k_cap, uint8_t* __restrict__ qT,
                                                         uint8_t* __restrict__ scaleT, uint8_t* __restrict__ q0,
                                                         uint8_t* __restrict__ s0, uint32_t* flag, GatherArgs ga) {
  extern __shared__ int64_t sh[];  // grouped: [0,G]: row offsets; [G+1, 2G+2): padded starts
  __shared__ __align__(16) uint16_t xt[2 * QT_R * QT_LD];  // two position units, bf16, row-major
  __shared__ __align__(16) uint8_t ct[QT_C * QT_CT];    // their codes, column-major (128 per column)
  __shared__ uint8_t st[QT_C * 4];                      // their scales, four per column
  int64_t* roff = sh;
  int64_t* kpad = sh + G + 1;
  const bool grouped = group_sizes != nullptr;
  if (grouped) {
    // row offsets and padded starts: each thread sums its run of groups,
    // a block scan of the sums, then each thread writes its run's prefixes
    // (the scans live in the tile buffer, unused until the first tile: the
    //  kernel's LDS then stays small enough for five workgroups per CU)
    int64_t* scan_r = reinterpret_cast<int64_t*>(xt);
    int64_t* scan_k = scan_r + 256;
    static_assert(sizeof(xt) >= 2 * 256 * sizeof(int64_t), "the scans fit the tile buffer");
    const int per = (G + 255) / 256, t0 = threadIdx.x * per;
    int64_t lr = 0;
    bool neg = false;
    for (int g = t0; g < min(G, t0 + per); ++g) {
      const int32_t v = group_sizes[g];
      neg |= v < 0;
      lr += max(v, 0);
    }
    scan_r[threadIdx.x] = lr;
    __syncthreads();
    for (int o = 1; o < 256; o <<= 1) {   // inclusive scan of the run sums
      const int64_t v = threadIdx.x >= o ? scan_r[threadIdx.x - o] : 0;
      __syncthreads();
      scan_r[threadIdx.x] += v;
      __syncthreads();
    }
    // clamp the rows to `rows` as the groups are walked in order
    int64_t o = scan_r[threadIdx.x] - lr, lk = 0;
    for (int g = t0; g < min(G, t0 + per); ++g) {
      const int64_t sz = min((int64_t)max(group_sizes[g], 0), max((int64_t)0, rows - o));
      lk += (sz + 63) / 64 * 64;
      o += max(group_sizes[g], 0);
    }
    scan_k[threadIdx.x] = lk;
    __syncthreads();
    for (int o2 = 1; o2 < 256; o2 <<= 1) {
      const int64_t v = threadIdx.x >= o2 ? scan_k[threadIdx.x - o2] : 0;
      __syncthreads();
      scan_k[threadIdx.x] += v;
      __syncthreads();
    }
    int64_t ro = scan_r[threadIdx.x] - lr, ko = scan_k[threadIdx.x] - lk;
    for (int g = t0; g < min(G, t0 + per); ++g) {
      const int64_t sz = min((int64_t)max(group_sizes[g], 0), max((int64_t)0, rows - ro));
      roff[g] = min(ro, rows);
      kpad[g] = ko;
      ro += max(group_sizes[g], 0);
      ko += (sz + 63) / 64 * 64;
    }
    if (threadIdx.x == 255) {
      roff[G] = min(scan_r[255], rows);
      kpad[G] = scan_k[255];
    }
    if (blockIdx.x == 0 && __any(neg) && (threadIdx.x & 63) == 0) raise_flag(flag, MOE_FLAG_NEGATIVE_SIZE);
    if (blockIdx.x == 0 && threadIdx.x == 255 && scan_r[255] > rows) raise_flag(flag, MOE_FLAG_ROWS_OVER_CAP);
    __syncthreads();
  }
  const int64_t tpb = rows / QT_R;   // batched: position units per batch
  const int64_t ntk = grouped ? kpad[G] / QT_R : (int64_t)G * tpb;
  const int64_t ntp = (ntk + 1) / 2;   // pairs of units: a column's 128 codes leave as one line
  // PRODUCER 2 (SwiGLU backward, f % 32 == 0): a tile's 64 columns are the
  // gate columns c0 .. c0 + 31 and the up columns f + c0 .. f + c0 + 31, so
  // one read of g, u and dh gives both halves; otherwise 64 consecutive columns
  const int fh = cols / 2;
  const int ntc = PRODUCER == 2 ? (fh + 31) / 32 : (cols + QT_C - 1) / QT_C;
  auto gcol = [&](int c0, int c) { return PRODUCER == 2 ? (c < 32 ? c0 + c : fh + c0 + (c - 32)) : c0 + c; };
  auto colvalid = [&](int c0, int c) { return PRODUCER == 2 ? c0 + (c & 31) < fh : c0 + c < cols; };
  const int t = threadIdx.x;
  // A tile's place: for each unit (64 positions) of the pair its first row,
  // its valid rows and its first code and scale in column 0's qT / scaleT row
  // (read through sel with constant indices: no array lives in scratch)
  struct Tile {
    int64_t r0[2];
    int n[2];
    int val[2];   // the unit exists (int, not bool: a bool pair was kept in scratch)
    uint8_t* qb[2];
    uint8_t* sb[2];
    int c0;
  };
  auto describe = [&](int64_t tile, Tile& D) {
#ifdef QT_COL_MAJOR
    const int64_t ct = tile / ntp, tp = tile - ct * ntp;
    D.c0 = (int)ct * (PRODUCER == 2 ? 32 : QT_C);
#else
    const int64_t tp = tile / ntc;
    D.c0 = (int)(tile - tp * ntc) * (PRODUCER == 2 ? 32 : QT_C);
#endif
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t tk = 2 * tp + h;
      D.val[h] = tk < ntk;
      D.r0[h] = 0;
      D.n[h] = 0;
      D.qb[h] = qT;
      D.sb[h] = scaleT;
      if (!D.val[h]) continue;
      if (grouped) {
        int lo = 0, hi = G - 1;   // last g with kpad[g] <= 64 tk
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (kpad[mid] <= QT_R * tk) lo = mid; else hi = mid - 1;
        }
        // the same in every lane (read from LDS): kept in scalar registers
        D.r0[h] = uniform64(roff[lo] + (QT_R * tk - kpad[lo]));
        D.n[h] = __builtin_amdgcn_readfirstlane((int)max((int64_t)0, min((int64_t)QT_R, roff[lo + 1] - D.r0[h])));
        D.qb[h] = qT + QT_R * tk;
        D.sb[h] = scaleT + 2 * tk;
      } else {
        const int64_t g = tk / tpb, b = tk - g * tpb;
        D.r0[h] = g * rows + QT_R * b;
        D.n[h] = QT_R;
        D.qb[h] = qT + g * cols * rows + QT_R * b;
        D.sb[h] = scaleT + g * cols * (rows / 32) + 2 * b;
      }
    }
  };
  const int64_t ldq = grouped ? k_cap : rows;
  // The pair's rows come in as 16-byte pieces of 8 columns held in registers
  // until the LDS is free: PRODUCER 0 four pieces of x per thread (128 rows x
  // 8 pieces); PRODUCER 1 the g, u and dh pieces behind four dgu pieces;
  // PRODUCER 2 those behind two (gate, up) piece pairs (128 rows x 4 pairs).
  // The next tile's loads are issued as soon as this tile's rows are in LDS,
  // so they are in flight while this tile is quantised and written out.
  constexpr int NP = PRODUCER == 2 ? 2 : 4;   // pieces (pairs) per thread
  constexpr int NL = PRODUCER == 1 || PRODUCER == 2 ? 3 : 1;   // loads per piece
  constexpr bool GATHER = PRODUCER == 3;
  uint4 raw[NP][NL];
  // PRODUCER 3: the pairs of this thread's four rows of the tile to be
  // loaded next (read a tile ahead, so that the gather waits for no index),
  // and the routing weights of the rows being loaded
  int32_t pidx[4];
  float wv[4];
  // the index loads: every lane loads (a row past its unit's rows, or of an
  // absent unit, reads the tile's first row's entry), so the number of
  // loads issued after a tile's data loads never varies
  auto load_idx = [&](const Tile& D) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int rr = (t + 256 * k) >> 3, h = rr >> 6, r = rr & 63;
      const int64_t row = r < sel(h, D.n) ? sel(h, D.r0) + r : D.r0[0];
      pidx[k] = ga.src[row];
    }
  };
  auto load = [&](const Tile& D) {
#pragma unroll
    for (int k = 0; k < NP; ++k) {
#pragma unroll
      for (int l = 0; l < NL; ++l) raw[k][l] = make_uint4(0, 0, 0, 0);
      const int u = t + 256 * k;
      if constexpr (PRODUCER == 2) {
        const int rr = u >> 2, j = D.c0 + 8 * (u & 3), h = rr >> 6, r = rr & 63;
        if (r < sel(h, D.n) && j < fh) {
          const int64_t row = sel(h, D.r0) + r;
          raw[k][0] = *reinterpret_cast<const uint4*>(x + row * cols + j);
          raw[k][1] = *reinterpret_cast<const uint4*>(x + row * cols + fh + j);
          raw[k][2] = *reinterpret_cast<const uint4*>(dh + row * fh + j);
        }
      } else if constexpr (GATHER) {
        const int rr = u >> 3, c = (u & 7) * 8, h = rr >> 6, r = rr & 63;
        const uint32_t pair = min((uint32_t)pidx[k], ga.last);
        if (r < sel(h, D.n) && D.c0 + c < cols) {
          const int64_t tok = (int64_t)(((uint64_t)pair * ga.magic) >> 40);
          raw[k][0] = *reinterpret_cast<const uint4*>(x + tok * cols + D.c0 + c);
        }
        // in every lane and either way (a padding row's weight multiplies
        // zeros), so the loads after each data load are always the same
        wv[k] = ga.wsrc[pair];
      } else {
        const int rr = u >> 3, c = (u & 7) * 8, h = rr >> 6, r = rr & 63;
        if (r < sel(h, D.n) && D.c0 + c < cols) {
          const int64_t row = sel(h, D.r0) + r;
          if constexpr (PRODUCER == 0) {
            raw[k][0] = *reinterpret_cast<const uint4*>(x + row * cols + D.c0 + c);
          } else {
            const int j = (D.c0 + c) % fh;   // f % 8 == 0: a piece is all gate or all up
            raw[k][0] = *reinterpret_cast<const uint4*>(x + row * cols + j);
            raw[k][1] = *reinterpret_cast<const uint4*>(x + row * cols + fh + j);
            raw[k][2] = *reinterpret_cast<const uint4*>(dh + row * fh + j);
          }
        }
      }
    }
  };
  // the registers to LDS; the SwiGLU producers form dgu here (zero pieces,
  // those of padding rows and absent columns, give zero)
  auto stage = [&](const Tile& D) {
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      const int u = t + 256 * k;
      if constexpr (PRODUCER == 2) {
        const int rr = u >> 2, jp = u & 3;
        float g[8], uu[8], dd[8], dg[8], du[8];
        unpack8(raw[k][0], g);
        unpack8(raw[k][1], uu);
        unpack8(raw[k][2], dd);
#pragma unroll
        for (int e = 0; e < 8; ++e) swiglu_grad(g[e], uu[e], dd[e], dg[e], du[e]);
        const uint4 vg = pack8(dg), vu = pack8(du);
        uint32_t* d = reinterpret_cast<uint32_t*>(xt + rr * QT_LD + 8 * jp);
        d[0] = vg.x; d[1] = vg.y; d[2] = vg.z; d[3] = vg.w;
        d = reinterpret_cast<uint32_t*>(xt + rr * QT_LD + 32 + 8 * jp);
        d[0] = vu.x; d[1] = vu.y; d[2] = vu.z; d[3] = vu.w;
      } else {
        const int rr = u >> 3, c = (u & 7) * 8;
        uint4 v = raw[k][0];
        if constexpr (GATHER) {
          if (ga.w) {   // bf16(w * dy) as moe_combine_backward forms dy_perm
            float g[8];
            unpack8(raw[k][0], g);
            v = mul8_bf16(wv[k], g);
          }
        }
        if constexpr (PRODUCER == 1) {
          float g[8], uu[8], dd[8], dg[8], du[8];
          unpack8(raw[k][0], g);
          unpack8(raw[k][1], uu);
          unpack8(raw[k][2], dd);
#pragma unroll
          for (int e = 0; e < 8; ++e) swiglu_grad(g[e], uu[e], dd[e], dg[e], du[e]);
          v = pack8(D.c0 + c < fh ? dg : du);
        }
        uint32_t* d = reinterpret_cast<uint32_t*>(xt + rr * QT_LD + c);   // 4-byte aligned (QT_LD even)
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
      }
    }
  };
  const int64_t ntiles = ntp * ntc;
  // Round k of the grid takes tiles k * grid .. (k + 1) * grid - 1.  The
  // hardware deals workgroups to the 8 XCDs in turn (block b to XCD b % 8),
  // so when the grid is a multiple of 8 each XCD gets a run of consecutive
  // tiles: the tiles that share output lines then share that XCD's L2.
  const int64_t per_xcd = gridDim.x % 8 == 0 ? gridDim.x / 8 : 0;
  const int64_t slot = per_xcd ? (blockIdx.x % 8) * per_xcd + blockIdx.x / 8 : blockIdx.x;
  auto tile_of = [&](int64_t k) { return k * gridDim.x + slot; };
  if (tile_of(0) >= ntiles) return;
  // 1. the first tile's rows into LDS; each later tile's are staged at the
  //    end of the previous pass, after that pass's stores (the loop is so
  //    rotated that the wait for those rows counts the stores in between)
  //    The gather first needs the pairs of tile 0's rows, then of tile 1's.
  Tile cur;
  describe(tile_of(0), cur);
  if constexpr (GATHER) load_idx(cur);
  load(cur);
  if constexpr (GATHER) {
    Tile t1 = cur;
    if (tile_of(1) < ntiles) describe(tile_of(1), t1);
    load_idx(t1);
  }
  stage(cur);
  // A pass's gather waits for the pairs loaded in the pass before, with
  // that pass's stores issued after them (not waited for).  Tile 1's pairs
  // are waited for here instead, so that entering the first pass adds no
  // path on which the gather's wait would have to count fewer operations.
  if constexpr (GATHER) asm volatile("" ::"v"(pidx[0]), "v"(pidx[1]), "v"(pidx[2]), "v"(pidx[3]));
  for (int64_t k = 0;; ++k) {
    const int c0 = cur.c0;
    const bool more = tile_of(k + 1) < ntiles;
    // the gather's pairs for the next tile, waited for on every path (also
    // the last pass's, which loads nothing), so that no later write of
    // their registers waits again
    if constexpr (GATHER) asm volatile("" ::"v"(pidx[0]), "v"(pidx[1]), "v"(pidx[2]), "v"(pidx[3]));
    Tile nxt = cur;
    if (more) {   // the next tile's loads are in flight while this one is quantised and stored
      describe(tile_of(k + 1), nxt);
      load(nxt);
    }
    if constexpr (GATHER) {   // and the pairs of the tile after it (or again those of a tile at hand)
      Tile n2 = nxt;
      if (tile_of(k + 2) < ntiles) describe(tile_of(k + 2), n2);
      load_idx(n2);
    }
    __syncthreads();
    // 2a. one thread per (column, 32-position block): amax, scale, 32 codes
    //     into the column, on the column's values paired down the rows
    {
      const int c = t & (QT_C - 1), b = t >> 6;   // b = 0..3 over the pair's 128 positions
      uint32_t pr[16];   // rows 32 b + 2 i (low half) and 32 b + 2 i + 1 (high half)
      uint32_t m = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pr[i] = (uint32_t)xt[(32 * b + 2 * i) * QT_LD + c] | ((uint32_t)xt[(32 * b + 2 * i + 1) * QT_LD + c] << 16);
        asm volatile("" : "+v"(pr[i]));   // one register per pair, not its two halves kept apart
        m = max_u16x2(m, mag_pair(pr[i]));
      }
      const int e = mx_exponent(amax_of_pair(m));
      st[4 * c + b] = (uint8_t)(e + 127);
      uint32_t w[8];
      if (e != kMxNaN) {
        const float sc = mx_scale_operand(e);
        const uint32_t lim2 = mx_clamp_pair(e);
#pragma unroll
        for (int q = 0; q < 8; ++q) w[q] = mx_codes4_pairs(pr[2 * q], pr[2 * q + 1], sc, lim2);
      } else {
        // a NaN block's codes are NaN only at the group's rows: the padding
        // positions past them keep zero codes, as in every other block
        const int nv = min(32, max(0, sel(b >> 1, cur.n) - 32 * (b & 1)));
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          w[q] = mx_nan_codes4_pairs(pr[2 * q], pr[2 * q + 1]);
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (4 * q + k >= nv) w[q] &= ~(0xFFu << (8 * k));
        }
      }
      uint4* d = reinterpret_cast<uint4*>(ct + c * QT_CT + 32 * b);
      d[0] = make_uint4(w[0], w[1], w[2], w[3]);
      d[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
    // 2b. one thread per (row, 32-column block): the axis-0 quantisation of the
    //     valid rows, a row's two blocks in neighbouring lanes.  A thread
    //     without a valid row takes the tile's first row (always valid) and
    //     stores the same bytes to the same place as that row's threads:
    //     every thread issues the same stores, so the wait for the next
    //     tile's loads need not wait for these stores too.  When both blocks
    //     exist and are adjacent (not the SwiGLU split), the two lanes swap
    //     halves so that each store writes 32 contiguous bytes of the row,
    //     and both store the row's two scales as one 2-byte word; otherwise
    //     (cols % 64 != 0) a lane without its block takes block 0.
    if constexpr (ROWS) {
      // the same for the whole tile; cols % 64 == 0 keeps the scale word 2-byte aligned
      const bool pair_ok = PRODUCER != 2 && cols % 64 == 0 && colvalid(c0, 32);
      int rr = t >> 1, b = t & 1;
      if (!((rr & 63) < sel(rr >> 6, cur.n))) rr = 0;
      if (!pair_ok && !colvalid(c0, 32 * b)) rr = b = 0;
      const int cb = gcol(c0, 32 * b), h = rr >> 6, r = rr & 63;
      {
        const uint32_t* xr = reinterpret_cast<const uint32_t*>(xt + rr * QT_LD + 32 * b);   // QT_LD even
        uint32_t pr[16];   // columns 2 i and 2 i + 1
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          pr[i] = xr[i];
          m = max_u16x2(m, mag_pair(pr[i]));
        }
        const int e = mx_exponent(amax_of_pair(m));
        uint32_t w[8];
        if (e != kMxNaN) {
          const float sc = mx_scale_operand(e);
          const uint32_t lim2 = mx_clamp_pair(e);
#pragma unroll
          for (int q = 0; q < 8; ++q) w[q] = mx_codes4_pairs(pr[2 * q], pr[2 * q + 1], sc, lim2);
        } else {
#pragma unroll
          for (int q = 0; q < 8; ++q) w[q] = mx_nan_codes4_pairs(pr[2 * q], pr[2 * q + 1]);
        }
        const int64_t row = sel(h, cur.r0) + r;
        // the swap: block 0's lane keeps its first 16 codes and receives
        // block 1's first 16; block 1's lane keeps its last 16 and receives
        // block 0's last 16 (lanes t and t ^ 1 by DPP)
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (uint32_t)dpp_swap1((int)(b ? w[i] : w[4 + i]));
        const uint32_t eo = (uint32_t)dpp_swap1(e + 127);
        uint8_t* rowq = q0 + row * cols;
        if (pair_ok) {
          const uint4 lo = b ? make_uint4(o[0], o[1], o[2], o[3]) : make_uint4(w[0], w[1], w[2], w[3]);
          const uint4 hi = b ? make_uint4(w[4], w[5], w[6], w[7]) : make_uint4(o[0], o[1], o[2], o[3]);
          *reinterpret_cast<uint4*>(rowq + c0 + 16 * b) = lo;
          *reinterpret_cast<uint4*>(rowq + c0 + 32 + 16 * b) = hi;
          const uint32_t mine = (uint32_t)(e + 127);
          *reinterpret_cast<uint16_t*>(s0 + row * (cols / 32) + c0 / 32) =
              (uint16_t)(b ? (eo | (mine << 8)) : (mine | (eo << 8)));
        } else {
          uint4* d = reinterpret_cast<uint4*>(rowq + cb);
          d[0] = make_uint4(w[0], w[1], w[2], w[3]);
          d[1] = make_uint4(w[4], w[5], w[6], w[7]);
          s0[row * (cols / 32) + cb / 32] = (uint8_t)(e + 127);
        }
      }
    }
    __syncthreads();
    // 3. column rows out: lanes (column, 16-byte piece of the pair's 128 codes),
    //    so one store instruction writes 8 columns x 128 contiguous bytes when the
    //    two units are adjacent in the column row; the scale pairs
#pragma unroll
    //    (a lane of an absent column or unit repeats the store of column 0,
    //    unit 0, and each of a column's four lanes stores the scale pair:
    //    every lane stores, with the same bytes wherever two lanes meet)
    for (int k = 0; k < 2; ++k) {
      const int idx = t + 256 * k;
      int c = idx >> 3, p8 = idx & 7;
      if (!(sel(p8 >> 2, cur.val) && colvalid(c0, c))) c = 0, p8 &= 3;
      const int h = p8 >> 2;
      const int64_t col = gcol(c0, c);
      *reinterpret_cast<uint4*>(sel(h, cur.qb) + col * ldq + 16 * (p8 & 3)) =
          *reinterpret_cast<const uint4*>(ct + c * QT_CT + 16 * p8);
      *reinterpret_cast<uint16_t*>(sel(h, cur.sb) + col * (ldq / 32)) =
          (uint16_t)(st[4 * c + 2 * h] | ((uint16_t)st[4 * c + 2 * h + 1] << 8));
    }
    if (!more) break;
    __syncthreads();   // this tile's LDS is read out
    stage(nxt);
    cur = nxt;
  }
}

// MXFP4 (E2M1 codes, E8M0 scale per 32 along the columns), four lanes per
// 32-element block.  Scale 2^e with e = floor(log2 amax) - 2 (2 = the largest
// E2M1 exponent), clamped to [-127, 127]; codes round x / 2^e to the nearest
// of 0, 0.5, 1, 1.5, 2, 3, 4, 6 with ties to the even mantissa bit, saturate
// past 6 and keep the sign (also of a zero).  Output: codes [rows, cols / 2],
// element 2i in the low nibble of byte i; scales stage-major [cols / 128]
// [rows][4] (the layout the MXFP4 grouped GEMM loads a stage from).
// E2M1 code of y: below 2 the grid in units of 0.5 is the integers 0..4
// (codes 0..3, and 4 = 2.0), on [2, 4) it is 2, 3, 4 (codes 4..6), on [4, 8)
// it is 4, 6 in steps of 2 (codes 6, 7); rintf's ties-to-even on those
// integers is the format's ties-to-even mantissa bit, and past 6 saturates
__device__ __forceinline__ uint32_t e2m1_code(float y) {
  const float m = fabsf(y);
  const float c = m < 2.f ? rintf(2.f * m) : m < 4.f ? rintf(m) + 2.f : fminf(rintf(0.5f * m) + 4.f, 7.f);
  return (uint32_t)c | ((__float_as_uint(y) >> 28) & 8u);
}

__global__ __launch_bounds__(256) void mx4_quant_rows_kernel(const uint16_t* __restrict__ x, uint32_t rows, uint32_t cols,
                                                             uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  // lane: 8 consecutive elements (one 16-byte load); four lanes hold a
  // 32-block and sixteen lanes one 128-code stage of a row, whose four scale
  // bytes go out as one word.  Indices fit 32 bits (checked by the caller);
  // the grid-stride step is a multiple of 16, so groups move together.
  const uint32_t c8 = cols / 8;
  const uint32_t total = rows * c8;
  const int lane = threadIdx.x & 63;
  for (uint32_t v = blockIdx.x * 256u + threadIdx.x; v - (uint32_t)(lane & 15) < total; v += gridDim.x * 256u) {
    const bool live = v < total;
    const uint32_t r = live ? v / c8 : 0u;
    const uint32_t k8 = live ? v - r * c8 : 0u;
    float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (live) unpack8(reinterpret_cast<const uint4*>(x)[v], f);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = mx_absmax(amax, f[i]);
    amax = mx_absmax(amax, __shfl_xor(amax, 1, 64));
    amax = mx_absmax(amax, __shfl_xor(amax, 2, 64));
    const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFF);
    const int e = ef == 0 ? -127 : ef == 255 ? kMxNaN : max(-127, min(127, ef - 127 - 2));
    const uint32_t byte = (uint32_t)(e + 127);
    const int g0 = lane & ~15;
    const uint32_t word = __shfl(byte, g0, 64) | (__shfl(byte, g0 + 4, 64) << 8) | (__shfl(byte, g0 + 8, 64) << 16) |
                          (__shfl(byte, g0 + 12, 64) << 24);
    if (live) {
      uint32_t codes = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        codes |= (e == kMxNaN ? 7u | ((__float_as_uint(f[i]) >> 28) & 8u) : e2m1_code(scale_pow2(f[i], e))) << (4 * i);
      reinterpret_cast<uint32_t*>(q)[v] = codes;
      if ((k8 & 15u) == 0) reinterpret_cast<uint32_t*>(sc)[(size_t)(k8 >> 4) * rows + r] = word;
    }
  }
}

}  // namespace moe

namespace {

moe_status_t quant_t_launch(const uint16_t* x, const uint16_t* dh, int64_t rows, int32_t cols,
                            const int32_t* group_sizes, int32_t G, int64_t k_cap, uint8_t* qT, uint8_t* scaleT,
                            uint8_t* q0, uint8_t* s0, uint32_t* flag, const moe::GatherArgs* ga, hipStream_t s) {
  const int64_t ntk = group_sizes ? k_cap / 64 : (int64_t)G * (rows / 64);   // an upper bound when grouped
  const int64_t work = (ntk + 1) / 2 * ((cols + 63) / 64);   // pairs of 64-position units
  if (work == 0) return MOE_OK;
  const size_t shmem = group_sizes ? sizeof(int64_t) * (size_t)(2 * G + 2) : 0;
  // one resident wave of workgroups, each looping over its tiles (a second
  // wave would start only as the first drains, and run on a part of the chip)
  auto launch = [&](auto kern) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, shmem) != hipSuccess) {
      (void)hipGetLastError();   // the query's failure is not the launch's
      per_cu = 1;
    }
    per_cu = std::max(per_cu, 1);
    const int64_t blocks = std::min<int64_t>(work, (int64_t)moe_host::device_cu_count() * per_cu);
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), shmem, s, x, dh, rows, cols, group_sizes, G, k_cap,
                       qT, scaleT, q0, s0, flag, ga ? *ga : moe::GatherArgs{nullptr, nullptr, nullptr, 0, 0});
  };
  if (ga) {
    if (q0) launch(moe::mx_quant_t_kernel<3, true>);
    else launch(moe::mx_quant_t_kernel<3, false>);
  } else if (q0) {
    if (dh && (cols / 2) % 32 == 0) launch(moe::mx_quant_t_kernel<2, true>);
    else if (dh) launch(moe::mx_quant_t_kernel<1, true>);
    else launch(moe::mx_quant_t_kernel<0, true>);
  } else {
    if (dh && (cols / 2) % 32 == 0) launch(moe::mx_quant_t_kernel<2, false>);
    else if (dh) launch(moe::mx_quant_t_kernel<1, false>);
    else launch(moe::mx_quant_t_kernel<0, false>);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace

extern "C" moe_status_t mxfp8_quantize_transposed_launch(const uint16_t* x, const uint16_t* dh, int64_t rows,
                                                         int32_t cols, const int32_t* group_sizes, int32_t G,
                                                         int64_t k_cap, uint8_t* qT, uint8_t* scaleT, uint8_t* q0,
                                                         uint8_t* s0, uint32_t* flag, hipStream_t s) {
  return quant_t_launch(x, dh, rows, cols, group_sizes, G, k_cap, qT, scaleT, q0, s0, flag, nullptr, s);
}

extern "C" moe_status_t mxfp8_gather_quantize_launch(const uint16_t* x, const int32_t* perm_src, const float* w,
                                                     int32_t K, int64_t rows, int32_t cols,
                                                     const int32_t* group_sizes, int32_t G, int64_t k_cap,
                                                     uint8_t* qT, uint8_t* scaleT, uint8_t* q0, uint8_t* s0,
                                                     uint32_t* flag, hipStream_t s) {
  const moe::GatherArgs ga{perm_src, w, w ? w : reinterpret_cast<const float*>(perm_src),
                           ((uint64_t)1 << 40) / (uint64_t)K + 1, (uint32_t)(rows - 1)};
  return quant_t_launch(x, nullptr, rows, cols, group_sizes, G, k_cap, qT, scaleT, q0, s0, flag, &ga, s);
}

extern "C" moe_status_t mxfp4_quantize_launch(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* q,
                                              uint8_t* scale, hipStream_t s) {
  const int64_t n = rows * (cols / 8);
  if (n == 0) return MOE_OK;
  if (n > (int64_t)UINT32_MAX - 65536 * 256) return MOE_ERR_UNSUPPORTED;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, (int64_t)moe_host::device_cu_count() * 32);
  hipLaunchKernelGGL(moe::mx4_quant_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, (uint32_t)rows,
                     (uint32_t)cols, q, scale);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status_t mxfp8_group_quantize_launch(const uint16_t* x, int64_t rows, int32_t cols, int32_t axis,
                                                    const int32_t* group_sizes, int32_t G, uint8_t* q, uint8_t* scale,
                                                    uint32_t* flag, hipStream_t s) {
  if (rows == 0) return MOE_OK;
  const int64_t cap = (int64_t)moe_host::device_cu_count() * 16;
  if (axis == 0) {
    const int64_t work = rows * (cols / 8);
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((work + 255) / 256, cap));
    hipLaunchKernelGGL(moe::mx_quant_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, s, x, rows, cols, group_sizes,
                       G, q, scale);
  } else {
    const int64_t work = (rows / 32 + G) * (cols / 8);
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((work + 255) / 256, cap));
    const size_t shmem = sizeof(int64_t) * (size_t)(2 * G + 2);
    hipLaunchKernelGGL(moe::mx_quant_cols_kernel, dim3((unsigned)blocks), dim3(256), shmem, s, x, rows, cols,
                       group_sizes, G, q, scale, flag);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
