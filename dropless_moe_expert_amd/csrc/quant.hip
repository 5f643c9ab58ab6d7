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
constexpr int QT_LD = QT_C + 2;   // bf16 per LDS row: the pad staggers the column reads over the banks

// PRODUCER 0: the tile is read from x [rows, cols].  PRODUCER 1: the tile
// is the SwiGLU backward dgu [rows, cols = 2f] (bf16-rounded, as
// moe_swiglu_backward stores it), made from x = gu [rows, 2f] and dh
// [rows, f]: dgu never exists in bf16.
template <int PRODUCER>
__global__ __launch_bounds__(256) void mx_quant_t_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ dh, int64_t rows, int cols,
                                                         const int32_t* __restrict__ group_sizes, int G,
                                                         int64_t k_cap, uint8_t* __restrict__ qT,
                                                         uint8_t* __restrict__ scaleT, uint8_t* __restrict__ q0,
                                                         uint8_t* __restrict__ s0, uint32_t* flag) {
  extern __shared__ int64_t sh[];  // grouped: [0,G]: row offsets; [G+1, 2G+2): padded starts
  __shared__ uint16_t xt[2 * QT_R * QT_LD];             // two position units, bf16, row-major
  __shared__ __align__(16) uint8_t ct[QT_C * 2 * QT_R]; // their codes, column-major (128 per column)
  __shared__ uint8_t st[QT_C * 4];                      // their scales, four per column
  int64_t* roff = sh;
  int64_t* kpad = sh + G + 1;
  const bool grouped = group_sizes != nullptr;
  if (grouped) {
    // row offsets and padded starts: each thread sums its run of groups,
    // a block scan of the sums, then each thread writes its run's prefixes
    __shared__ int64_t scan_r[256], scan_k[256];
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
  for (int64_t tile = blockIdx.x; tile < ntp * ntc; tile += gridDim.x) {
    const int64_t tp = tile / ntc;
    const int c0 = (int)(tile - tp * ntc) * (PRODUCER == 2 ? 32 : QT_C);
    // each unit (64 positions) of the pair resolves its own rows and outputs
    int64_t r0[2], ldq = grouped ? k_cap : rows;
    int n[2];
    bool val[2];
    uint8_t* qb[2];   // the unit's first code in column 0's qT row
    uint8_t* sb[2];   // its first scale in column 0's scaleT row
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t tk = 2 * tp + h;
      val[h] = tk < ntk;
      r0[h] = 0;
      n[h] = 0;
      qb[h] = qT;
      sb[h] = scaleT;
      if (!val[h]) continue;
      if (grouped) {
        int lo = 0, hi = G - 1;   // last g with kpad[g] <= 64 tk
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (kpad[mid] <= QT_R * tk) lo = mid; else hi = mid - 1;
        }
        r0[h] = roff[lo] + (QT_R * tk - kpad[lo]);
        n[h] = (int)max((int64_t)0, min((int64_t)QT_R, roff[lo + 1] - r0[h]));
        qb[h] = qT + QT_R * tk;
        sb[h] = scaleT + 2 * tk;
      } else {
        const int64_t g = tk / tpb, b = tk - g * tpb;
        r0[h] = g * rows + QT_R * b;
        n[h] = QT_R;
        qb[h] = qT + g * cols * rows + QT_R * b;
        sb[h] = scaleT + g * cols * (rows / 32) + 2 * b;
      }
    }
    // 1. the pair's rows: 128 rows x 8 pieces of 8 columns, four per thread
    __syncthreads();   // the previous tile's LDS is read out
    if constexpr (PRODUCER == 2) {
      // 128 rows x 4 pieces of 8 gate/up pairs, two per thread: dg to columns
      // 8 jp .., du to 32 + 8 jp ..
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int u = t + 256 * k, rr = u >> 2, jp = u & 3, j = c0 + 8 * jp;
        const int h = rr >> 6, r = rr & 63;
        uint4 vg = make_uint4(0, 0, 0, 0), vu = make_uint4(0, 0, 0, 0);
        if (r < n[h] && j < fh) {
          const int64_t row = r0[h] + r;
          float g[8], uu[8], dd[8], dg[8], du[8];
          unpack8(*reinterpret_cast<const uint4*>(x + row * cols + j), g);
          unpack8(*reinterpret_cast<const uint4*>(x + row * cols + fh + j), uu);
          unpack8(*reinterpret_cast<const uint4*>(dh + row * fh + j), dd);
#pragma unroll
          for (int e = 0; e < 8; ++e) swiglu_grad(g[e], uu[e], dd[e], dg[e], du[e]);
          vg = pack8(dg);
          vu = pack8(du);
        }
        uint32_t* d = reinterpret_cast<uint32_t*>(xt + rr * QT_LD + 8 * jp);
        d[0] = vg.x; d[1] = vg.y; d[2] = vg.z; d[3] = vg.w;
        d = reinterpret_cast<uint32_t*>(xt + rr * QT_LD + 32 + 8 * jp);
        d[0] = vu.x; d[1] = vu.y; d[2] = vu.z; d[3] = vu.w;
      }
    } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = t + 256 * k, rr = u >> 3, c = (u & 7) * 8;
      const int h = rr >> 6, r = rr & 63;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < n[h] && c0 + c < cols) {
        const int64_t row = r0[h] + r;
        if constexpr (PRODUCER == 0) {
          v = *reinterpret_cast<const uint4*>(x + row * cols + c0 + c);
        } else {
          const int f = cols / 2, j = (c0 + c) % f;   // f % 8 == 0: a piece is all gate or all up
          float g[8], uu[8], dd[8], dg[8], du[8];
          unpack8(*reinterpret_cast<const uint4*>(x + row * cols + j), g);
          unpack8(*reinterpret_cast<const uint4*>(x + row * cols + f + j), uu);
          unpack8(*reinterpret_cast<const uint4*>(dh + row * f + j), dd);
#pragma unroll
          for (int e = 0; e < 8; ++e) swiglu_grad(g[e], uu[e], dd[e], dg[e], du[e]);
          v = pack8(c0 + c < f ? dg : du);
        }
      }
      uint32_t* d = reinterpret_cast<uint32_t*>(xt + rr * QT_LD + c);   // 4-byte aligned (QT_LD even)
      d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
    }
    }
    __syncthreads();
    // 2a. one thread per (column, 32-position block): amax, scale, 32 codes into the column
    {
      const int c = t & (QT_C - 1), b = t >> 6;   // b = 0..3 over the pair's 128 positions
      float amax = 0.f;
#pragma unroll 8
      for (int i = 0; i < 32; ++i) amax = mx_absmax(amax, __uint_as_float((uint32_t)xt[(32 * b + i) * QT_LD + c] << 16));
      const int e = mx_exponent(amax);
      st[4 * c + b] = (uint8_t)(e + 127);
      uint32_t w[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float((uint32_t)xt[(32 * b + 4 * q + i) * QT_LD + c] << 16);
        w[q] = mx_codes4(f[0], f[1], f[2], f[3], e);
      }
      if (e == kMxNaN) {
        // a NaN block's codes are NaN only at the group's rows: the padding
        // positions past them keep zero codes, as in every other block
        const int nv = min(32, max(0, n[b >> 1] - 32 * (b & 1)));
#pragma unroll
        for (int q = 0; q < 8; ++q)
#pragma unroll
          for (int k = 0; k < 4; ++k)
            if (4 * q + k >= nv) w[q] &= ~(0xFFu << (8 * k));
      }
      uint4* d = reinterpret_cast<uint4*>(ct + c * (2 * QT_R) + 32 * b);
      d[0] = make_uint4(w[0], w[1], w[2], w[3]);
      d[1] = make_uint4(w[4], w[5], w[6], w[7]);
    }
    // 2b. one thread per (row, 32-column block): the axis-0 quantisation of the valid rows
    if (q0) {
      const int rr = t >> 1, b = t & 1, cb = gcol(c0, 32 * b);
      const int h = rr >> 6, r = rr & 63;
      if (r < n[h] && colvalid(c0, 32 * b)) {
        // two passes over the row's 32 values in LDS (pairs per 4-byte read):
        // amax, then the codes; few live registers keep the occupancy up
        const uint32_t* xr = reinterpret_cast<const uint32_t*>(xt + rr * QT_LD + 32 * b);   // QT_LD even
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t p = xr[i];
          amax = mx_absmax(mx_absmax(amax, __uint_as_float(p << 16)), __uint_as_float(p & 0xFFFF0000u));
        }
        const int e = mx_exponent(amax);
        asm volatile("" ::: "memory");   // re-read the row below instead of keeping 16 words live
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t p0 = xr[2 * q], p1 = xr[2 * q + 1];
          w[q] = mx_codes4(__uint_as_float(p0 << 16), __uint_as_float(p0 & 0xFFFF0000u), __uint_as_float(p1 << 16),
                           __uint_as_float(p1 & 0xFFFF0000u), e);
        }
        const int64_t row = r0[h] + r;
        uint4* d = reinterpret_cast<uint4*>(q0 + row * cols + cb);
        d[0] = make_uint4(w[0], w[1], w[2], w[3]);
        d[1] = make_uint4(w[4], w[5], w[6], w[7]);
        s0[row * (cols / 32) + cb / 32] = (uint8_t)(e + 127);
      }
    }
    __syncthreads();
    // 3. column rows out: lanes (column, 16-byte piece of the pair's 128 codes),
    //    so one store instruction writes 8 columns x 128 contiguous bytes when the
    //    two units are adjacent in the column row; the scale pairs
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int idx = t + 256 * k, c = idx >> 3, p8 = idx & 7, h = p8 >> 2;
      if (val[h] && colvalid(c0, c)) {
        const int64_t col = gcol(c0, c);
        *reinterpret_cast<uint4*>(qb[h] + col * ldq + 16 * (p8 & 3)) =
            *reinterpret_cast<const uint4*>(ct + c * (2 * QT_R) + 16 * p8);
        if ((p8 & 3) == 0)
          *reinterpret_cast<uint16_t*>(sb[h] + col * (ldq / 32)) =
              (uint16_t)(st[4 * c + 2 * h] | ((uint16_t)st[4 * c + 2 * h + 1] << 8));
      }
    }
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

extern "C" moe_status_t mxfp8_quantize_transposed_launch(const uint16_t* x, const uint16_t* dh, int64_t rows,
                                                         int32_t cols,
                                                         const int32_t* group_sizes, int32_t G, int64_t k_cap,
                                                         uint8_t* qT, uint8_t* scaleT, uint8_t* q0, uint8_t* s0,
                                                         uint32_t* flag, hipStream_t s) {
  const int64_t cap = (int64_t)moe_host::device_cu_count() * 8;
  const int64_t ntk = group_sizes ? k_cap / 64 : (int64_t)G * (rows / 64);   // an upper bound when grouped
  const int64_t work = (ntk + 1) / 2 * ((cols + 63) / 64);   // pairs of 64-position units
  if (work == 0) return MOE_OK;
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(work, cap));
  const size_t shmem = group_sizes ? sizeof(int64_t) * (size_t)(2 * G + 2) : 0;
  if (dh && (cols / 2) % 32 == 0) {
    hipLaunchKernelGGL(moe::mx_quant_t_kernel<2>, dim3((unsigned)blocks), dim3(256), shmem, s, x, dh, rows, cols,
                       group_sizes, G, k_cap, qT, scaleT, q0, s0, flag);
  } else if (dh) {
    hipLaunchKernelGGL(moe::mx_quant_t_kernel<1>, dim3((unsigned)blocks), dim3(256), shmem, s, x, dh, rows, cols,
                       group_sizes, G, k_cap, qT, scaleT, q0, s0, flag);
  } else {
    hipLaunchKernelGGL(moe::mx_quant_t_kernel<0>, dim3((unsigned)blocks), dim3(256), shmem, s, x, dh, rows, cols,
                       group_sizes, G, k_cap, qT, scaleT, q0, s0, flag);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
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
