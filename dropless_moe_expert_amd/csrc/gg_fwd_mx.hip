// Grouped GEMM, ragged along rows, MXFP8 operands (E4M3 codes, E8M0 scale
// per 32 along K), bf16 output, optional SwiGLU epilogue.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", section "Optimization 1: Grouped GEMM": MXFP8 block scaling for
// the expert matmuls, fed by the group-aware quantisation kernels.
//
// Same pipeline as the bf16 forward kernel (persistent tiles from the device
// group prefix, 256 x 256 tiles, 8 wavefronts in a ping-pong schedule,
// direct-to-LDS loads in 64-byte rows, stages loaded three ahead), with K
// staged 64 codes at a time and
// v_mfma_scale_f32_32x32x64_f8f6f4: lane l holds row l % 32 and, for the
// lane group g = l / 32, codes k = 16g..16g+15 and 32+16g..32+16g+15 of the
// stage plus the scale of k-block g (layout verified on the hardware).
// Each stage also carries its weight rows' scales: a row's two scale bytes
// arrive by a 2-byte direct load into one LDS word.  The activation rows'
// scales travel 8 stages at a time (a row's 16 bytes for 512 codes are
// contiguous in memory), spread over the loads of the previous 8 stages into
// one of three 8 KB LDS areas: one 2-byte load per row and stage, each from
// its own row, had cost 13 % of the gate/up GEMM's time.  Four stages of
// 33 KB and the three scale areas fit LDS (156 KB).
#include <atomic>

#include "gg_pipeline.h"

namespace moe {
namespace fwd {

constexpr int WM = 4;                          // wavefront grid 4 (m) x 2 (n)
constexpr int NWAVE = WM * WN, THREADS = NWAVE * 64;
constexpr int WTM = BM / WM;                   // 64 x 128 per wavefront
constexpr int LPW = (BM + BN) / 16 / NWAVE;    // direct row loads per wavefront and stage (4)
namespace mx {

constexpr int SC_W = 2 * XOFF;                  // W scale words [BN]
constexpr int MSTAGE = SC_W + BN * 4;           // 33 KB
constexpr int LPW_MX = LPW + 1;                 // per wavefront and stage: the row loads + 1 scale load
// X scale areas: area c % 3 holds chunk c (stages 8c..8c+7); piece p (rows
// 32p..32p+31) at 1 KB p; in it, the word of lane t = 64 (w % 4) + l holds
// bytes 2 (t % 8) and 2 (t % 8) + 1 of row 32p + t / 8's 16 bytes, i.e. the
// two scales of stage 8c + t % 8
constexpr int XCH = 8;
constexpr int XCH_BYTES = 8 * 1024;
constexpr int NXCH = 3;
constexpr int MTN = WTN / 32, MTM = WTM / 32;   // 4 x 2 subtiles of 32 x 32
// packed weights: per (expert, n-tile, stage) 16 KB of codes in LDS slot
// order, then the 256 rows' scale words (bytes 2kt, 2kt + 1 of each row's
// scales, zero-extended to 4 bytes) in LDS order
constexpr int PK_CODES = BN * ROWB;
constexpr int PK_STAGE = PK_CODES + BN * 4;     // 17 KB

// One 2-byte direct load per wavefront and stage.  Wavefront w < 4, lane l:
// the two scale bytes of stage kt of W row 64 w + l into the low half of its
// LDS word.  Wavefront w >= 4: piece kt % 8 of X scale chunk kt / 8 + 1.
// Chunk c + 1's first piece goes out with stage 8c, while stage 8c - 4 is
// read; its area, (c + 1) % 3, last held chunk c - 2 (stages up to 8c - 9).
// Both kinds are one instruction with operands chosen per wavefront, so the
// loop has no branch on the wavefront's role.
struct Scales {
  uint32_t woff;        // W: the row's scale offset (packed: within the stage block)
  uint32_t xt2;         // X: this lane's two bytes' offset within a row's 16, 2 (t % 8)
  int xr;               // X: its row within a piece, t / 8
  int rows;             // valid rows of the tile
  int t;                // lane within the four wavefronts of its kind
  int is_w;             // a W-scale wavefront
  template <typename WRow>
  __device__ __forceinline__ void init(int64_t ld, WRow wrow, int rows_) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    is_w = wave < 4;
    t = (wave & 3) * 64 + lane;
    woff = (uint32_t)(wrow(t) * ld);
    xt2 = 2u * (uint32_t)(t & 7);
    xr = t >> 3;
    rows = rows_;
  }
  // this lane's offset for piece p of X chunk c (rows lds_b bytes apart, xlim
  // of them from the scales' base to the row's end): bytes past the row's
  // end re-read its first two (never used), so no load leaves the row
  __device__ __forceinline__ uint32_t xoff(int p, int c, int lds_b, int xlim) const {
    const uint32_t rb = (uint32_t)(min(32 * p + xr, rows - 1) * lds_b);
    const uint32_t cb = 16u * (uint32_t)c;
    return xt2 + cb < (uint32_t)xlim ? rb + cb + xt2 : rb;
  }
  __device__ __forceinline__ void load(uint32_t l0, uint32_t off, const uint8_t* base) const {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "global_load_lds_ushort %1, %2"
        :
        : "s"(l0), "v"(off), "s"(base)
        : "memory", "m0");
  }
  // the scale load that goes with stage s; wsrc: stage s's W scale source
  // (packed: the stage block, else the expert's scales + 2 s)
  __device__ __forceinline__ void issue(uint8_t* buf, uint8_t* xch, const uint8_t* wsrc, const uint8_t* xsb, int s,
                                        int lds_b, int xlim) const {
    const int c = s / XCH + 1, p = s % XCH;
    const uint32_t wq = (uint32_t)(wave_id() & 3) * 256;   // wavefront-uniform
    const uint32_t wl0 = (uint32_t)(uintptr_t)(lds_ptr_t)buf + SC_W + wq;
    const uint32_t xl0 = (uint32_t)(uintptr_t)(lds_ptr_t)xch + (c % NXCH) * XCH_BYTES + p * 1024 + wq;
    // the role is wavefront-uniform: keep the choice of LDS and global base
    // in scalar registers (the loads' m0 and base operands must be scalars)
    const bool w = __builtin_amdgcn_readfirstlane((int)is_w) != 0;
    const uint64_t base = (uint64_t)(uintptr_t)(w ? wsrc : xsb);
    const uint32_t blo = __builtin_amdgcn_readfirstlane((uint32_t)base);
    const uint32_t bhi = __builtin_amdgcn_readfirstlane((uint32_t)(base >> 32));
    // the offset is chosen per lane (threads < 256 are the W wavefronts), a
    // plain select: as a choice on the uniform role the compiler branched
    // around the X offset arithmetic and ran out of registers
    const uint32_t xof = xoff(p, c, lds_b, xlim);
    load(__builtin_amdgcn_readfirstlane(w ? wl0 : xl0), threadIdx.x < 256 ? woff : xof,
         reinterpret_cast<const uint8_t*>((uintptr_t)(((uint64_t)bhi << 32) | blo)));
  }
  // chunk 0, before stage 0: all eight loads by every wavefront (the W
  // wavefronts write the same words as the X ones)
  __device__ __forceinline__ void issue_first(uint8_t* xch, const uint8_t* xsb, int lds_b, int xlim) const {
    const uint32_t l0 = (uint32_t)(uintptr_t)(lds_ptr_t)xch + (uint32_t)(wave_id() & 3) * 256;
#pragma unroll
    for (int p = 0; p < XCH; ++p) load(l0 + p * 1024, xoff(p, 0, lds_b, xlim), xsb);
  }
};

struct Frags {
  i32x8_t w[MTN], x[MTM];
  int ws[MTN], xs[MTM];
};

__device__ __forceinline__ i32x8_t ld32(const uint8_t* rowp, int slot_lo, int slot_hi) {
  const uint4 lo = *reinterpret_cast<const uint4*>(rowp + slot_lo * 16);
  const uint4 hi = *reinterpret_cast<const uint4*>(rowp + slot_hi * 16);
  return i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// xsw: the words of stage kt in its X scale area, (const uint32_t*)area +
// kt % 8; row r's is at xsw[256 (r / 32) + 8 (r % 32)]
__device__ __forceinline__ void read_frags(const uint8_t* buf, Frags& fr, const uint32_t* xsw) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int wn = wave / WM, wm = wave % WM;
  const int r32 = lane & 31, g = lane >> 5;
  const int sw = swz_row<1>(r32);                // rows are 32-aligned bases + r32
  const int s_lo = g ^ sw, s_hi = (2 + g) ^ sw;
  const uint32_t* scw = reinterpret_cast<const uint32_t*>(buf + SC_W);
#pragma unroll
  for (int i = 0; i < MTN; ++i) {
    const int row = wn * WTN + i * 32 + r32;
    fr.w[i] = ld32(buf + row * ROWB, s_lo, s_hi);
    fr.ws[i] = (int)((scw[row] >> (8 * g)) & 0xFF);
  }
#pragma unroll
  for (int j = 0; j < MTM; ++j) {
    const int row = wm * WTM + j * 32 + r32;
    fr.x[j] = ld32(buf + XOFF + row * ROWB, s_lo, s_hi);
    fr.xs[j] = (int)((xsw[(row >> 5) * 256 + r32 * 8] >> (8 * g)) & 0xFF);
  }
}

// serpentine order, as in the bf16 kernel: consecutive MFMAs share an operand
__device__ __forceinline__ void mma(const Frags& fr, f32x16_t (&acc)[MTN][MTM]) {
#pragma unroll
  for (int i = 0; i < MTN; ++i)
#pragma unroll
    for (int jj = 0; jj < MTM; ++jj) {
      const int j = (i & 1) ? MTM - 1 - jj : jj;
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fr.w[i], fr.x[j], acc[i][j], 0, 0, 0, fr.ws[i], 0,
                                                                   fr.xs[j]);
    }
}

// 32x32 accumulator: element v of lane (r32, g) is n = 8*(v/4) + 4*g + v%4,
// m = r32 within the subtile.  SwiGLU: subtiles i < MTN/2 hold gate columns,
// i + MTN/2 the up columns of the same j.
// SwiGLU epilogues: EPI_SWIGLU stores h = bf16(silu(g) * u); EPI_SWIGLU_MXFP8
// quantises that bf16 h per 32 columns as mxfp8_group_quantize (axis 0) does,
// storing E4M3 codes to C and E8M0 scales to C_aux.  A 32-column block of a
// row lies in lanes (r32, 0) and (r32, 1) of one subtile, 16 values each, so
// its amax takes one exchange across the lane halves.  The quantised tile
// (256 rows x 128 codes, 256 x 4 scales) is assembled in LDS (the stage
// buffers, free once every wavefront has left the K loop) and written out by
// the whole workgroup as 16-byte row pieces and 4-byte scale words.
// Copies a tile staged in LDS out to global memory: row r (r < rows) of the
// tile lies in buffer r / WTM at (r % WTM) * RB, its 16-byte units u XOR-
// swizzled by (r % WTM) % UR; the first half of a row's units goes to
// columns col_a + 8u (those < lim_a), the second half to col_b + 8(u - UR/2)
// (those < lim_b), of rows ld bf16 elements apart from cbase.  Each
// thread's LDS reads go four at a time ahead of their stores, in a rolled
// loop; a piece is a 32-bit offset from cbase (256 rows of at most 2^22
// columns).
template <int RB>
__device__ __forceinline__ void copy_staged(uint8_t* s0, uint8_t* s1, uint8_t* s2, uint8_t* s3, uint8_t* cbase,
                                            int ld, int rows, int col_a, int lim_a, int col_b, int lim_b) {
  constexpr int UR = RB / 16;
  constexpr int NPT = BM * UR / THREADS;   // 16-byte pieces per thread
  constexpr int NB = 4;
  static_assert(BM * UR % THREADS == 0 && NPT % NB == 0, "whole batches");
  auto buf = [&](int i) { return i == 0 ? s0 : i == 1 ? s1 : i == 2 ? s2 : s3; };
#pragma unroll 1
  for (int k0 = 0; k0 < NPT; k0 += NB) {
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
      const bool first = u < UR / 2;
      const int col = first ? col_a + 8 * u : col_b + 8 * (u - UR / 2);
      if (row < rows && col < (first ? lim_a : lim_b))
        *reinterpret_cast<uint4*>(cbase + (uint32_t)(row * ld + col) * 2u) = v[k];
    }
  }
}

//
// The plain bf16 output (down GEMM, data and weight gradients) also leaves
// through LDS: each wavefront writes its 64 rows into the stage buffer of its
// row slot (16-byte units XOR-swizzled by row), then the workgroup copies
// whole 512-byte tile rows out as 16-byte pieces, each thread's LDS reads
// four at a time ahead of their stores.
template <int EPI>
__device__ __forceinline__ void store(const GGArgs& a, f32x16_t (&acc)[MTN][MTM], int64_t m0, int rows, int n0,
                                      int ncols, int f, uint8_t* lds_codes, uint8_t* lds_scales, uint8_t* s2,
                                      uint8_t* s3) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int wn = wave / WM, wm = wave % WM;
  const int r32 = lane & 31, g = lane >> 5;
  if constexpr (EPI == MOE_EPI_NONE) {
    constexpr int RB = 512, UR = RB / 16;   // bytes and 16-byte units per staged row
    auto buf = [&](int i) { return i == 0 ? lds_codes : i == 1 ? lds_scales : i == 2 ? s2 : s3; };
    __syncthreads();   // every wavefront has read its last stage
    uint8_t* sb = buf(wm);
#pragma unroll
    for (int j = 0; j < MTM; ++j) {
      const int rl = j * 32 + r32;   // row within the slot
#pragma unroll
      for (int i = 0; i < MTN; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = wn * WTN + i * 32 + q * 8 + g * 4;
          const uint2 w = make_uint2(pack_bf16x2(acc[i][j][q * 4], acc[i][j][q * 4 + 1]),
                                     pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]));
          *reinterpret_cast<uint2*>(sb + rl * RB + (((col >> 3) ^ (rl % UR)) << 4) + ((col >> 2) & 1) * 8) = w;
        }
      }
    }
    __syncthreads();
    copy_staged<RB>(lds_codes, lds_scales, s2, s3, a.C + m0 * (int64_t)ncols * 2, ncols, rows, n0, ncols,
                    n0 + BN / 2, ncols);
    return;
  }
  if constexpr (EPI == MOE_EPI_SWIGLU_MXFP8) {
    constexpr int TC = BN / 2;   // codes per tile row
    __syncthreads();             // every wavefront has read its last stage
#pragma unroll
    for (int j = 0; j < MTM; ++j) {
      const int mr = wm * WTM + j * 32 + r32;
#pragma unroll
      for (int i = 0; i < MTN / 2; ++i) {
        // h of this lane's 16 columns, rounded to bf16 exactly as the bf16 store does
        float h[16];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t p = pack_bf16x2(silu_f32(acc[i][j][2 * q]) * acc[i + MTN / 2][j][2 * q],
                                         silu_f32(acc[i][j][2 * q + 1]) * acc[i + MTN / 2][j][2 * q + 1]);
          h[2 * q] = bf16_bits_to_f32(p & 0xFFFFu);
          h[2 * q + 1] = bf16_bits_to_f32(p >> 16);
        }
        float amax = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) amax = mx_absmax(amax, h[v]);
        amax = mx_absmax(amax, __shfl_xor(amax, 32, 64));
        const int e = mx_exponent(amax);
        const int cb = wn * (WTN / 2) + i * 32;   // the block's first column in the tile
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t codes = mx_codes4(h[4 * q], h[4 * q + 1], h[4 * q + 2], h[4 * q + 3], e);
          *reinterpret_cast<uint32_t*>(lds_codes + mr * TC + cb + q * 8 + g * 4) = codes;
        }
        if (g == 0) lds_scales[mr * (TC / 32) + cb / 32] = (uint8_t)(e + 127);
      }
    }
    __syncthreads();
    // rows < rows, columns n0 + [0, 128) < f (f % 32 == 0: whole blocks)
    const int ncb = min(TC, f - n0);   // valid codes in a tile row (multiple of 32)
    for (int c = threadIdx.x; c < BM * (TC / 16); c += THREADS) {
      const int row = c / (TC / 16), piece = c % (TC / 16);
      if (row < rows && piece * 16 < ncb)
        *reinterpret_cast<uint4*>(a.C + (m0 + row) * (int64_t)f + n0 + piece * 16) =
            *reinterpret_cast<const uint4*>(lds_codes + row * TC + piece * 16);
    }
    const int64_t lds_row = f / 32;   // scale bytes per row
    for (int row = threadIdx.x; row < rows; row += THREADS) {
      uint8_t* dst = a.Caux + (m0 + row) * lds_row + n0 / 32;
      const uint32_t w = *reinterpret_cast<const uint32_t*>(lds_scales + row * (TC / 32));
      if (ncb == TC && (reinterpret_cast<uintptr_t>(dst) & 3u) == 0) {
        *reinterpret_cast<uint32_t*>(dst) = w;
      } else {
        for (int b = 0; b < ncb / 32; ++b) dst[b] = (uint8_t)(w >> (8 * b));
      }
    }
    return;
  }
  // SwiGLU without quantisation: h (and, with C_aux, the pre-activations
  // [gate | up] for the backward) staged through LDS as the plain output
  // is.  h is formed and packed first, so the accumulators are free once
  // the pre-activations are in LDS.
  if constexpr (EPI == MOE_EPI_SWIGLU) {
  auto buf = [&](int i) { return i == 0 ? lds_codes : i == 1 ? lds_scales : i == 2 ? s2 : s3; };
  uint8_t* sb = buf(wm);
  auto put = [&](int rb, int rl, int col, uint2 w) {
    const int ur = rb / 16;
    *reinterpret_cast<uint2*>(sb + rl * rb + (((col >> 3) ^ (rl % ur)) << 4) + ((col >> 2) & 1) * 8) = w;
  };
  uint2 hp[MTN / 2][MTM][4];
#pragma unroll
  for (int j = 0; j < MTM; ++j)
#pragma unroll
    for (int i = 0; i < MTN / 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = silu_f32(acc[i][j][q * 4 + e]) * acc[i + MTN / 2][j][q * 4 + e];
        hp[i][j][q] = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
      }
  __syncthreads();   // every wavefront has read its last stage
  if (a.Caux) {
#pragma unroll
    for (int j = 0; j < MTM; ++j) {
      const int rl = j * 32 + r32;
#pragma unroll
      for (int i = 0; i < MTN / 2; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = wn * (WTN / 2) + i * 32 + q * 8 + g * 4;
          put(512, rl, col, make_uint2(pack_bf16x2(acc[i][j][q * 4], acc[i][j][q * 4 + 1]),
                                       pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3])));
          put(512, rl, BN / 2 + col,
              make_uint2(pack_bf16x2(acc[i + MTN / 2][j][q * 4], acc[i + MTN / 2][j][q * 4 + 1]),
                         pack_bf16x2(acc[i + MTN / 2][j][q * 4 + 2], acc[i + MTN / 2][j][q * 4 + 3])));
        }
    }
    __syncthreads();
    copy_staged<512>(lds_codes, lds_scales, s2, s3, a.Caux + m0 * (int64_t)(2 * f) * 2, 2 * f, rows, n0, f,
                     f + n0, 2 * f);
    __syncthreads();   // every thread has read the pre-activations out
  }
#pragma unroll
  for (int j = 0; j < MTM; ++j) {
    const int rl = j * 32 + r32;
#pragma unroll
    for (int i = 0; i < MTN / 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) put(256, rl, wn * (WTN / 2) + i * 32 + q * 8 + g * 4, hp[i][j][q]);
  }
  __syncthreads();
  copy_staged<256>(lds_codes, lds_scales, s2, s3, a.C + m0 * (int64_t)f * 2, f, rows, n0, f, n0 + BN / 4, f);
  }
}

// The loads of one tile's K stages (64 codes each): X rows (the MFMA's m
// side), W rows or packed W blocks (its n side), their scales.
template <bool PACKED>
struct MxLoads {
  Rows<BM, NWAVE, 1> xl;
  Rows<BN, NWAVE, 1> wl;
  Scales sl;
  const uint8_t* xbase;   // stage 0 of the X rows
  const uint8_t* wbase;   // stage 0 of the W block (packed) or of the W rows
  int wstride;            // bytes from one stage's W block to the next
  const uint8_t* xsb;     // the X rows' scales at stage 0
  const uint8_t* wsb;     // unpacked: the W rows' scales at stage 0
  int lds_b;              // scale bytes per row
  int xlim;               // scale bytes from xsb to the end of an X row
  __device__ __forceinline__ void issue(uint8_t* buf, uint8_t* xch, int s) const {
    const uint8_t* wstage = wbase + (int64_t)s * wstride;
    wl.issue(buf, wstage);
    xl.issue(buf + XOFF, xbase + s * ROWB);
    sl.issue(buf, xch, PACKED ? wstage : wsb + 2 * s, xsb, s, lds_b, xlim);
  }
};

// One tile's K loop (nk >= 1 stages) into acc.
template <bool PACKED>
__device__ __forceinline__ void mx_k_loop(const MxLoads<PACKED>& ld, int nk, f32x16_t (&acc)[MTN][MTM], uint8_t* b0,
                                          uint8_t* b1, uint8_t* b2, uint8_t* b3, uint8_t* xch) {
  auto issue = [&](uint8_t* buf, int s) { ld.issue(buf, xch, s); };
  auto xscales = [&](int kt) {
    return reinterpret_cast<const uint32_t*>(xch + (kt / XCH % NXCH) * XCH_BYTES) + kt % XCH;
  };
  // Ping-pong schedule: step kt is a memory phase (issue stage kt + 3 into
  // the buffer of stage kt - 1, read stage kt's fragments and scales), a
  // barrier, and a compute phase (its 8 scaled MFMAs from registers).  The
  // second wavefront of every SIMD runs one barrier behind the first, so
  // one of the two issues MFMAs while the other reads LDS.  Every barrier
  // is preceded by this wavefront's wait for the stage the wavefronts
  // past it will read: stage kt before the memory phase, stage kt + 1
  // (and this step's LDS reads) before the compute phase.
  const bool second = wave_id() >= NWAVE / 2;
  auto barrier = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // wait until at most n stages' loads of this wavefront are in flight
  auto wait_stages = [&](int n) {
    if (n >= 2) {
      MOE_WAIT_VMCNT(2 * LPW_MX);
    } else if (n == 1) {
      MOE_WAIT_VMCNT(LPW_MX);
    } else {
      MOE_WAIT_VMCNT(0);
    }
  };
  Frags fr;
  auto step_fast = [&](uint8_t* cur, uint8_t* lbuf, int kt) {
    wait_stages(2);
    barrier();
    issue(lbuf, kt + 3);
    read_frags(cur, fr, xscales(kt));
    wait_stages(2);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    barrier();
    mma(fr, acc);
  };
  auto step = [&](uint8_t* cur, uint8_t* lbuf, int kt) {
    wait_stages(min(2, nk - 1 - kt));
    barrier();
    if (kt + 3 < nk) issue(lbuf, kt + 3);
    read_frags(cur, fr, xscales(kt));
    wait_stages(min(2, nk - 2 - kt));
    __builtin_amdgcn_s_waitcnt(0xC07F);
    if (!(second && kt == nk - 1)) barrier();   // evens the two halves' barrier counts
    mma(fr, acc);
  };

  __syncthreads();
  ld.sl.issue_first(xch, ld.xsb, ld.lds_b, ld.xlim);
  issue(b0, 0);
  if (nk > 1) issue(b1, 1);
  if (nk > 2) issue(b2, 2);
  if (second) {   // the half-step offset; stage 0 must have landed before it
    wait_stages(min(2, nk - 1));
    barrier();
  }
  int kt = 0;
  for (; kt + 7 <= nk; kt += 4) {   // every step of the group issues a stage (kt + 6 < nk)
    step_fast(b0, b3, kt);
    step_fast(b1, b0, kt + 1);
    step_fast(b2, b1, kt + 2);
    step_fast(b3, b2, kt + 3);
  }
  if (kt < nk) step(b0, b3, kt);
  if (kt + 1 < nk) step(b1, b0, kt + 1);
  if (kt + 2 < nk) step(b2, b1, kt + 2);
  if (kt + 3 < nk) step(b3, b2, kt + 3);
  if (kt + 4 < nk) step(b0, b3, kt + 4);
  if (kt + 5 < nk) step(b1, b0, kt + 5);
}

// Split tail (gg_pipeline.h): the counters of this kernel's calls.
__device__ SplitSlots g_split_sched_mx = initial_split_slots();

// Unit tail_unit of a split tail: its partial sums (acc) go to its slot of
// the workspace, each thread's accumulators in register order; it counts
// itself in at its tile; true, with acc holding the tile's sums (its units'
// partials added in split order), to the unit that completes the tile.
__device__ __forceinline__ bool split_reduce_mx(const GGArgs& a, const SplitTail& sp, int64_t tail_unit,
                                                f32x16_t (&acc)[MTN][MTM], int32_t* box) {
  constexpr int SLOT = BM * BN;
  static_assert(MTN * MTM * 16 * THREADS == SLOT, "a unit's partials fill its slot");
  const int t = threadIdx.x;
  const int64_t tile_tail = tail_unit / sp.S;
  float* const mine = a.part + tail_unit * SLOT;
#pragma unroll
  for (int i = 0; i < MTN; ++i)
#pragma unroll
    for (int j = 0; j < MTM; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<f32x4_t*>(mine + (((i * MTM + j) * 4 + q) * THREADS + t) * 4) =
            f32x4_t{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");   // this thread's partials are visible to the device
  __syncthreads();                                      // every thread's, and every wavefront has left its K loop
  if (t == 0) {
    DeviceWord w{g_split_sched_mx.w[a.sched_slot] + tile_tail};
    box[0] = (int32_t)tq::take(w, a.sched_epoch) == sp.S - 1;
  }
  __syncthreads();
  if (!__builtin_amdgcn_readfirstlane(box[0])) return false;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // the other units' partials
  const float* const first = a.part + tile_tail * sp.S * SLOT;
#pragma unroll
  for (int i = 0; i < MTN; ++i)
#pragma unroll
    for (int j = 0; j < MTM; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t off = (((i * MTM + j) * 4 + q) * THREADS + t) * 4;
        f32x4_t v = *reinterpret_cast<const f32x4_t*>(first + off);
        for (int u = 1; u < sp.S; ++u) v += *reinterpret_cast<const f32x4_t*>(first + u * SLOT + off);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[i][j][4 * q + e] = v[e];
      }
  return true;
}

template <int EPI, bool PACKED, bool SPLIT = false>
__global__ void __launch_bounds__(THREADS, 1) gg_fwd_mx_kernel(GGArgs a) {
  __shared__ __align__(1024) uint8_t b0[MSTAGE];
  __shared__ __align__(1024) uint8_t b1[MSTAGE];
  __shared__ __align__(1024) uint8_t b2[MSTAGE];
  __shared__ __align__(1024) uint8_t b3[MSTAGE];
  __shared__ __align__(1024) uint8_t xch[NXCH * XCH_BYTES];   // X scales, 8 stages per area
  __shared__ int32_t split_box[1];                             // SPLIT: a unit's arrival result

  if (blockIdx.x == 0 && threadIdx.x < 64) {
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
  const int64_t lda_b = a.K;            // one byte per code
  const int64_t lds_b = a.K / 32;       // scale bytes per row
  const int nk_all = a.K / 64;

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
    constexpr bool SWI = EPI != MOE_EPI_NONE;   // either SwiGLU epilogue: gate/up tile geometry
    const int n0 = SWI ? nt * (BN / 2) : nt * BN;
    const int nrows_b = SWI ? 2 * f : a.N;

    auto xrow = [&](int r) -> int64_t { return min(r, rows - 1); };
    auto wrow = [&](int r) -> int64_t {
      if constexpr (SWI) {
        const int wn = r / WTN, q = r % WTN;
        const int jj = min(n0 + wn * (WTN / 2) + (q % (WTN / 2)), f - 1);
        return q < WTN / 2 ? jj : f + jj;
      } else {
        return min(n0 + r, a.N - 1);
      }
    };
    Rows<BM, NWAVE, 1> xl;
    Rows<BN, NWAVE, 1> wl;
    Scales sl;
    xl.init(lda_b, xrow);
    sl.init(lds_b, wrow, rows);
    if constexpr (PACKED) {
      const int wave = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
      for (int i = 0; i < Rows<BN, NWAVE, 1>::N; ++i) wl.off[i] = (uint32_t)(((i * NWAVE + wave) * 64 + lane) * 16);
      sl.woff = (uint32_t)(PK_CODES + sl.t * 4);
    } else {
      wl.init(lda_b, wrow);
    }
    const int wstride = PACKED ? PK_STAGE : ROWB;
    // operands and scales from the unit's first stage kt0 on (2 scale bytes per row and stage)
    const uint8_t* xbase = a.A + m0 * lda_b + (int64_t)kt0 * ROWB;
    const uint8_t* wbase = (PACKED ? a.B + ((int64_t)g * a.n_tiles + nt) * nk_all * PK_STAGE
                                   : a.B + (int64_t)g * nrows_b * lda_b) +
                           (int64_t)kt0 * wstride;
    const uint8_t* xsb = a.As + m0 * lds_b + 2 * kt0;
    const uint8_t* wsb = PACKED ? nullptr : a.Bs + (int64_t)g * nrows_b * lds_b + 2 * kt0;
    const int xlim = (int)lds_b - 2 * kt0;   // scale bytes from xsb to the end of an X row

    f32x16_t acc[MTN][MTM];
#pragma unroll
    for (int i = 0; i < MTN; ++i)
#pragma unroll
      for (int j = 0; j < MTM; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    const MxLoads<PACKED> ld{xl, wl, sl, xbase, wbase, wstride, xsb, wsb, (int)lds_b, xlim};
    mx_k_loop<PACKED>(ld, nk, acc, b0, b1, b2, b3, xch);
    if constexpr (SPLIT) {
      // a split unit: partial sums to the workspace; the unit that completes
      // the tile adds them, in split order, and runs the epilogue
      if (tail_unit >= 0 && !split_reduce_mx(a, sp, tail_unit, acc, split_box)) continue;
    }
    store<EPI>(a, acc, m0, rows, n0, SWI ? f : a.N, f, b0, b1, b2, b3);
  }
  if constexpr (SPLIT) {
    if (sp.S > 1) split_finish(a, g_split_sched_mx.w[a.sched_slot], split_box);
  }
}

// Packs codes [G, rows_b, K] and scales [G, rows_b, K/32] (rows_b = N, or the
// fused 2f of SwiGLU) into the (expert, n-tile, stage) blocks the PACKED
// kernel reads: 1024 16-byte code chunks, then 64 chunks of 4 scale words.
template <int EPI>
__global__ __launch_bounds__(256) void pack_mx_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ sc,
                                                     int G, int N, int K, int n_tiles, uint4* __restrict__ out) {
  const int nk = K / 64;
  constexpr int UNITS = PK_STAGE / 16;   // 1088 per block
  const int64_t total = (int64_t)G * n_tiles * nk * UNITS;
  const int f = N / 2;
  const int nrows_b = (EPI == MOE_EPI_SWIGLU) ? 2 * f : N;
  const int sld = K / 32;
  auto src_row = [&](int nt, int r, bool& valid) -> int {
    if constexpr (EPI == MOE_EPI_SWIGLU) {
      const int n0 = nt * (BN / 2), wn = r / WTN, qq = r % WTN;
      const int jj = n0 + wn * (WTN / 2) + (qq % (WTN / 2));
      valid = jj < f;
      return qq < WTN / 2 ? jj : f + jj;
    } else {
      const int row = nt * BN + r;
      valid = row < N;
      return row;
    }
  };
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < total; c += (int64_t)gridDim.x * blockDim.x) {
    const int u = (int)(c % UNITS);
    const int64_t blk = c / UNITS;
    const int kt = (int)(blk % nk);
    const int64_t gn = blk / nk;
    const int nt = (int)(gn % n_tiles), g = (int)(gn / n_tiles);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (u < PK_CODES / 16) {
      const int slot = u & 3, r = u >> 2;
      const int chunk = slot ^ swz_row<1>(r);
      bool valid;
      const int row = src_row(nt, r, valid);
      if (valid) v = *reinterpret_cast<const uint4*>(q + ((int64_t)g * nrows_b + row) * K + kt * 64 + chunk * 16);
    } else {
      uint32_t wv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bool valid;
        const int row = src_row(nt, (u - PK_CODES / 16) * 4 + e, valid);
        wv[e] = 0;
        if (valid) {
          const uint8_t* p = sc + ((int64_t)g * nrows_b + row) * sld + 2 * kt;
          wv[e] = (uint32_t)p[0] | ((uint32_t)p[1] << 8);
        }
      }
      v = make_uint4(wv[0], wv[1], wv[2], wv[3]);
    }
    out[c] = v;
  }
}


// Weight gradient in MXFP8 (the group-aware MXFP8 backward: blog sections
// "What specialized optimizations are required for dropless MoE?" and
// "Optimization 1"): C[g] [P, Q] = sum over group g's rows r of
// A[r, p] * B[r, q], both operands quantised down their rows (blocks of 32
// restarting at every group) and stored transposed by
// mxfp8_quantize_transposed: codes [P | Q, k_cap] with group g at positions
// [K_g, K_g + 64 ceil(s_g / 64)), zero codes past its rows.  A tile
// (g, p-tile, q-tile) is the forward K loop over those positions with the A
// rows as X and the B rows as W; the padding multiplies to zero, and an
// empty group stores zeros.  Tiles come from dynamic queues as in the bf16
// weight gradient: groups ranked largest first (each workgroup ranks them
// into a 2 KB LDS table), dealt to the queues in a snake over the ranks.
// The queues are tile_queue.h's epoch-tagged words, one slot per launch.
__device__ tq::Slots g_wgrad_mx_sched = tq::initial_slots();

__global__ void __launch_bounds__(THREADS, 1) gg_wgrad_mx_kernel(GGArgs a) {
  __shared__ __align__(1024) uint8_t b0[MSTAGE];
  __shared__ __align__(1024) uint8_t b1[MSTAGE];
  __shared__ __align__(1024) uint8_t b2[MSTAGE];
  __shared__ __align__(1024) uint8_t b3[MSTAGE];
  __shared__ __align__(1024) uint8_t xch[NXCH * XCH_BYTES];
  __shared__ uint16_t by_rank[1024];   // group of each rank, largest first (ties: lower index first)

  const int P = a.M, Q = a.N;
  for (int g = threadIdx.x; g < a.G; g += THREADS) {
    const int sg = max(a.sizes[g], 0);
    int r = 0;
    for (int h = 0; h < a.G; ++h) {
      const int sh = max(a.sizes[h], 0);
      r += (sh > sg) || (sh == sg && h < g);
    }
    by_rank[r] = (uint16_t)g;
  }
  const int64_t k_cap = a.K, lds_b = a.K / 32;
  const int per_group = a.p_tiles * a.n_tiles;

  // group g's padded start K_g and padded length, from the device sizes
  // clamped as the quantiser clamps them (>= 0, rows up to m_cap)
  auto group_range = [&](int g, int64_t& kg, int64_t& len) {
    const int lane = threadIdx.x & 63;
    int64_t rbase = 0, kbase = 0;
    kg = 0;
    len = 0;
    for (int c = 0; c < a.G; c += 64) {
      const int gi = c + lane;
      const int64_t sz = gi < a.G ? (int64_t)max(a.sizes[gi], 0) : 0;
      const int64_t rincl = wave_incl_scan(sz);
      const int64_t n = min(rbase + rincl, a.m_cap) - min(rbase + rincl - sz, a.m_cap);
      const int64_t pad = (n + 63) / 64 * 64;
      const int64_t kincl = wave_incl_scan(pad);
      if (g >= c && g < c + 64) {
        kg = kbase + __shfl(kincl - pad, g - c, 64);
        len = __shfl(pad, g - c, 64);
      }
      rbase += __shfl(rincl, 63, 64);
      kbase += __shfl(kincl, 63, 64);
    }
    kg = wave_u64(kg);
    len = wave_u64(len);
  };

  auto process = [&](int g, int rem) {
    const int pt = rem / a.n_tiles, qt = rem - pt * a.n_tiles;
    const int p0 = pt * BM, q0 = qt * BN;
    const int rows = min(BM, P - p0), wrows = min(BN, Q - q0);
    int64_t kg, len;
    group_range(g, kg, len);
    const int nk = (int)(len / 64);
    f32x16_t acc[MTN][MTM];
#pragma unroll
    for (int i = 0; i < MTN; ++i)
#pragma unroll
      for (int j = 0; j < MTM; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    if (nk > 0) {
      auto xrow = [&](int r) -> int64_t { return p0 + min(r, rows - 1); };
      auto wrow = [&](int r) -> int64_t { return q0 + min(r, wrows - 1); };
      MxLoads<false> ld;
      ld.xl.init(k_cap, xrow);
      ld.wl.init(k_cap, wrow);
      ld.sl.init(lds_b, wrow, rows);
      ld.xbase = a.A + kg;
      ld.wbase = a.B + kg;
      ld.wstride = ROWB;
      ld.xsb = a.As + (int64_t)p0 * lds_b + kg / 32;
      ld.wsb = a.Bs + kg / 32;
      ld.lds_b = (int)lds_b;
      ld.xlim = (int)(lds_b - kg / 32);
      mx_k_loop<false>(ld, nk, acc, b0, b1, b2, b3, xch);
    }
    GGArgs ag = a;
    ag.C = a.C + (int64_t)g * P * Q * 2;
    store<MOE_EPI_NONE>(ag, acc, p0, rows, q0, Q, 0, b0, b1, b2, b3);
  };

  __syncthreads();
  tq_walk(g_wgrad_mx_sched.w[a.sched_slot], a.sched_epoch, a.sched_next, a.G, per_group,
          [&](int rank, int rem) { process(by_rank[rank], rem); });
}

}  // namespace mx
}  // namespace fwd

size_t packed_mx_weight_bytes(int G, int N, int K, int epilogue) {
  const int ncols = epilogue == MOE_EPI_SWIGLU ? N / 2 : N;
  const int bn = epilogue == MOE_EPI_SWIGLU ? fwd::BN / 2 : fwd::BN;
  const int64_t n_tiles = (ncols + bn - 1) / bn;
  return (size_t)G * n_tiles * (K / 64) * fwd::mx::PK_STAGE;
}

moe_status_t launch_pack_mx_weights(const uint8_t* q, const uint8_t* sc, int G, int N, int K, int epilogue, void* out,
                                    hipStream_t s) {
  const int ncols = epilogue == MOE_EPI_SWIGLU ? N / 2 : N;
  const int bn = epilogue == MOE_EPI_SWIGLU ? fwd::BN / 2 : fwd::BN;
  const int n_tiles = (ncols + bn - 1) / bn;
  const int64_t units = (int64_t)G * n_tiles * (K / 64) * (fwd::mx::PK_STAGE / 16);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((units + 255) / 256, (int64_t)moe_host::device_cu_count() * 16));
  if (epilogue == MOE_EPI_SWIGLU) {
    hipLaunchKernelGGL((fwd::mx::pack_mx_kernel<MOE_EPI_SWIGLU>), dim3((unsigned)blocks), dim3(256), 0, s, q, sc, G, N,
                       K, n_tiles, reinterpret_cast<uint4*>(out));
  } else {
    hipLaunchKernelGGL((fwd::mx::pack_mx_kernel<MOE_EPI_NONE>), dim3((unsigned)blocks), dim3(256), 0, s, q, sc, G, N, K,
                       n_tiles, reinterpret_cast<uint4*>(out));
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t launch_wgrad_mx(const GGArgs& a, hipStream_t s) {
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
  hipLaunchKernelGGL(fwd::mx::gg_wgrad_mx_kernel, dim3((unsigned)grid), dim3(fwd::THREADS), 0, s, b);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t launch_fwd_mx(const GGArgs& a, int epilogue, int packed, hipStream_t s) {
  GGArgs b = a;
  const bool swi = epilogue != MOE_EPI_NONE;
  const int ncols = swi ? a.N / 2 : a.N;
  const int bn = swi ? fwd::BN / 2 : fwd::BN;
  b.n_tiles = (ncols + bn - 1) / bn;
  const int64_t max_tiles = ((a.m_cap + fwd::BM - 1) / fwd::BM + a.G) * b.n_tiles;
  int64_t grid = moe_host::device_cu_count();
  if (max_tiles < grid) grid = max_tiles;
  if (grid <= 0) grid = 1;
  const dim3 g((unsigned)grid), t(fwd::THREADS);
  using namespace fwd::mx;
  if (fwd::use_split_tail(b.part != nullptr, max_tiles, grid, a.K / 64)) {
    // the split-tail instantiation (gg_pipeline.h); its counters' slot and epoch
    static std::atomic<uint64_t> launches{0};
    const uint64_t n = launches.fetch_add(1u, std::memory_order_relaxed);
    b.sched_slot = tq::launch_slot(n);
    b.sched_epoch = tq::launch_epoch(n);
    b.sched_next = tq::slot_next_epoch(n);
    if (packed) {
      if (epilogue == MOE_EPI_SWIGLU_MXFP8) {
        hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_SWIGLU_MXFP8, true, true>), g, t, 0, s, b);
      } else if (epilogue == MOE_EPI_SWIGLU) {
        hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_SWIGLU, true, true>), g, t, 0, s, b);
      } else {
        hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_NONE, true, true>), g, t, 0, s, b);
      }
    } else if (epilogue == MOE_EPI_SWIGLU_MXFP8) {
      hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_SWIGLU_MXFP8, false, true>), g, t, 0, s, b);
    } else if (epilogue == MOE_EPI_SWIGLU) {
      hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_SWIGLU, false, true>), g, t, 0, s, b);
    } else {
      hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_NONE, false, true>), g, t, 0, s, b);
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
  }
  if (packed) {
    if (epilogue == MOE_EPI_SWIGLU_MXFP8) {
      hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_SWIGLU_MXFP8, true>), g, t, 0, s, b);
    } else if (epilogue == MOE_EPI_SWIGLU) {
      hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_SWIGLU, true>), g, t, 0, s, b);
    } else {
      hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_NONE, true>), g, t, 0, s, b);
    }
  } else if (epilogue == MOE_EPI_SWIGLU_MXFP8) {
    hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_SWIGLU_MXFP8, false>), g, t, 0, s, b);
  } else if (epilogue == MOE_EPI_SWIGLU) {
    hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_SWIGLU, false>), g, t, 0, s, b);
  } else {
    hipLaunchKernelGGL((gg_fwd_mx_kernel<MOE_EPI_NONE, false>), g, t, 0, s, b);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
