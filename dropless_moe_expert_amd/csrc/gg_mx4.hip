// MXFP4 grouped GEMM, forward (ragged M): E2M1 codes with an E8M0 scale per
// 32 along K for both operands, fp32 accumulation, bf16 output, optionally
// the SwiGLU epilogue.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", section "Optimization 1: Grouped GEMM" (all experts in one call,
// each with its true token count, counts on the device) and its closing plan
// of a 4-bit format (NVFP4 there; on gfx950 the MX 4-bit format E2M1 runs on
// the same scaled MFMA as MXFP8).
//
// Operand layout (the boundary's MXFP4 tensors): codes row-major, two per
// byte, element 2i in the low nibble of byte i; scales stage-major,
// [K/128][rows][4]: the four scale bytes of a row's 128-code stage are one
// word, and one stage of a tile's rows is one contiguous block.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with both formats E2M1 (cbsz = blgp = 4)
// reads 4 registers per operand: lane l holds row l % 32 and codes
// k = 32g .. 32g + 31 (g = l / 32) of the 64-code step, and gives the scale
// of (row l % 32, 32-block g) (layout measured on the hardware against a CPU
// model with a different scale per block).
//
// Tiles of 256 token rows x 256 weight rows walk the group offsets on the
// device exactly as the other forward kernels (locate, XCD-aware worker
// ids).  Eight wavefronts, 2 (m) x 4 (n), each own 128 x 64 of the tile as
// 4 x 2 MFMA subtiles.  A stage holds 128 codes of every tile row (64-byte
// LDS rows, direct-to-LDS loads, slot swizzle (row >> 2) & 3) and the rows'
// scale words; four stages are in flight, loads issued three ahead, one
// barrier per stage.  SwiGLU reads the unpacked [gate; up] weight: tile row r
// of wavefront column wn maps to gate row 32 wn + r (r < 32) or the up row of
// the same column, so each wavefront holds both halves of its 32 outputs.
#include "gg_pipeline.h"

namespace moe {
namespace fwd {
namespace mx4 {

constexpr int NWAVE = 8, THREADS = NWAVE * 64;
constexpr int WM = 2, WN = 4;                 // wavefront grid (m, n)
constexpr int WTM = BM / WM, WTN = BN / WN;   // 128 x 64 per wavefront
constexpr int MTM = WTM / 32, MTN = WTN / 32; // 4 x 2 subtiles of 32 x 32
constexpr int CODES_B = (BM + BN) * 64;       // 32 KB of codes per stage
constexpr int STAGE_B = CODES_B + (BM + BN) * 4;   // + one scale word per row
constexpr int NS = 4;
constexpr int NB = (BM + BN) / 16 / NWAVE + 1;      // loads per wavefront and stage (4 code rows + 1 scale)

__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }

template <int NBV>
__device__ __forceinline__ void wait_stages(int q) {
  if (q <= 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  else if (q == 1) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NBV) : "memory");
  else asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NBV) : "memory");
}

__device__ __forceinline__ i32x8_t frag(const uint8_t* p) {
  const uint4 v = *reinterpret_cast<const uint4*>(p);
  return i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
}

template <int EPI>
__global__ void __launch_bounds__(THREADS, 1) gg_fwd_mx4_kernel(GGArgs a) {
  __shared__ __align__(1024) uint8_t lds[NS * STAGE_B];

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

  constexpr bool SWI = EPI == MOE_EPI_SWIGLU;
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int wm = wave % WM, wn = wave / WM;
  const int r32 = lane & 31, g = lane >> 5;
  const int wid = worker_id();
  const int f = a.N / 2;
  const int64_t total = count_mtiles(a) * a.n_tiles;
  const int64_t ldb = a.K / 2;              // code bytes per row
  const int nst = a.K / 128;
  const int64_t GN = (int64_t)a.G * a.N;    // weight rows (scale rows of B)
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_ptr_t)lds;

  for (int64_t tile = wid; tile < total; tile += gridDim.x) {
    const TileGroup tg = locate(a, tile);
    const int ge = tg.g, nt = tg.nt;
    const int64_t m0 = tg.m0;
    const int rows = tg.rows;
    const int n0 = SWI ? nt * (BN / 2) : nt * BN;   // first output column of the tile

    // tile row -> row of the expert's weight [N, K]
    auto wrow = [&](int r) -> int64_t {
      if constexpr (SWI) {
        const int q = r % WTN, jj = min(n0 + (r / WTN) * (WTN / 2) + (q % (WTN / 2)), f - 1);
        return q < WTN / 2 ? jj : f + jj;
      } else {
        return min(n0 + r, a.N - 1);
      }
    };
    auto xrow = [&](int r) -> int64_t { return min(r, rows - 1); };
    Rows<BM, NWAVE, 1> xl;
    Rows<BN, NWAVE, 1> wl;
    xl.init(ldb, xrow);
    wl.init(ldb, wrow);
    // scale words: wavefronts 0-3 load the x rows 64 w .. 64 w + 63, 4-7 the weight rows
    const int srow = 64 * (wave & 3) + lane;
    const uint32_t soff = (uint32_t)((wave < 4 ? xrow(srow) : wrow(srow)) * 4);
    const uint8_t* xcb = a.A + m0 * ldb;
    const uint8_t* wcb = a.B + (int64_t)ge * a.N * ldb;
    const uint8_t* xsb = a.As + m0 * 4;
    const uint8_t* wsb = a.Bs + (int64_t)ge * a.N * 4;

    auto issue = [&](int st) {
      uint8_t* sb = lds + (st % NS) * STAGE_B;
      xl.issue(sb, xcb + st * 64);
      wl.issue(sb + BM * 64, wcb + st * 64);
      const uint8_t* base = wave < 4 ? xsb + (int64_t)st * a.m_cap * 4 : wsb + (int64_t)st * GN * 4;
      const uint32_t m0l = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((st % NS) * STAGE_B + CODES_B + wave * 256));
      asm volatile(
          "s_mov_b32 m0, %0\n\t"
          "s_nop 0\n\t"
          "global_load_lds_dword %1, %2"
          :
          : "s"(m0l), "v"(soff), "s"(base)
          : "memory", "m0");
    };

    f32x16_t acc[MTN][MTM];
#pragma unroll
    for (int i = 0; i < MTN; ++i)
#pragma unroll
      for (int j = 0; j < MTM; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    __syncthreads();   // the previous tile's last stage reads are done
    for (int st = 0; st < NS - 1 && st < nst; ++st) issue(st);
    for (int st = 0; st < nst; ++st) {
      wait_stages<NB>(min(nst - 1, st + NS - 2) - st);
      asm volatile("s_barrier" ::: "memory");
      if (st + NS - 1 < nst) issue(st + NS - 1);
      const uint8_t* sb = lds + (st % NS) * STAGE_B;
      uint32_t xs[MTM], ws[MTN];
#pragma unroll
      for (int j = 0; j < MTM; ++j)
        xs[j] = *reinterpret_cast<const uint32_t*>(sb + CODES_B + (wm * WTM + 32 * j + r32) * 4);
#pragma unroll
      for (int i = 0; i < MTN; ++i)
        ws[i] = *reinterpret_cast<const uint32_t*>(sb + CODES_B + (BM + wn * WTN + 32 * i + r32) * 4);
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int c = 2 * s + g;   // 16-byte chunk = 32-code block of this lane
        i32x8_t xf[MTM], wf[MTN];
#pragma unroll
        for (int j = 0; j < MTM; ++j) {
          const int row = wm * WTM + 32 * j + r32;
          xf[j] = frag(sb + row * 64 + ((c ^ swz(row)) << 4));
        }
#pragma unroll
        for (int i = 0; i < MTN; ++i) {
          const int row = BM + wn * WTN + 32 * i + r32;
          wf[i] = frag(sb + row * 64 + ((c ^ swz(row)) << 4));
        }
#pragma unroll
        for (int i = 0; i < MTN; ++i)
#pragma unroll
          for (int j = 0; j < MTM; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                wf[i], xf[j], acc[i][j], 4, 4, 0, (int)((ws[i] >> (8 * c)) & 0xFFu), 0,
                (int)((xs[j] >> (8 * c)) & 0xFFu));
      }
    }

    // 32x32 accumulator: element v of lane (r32, g) is weight row 8 (v / 4) + 4 g + v % 4
    // of subtile i and token row r32 of subtile j.  The bf16 tile leaves
    // through LDS: every wavefront writes its rows (16-byte units XOR-
    // swizzled by row), then the workgroup copies whole rows out as 16-byte
    // pieces, each thread's LDS reads four at a time ahead of their stores.
    constexpr int RB = SWI ? 256 : 512, UR = RB / 16;   // bytes and 16-byte units per tile row
    static_assert(BM * RB <= NS * STAGE_B, "the tile fits in the stage buffers");
    auto put = [&](int row, int col, uint2 w) {
      *reinterpret_cast<uint2*>(lds + row * RB + (((col >> 3) ^ (row % UR)) << 4) + ((col >> 2) & 1) * 8) = w;
    };
    __syncthreads();   // every wavefront has read its last stage
#pragma unroll
    for (int j = 0; j < MTM; ++j) {
      const int mr = wm * WTM + 32 * j + r32;
      if constexpr (SWI) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float h[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = silu_f32(acc[0][j][q * 4 + e]) * acc[1][j][q * 4 + e];
          put(mr, wn * (WTN / 2) + q * 8 + g * 4, make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3])));
        }
      } else {
#pragma unroll
        for (int i = 0; i < MTN; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            put(mr, wn * WTN + 32 * i + q * 8 + g * 4,
                make_uint2(pack_bf16x2(acc[i][j][q * 4], acc[i][j][q * 4 + 1]),
                           pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3])));
      }
    }
    __syncthreads();
    {
      constexpr int NPT = BM * UR / THREADS;   // 16-byte pieces per thread
      constexpr int NBT = 4;
      static_assert(BM * UR % THREADS == 0 && NPT % NBT == 0, "whole batches");
      const int ld = SWI ? f : a.N;
      // a piece is a 32-bit offset from the tile's first row (256 rows of at
      // most 2^22 columns)
      uint8_t* const cbase = a.C + m0 * (int64_t)ld * 2;
#pragma unroll 1
      for (int k0 = 0; k0 < NPT; k0 += NBT) {
        uint4 v[NBT];
#pragma unroll
        for (int k = 0; k < NBT; ++k) {
          const int c = threadIdx.x + (k0 + k) * THREADS;
          const int row = c / UR, u = c - row * UR;
          v[k] = *reinterpret_cast<const uint4*>(lds + row * RB + ((u ^ (row % UR)) << 4));
        }
#pragma unroll
        for (int k = 0; k < NBT; ++k) {
          const int c = threadIdx.x + (k0 + k) * THREADS;
          const int row = c / UR, u = c - row * UR;
          const int col = n0 + 8 * u;
          if (row < rows && col < ld) *reinterpret_cast<uint4*>(cbase + (uint32_t)(row * ld + col) * 2u) = v[k];
        }
      }
    }
  }
}

}  // namespace mx4
}  // namespace fwd

moe_status_t launch_fwd_mx4(const GGArgs& a, int epilogue, hipStream_t s) {
  GGArgs b = a;
  const bool swi = epilogue == MOE_EPI_SWIGLU;
  const int ncols = swi ? a.N / 2 : a.N;
  const int bn = swi ? fwd::BN / 2 : fwd::BN;
  b.n_tiles = (ncols + bn - 1) / bn;
  const int64_t max_tiles = ((a.m_cap + fwd::BM - 1) / fwd::BM + a.G) * b.n_tiles;
  int64_t grid = moe_host::device_cu_count();
  if (max_tiles < grid) grid = max_tiles;
  if (grid <= 0) grid = 1;
  if (swi) {
    hipLaunchKernelGGL((fwd::mx4::gg_fwd_mx4_kernel<MOE_EPI_SWIGLU>), dim3((unsigned)grid), dim3(fwd::mx4::THREADS), 0,
                       s, b);
  } else {
    hipLaunchKernelGGL((fwd::mx4::gg_fwd_mx4_kernel<MOE_EPI_NONE>), dim3((unsigned)grid), dim3(fwd::mx4::THREADS), 0,
                       s, b);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

}  // namespace moe
