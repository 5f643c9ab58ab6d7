// Grouped GEMM over ragged expert groups (bf16 and MXFP8), persistent, with
// a device-side tile scheduler.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", section "Optimization 1: Grouped GEMM": every expert's matmul in
// one kernel call, each with its true token count, computing only the
// regions with valid tokens, with no device-to-host copy of the counts
// (which would break graph capture); MXFP8 block scaling for the expert
// matmuls.  Section "What specialized optimizations are required for
// dropless MoE?": the counts may be invisible to the CPU.
//
// Design (gfx950):
//  * The grid is a function of host arguments only (CU count, m_cap, G,
//    N, K).  Each workgroup reads group_sizes once, builds the row prefix and
//    the m-tile prefix of the groups in LDS, and walks the flat tile index
//    space [0, m_tiles * n_tiles) with a grid stride, so only tiles holding
//    valid rows are ever computed; the last tile of a group masks its tail.
//  * 256 x 256 output tile, 4 wavefronts (2 x 2), 128 x 128 per wavefront as
//    8 x 8 MFMA 16x16x32 bf16 (or 16x16x128 scaled fp8) accumulators.
//  * Operands are staged through LDS in 2 stages of 64 bf16 (128 fp8) along
//    K: 128-byte rows, 16-byte slots XOR-swizzled by (row >> 1) & 7.
//    K-contiguous sources go straight from HBM/L2 to LDS with
//    global_load_lds_dwordx4; K-outer sources (the data-gradient weight, both
//    weight-gradient operands) are loaded as 8x8 blocks, transposed in
//    registers and written as 16-byte rows.
//  * The MFMA computes D[n][m] (weights as the first operand), so each lane
//    holds 4 consecutive output columns of one row: 8-byte bf16 stores; for
//    SwiGLU a wavefront owns matching gate and up columns and applies
//    silu(g) * u in registers.
//  * Workgroup ids are remapped so that consecutive tiles run on the same XCD
//    (the hardware deals workgroups round-robin over the 8 XCDs), keeping the
//    A and B panels that neighbouring tiles share in one L2.
#include "gg_common.h"

namespace moe {

constexpr int kBM = 256, kBN = 256;     // output tile (rows m, columns n)
constexpr int kWM = 2, kWN = 2;         // wavefront grid
constexpr int kThreads = kWM * kWN * 64;
constexpr int kRowBytes = 128;          // one LDS row of a stage: 64 bf16 / 128 fp8
constexpr int kWTM = kBM / kWM, kWTN = kBN / kWN;  // wavefront tile
constexpr int kTM = kWTM / 16, kTN = kWTN / 16;    // MFMA subtiles per wavefront
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }

// ----------------------------------------------------------------- loaders
// K-contiguous rows straight into LDS.  Stage row r holds global row grow(r);
// 16-byte slot (r, s) holds chunk swz(r, s) of it.  Each lane issues R/8/NW
// loads; their 32-bit byte offsets (row * ld + chunk * 16) are computed once
// per tile, and every stage adds only a uniform base pointer.
template <int R>
struct DirectRows {
  static constexpr int NW = kThreads / 64;
  static constexpr int N = R / 8 / NW;
  uint32_t off[N];
  template <typename RowFn>
  __device__ __forceinline__ void init(int64_t ld_bytes, RowFn grow) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
    // swz(row, lane & 7) with row = (i*NW + wave)*8 + lane/8: (row >> 1) & 7 =
    // ((wave & 1) << 2) | (lane >> 4) for every i (NW even)
    static_assert(NW % 2 == 0, "swizzle shortcut needs an even wavefront count");
    const int chunk = (lane & 7) ^ (((wave & 1) << 2) | (lane >> 4));
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int row = (i * NW + wave) * 8 + (lane >> 3);
      off[i] = (uint32_t)(grow(row) * ld_bytes + chunk * 16);
    }
  }
  __device__ __forceinline__ void issue(uint8_t* lds, const uint8_t* base) const {
    const int wave = wave_id();
#pragma unroll
    for (int i = 0; i < N; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(base + off[i]), (lds_ptr_t)(lds + (i * NW + wave) * 1024), 16,
                                       0, 0);
  }
};

// Per-row 4-byte scale words (MXFP8: 4 blocks of 32 for a 128-wide stage).
template <int R>
struct DirectScales {
  static constexpr int NW = kThreads / 64;
  static constexpr int N = R / 64 / NW;
  uint32_t off[N];
  template <typename RowFn>
  __device__ __forceinline__ void init(int64_t ld, RowFn grow) {
    const int wave = wave_id(), lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < N; ++i) off[i] = (uint32_t)(grow((i * NW + wave) * 64 + lane) * ld);
  }
  __device__ __forceinline__ void issue(uint8_t* lds, const uint8_t* base) const {
    const int wave = wave_id();
#pragma unroll
    for (int i = 0; i < N; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(base + off[i]), (lds_ptr_t)(lds + (i * NW + wave) * 256), 4, 0,
                                       0);
  }
};

// K-outer source: element (k, c) at g[k * ld + c] (bf16).  Tile row r = column
// c0 + r; stage k-range [k0, k0 + 64) with rows k >= k_end read as zero and
// columns clamped to [0, ncols).  Each thread moves R / 256 blocks of 8 x 8.
template <int R>
struct KOuterLoad {
  uint4 v[R / kThreads][8];
  __device__ __forceinline__ void issue(const uint16_t* g, int64_t ld, int64_t k0, int64_t k_end, int c0, int ncols) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < R / kThreads; ++i) {
      const int b = t + i * kThreads;
      const int nb = b % (R / 8), kb = b / (R / 8);
      int c = c0 + nb * 8;
      if (c > ncols - 8) c = ncols - 8;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t k = k0 + kb * 8 + q;
        v[i][q] = (k < k_end) ? *reinterpret_cast<const uint4*>(g + k * ld + c) : make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(uint8_t* lds) {
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < R / kThreads; ++i) {
      const int b = t + i * kThreads;
      const int nb = b % (R / 8), kb = b / (R / 8);
      const uint32_t* w = reinterpret_cast<const uint32_t*>(v[i]);  // w[q*4 + p]: row k=q, cols 2p, 2p+1
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t o[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t lo = w[(2 * p) * 4 + (j >> 1)], hi = w[(2 * p + 1) * 4 + (j >> 1)];
          o[p] = (j & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
        }
        const int row = nb * 8 + j;
        *reinterpret_cast<uint4*>(lds + row * kRowBytes + swz(row, kb) * 16) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
};

// ----------------------------------------------------------------- compute
template <bool MX>
struct Frag;

template <>
struct Frag<false> {
  typedef bf16x8_t T;
};
template <>
struct Frag<true> {
  typedef i32x8_t T;
};

// A fragment row of a stage: tile rows base + 16*i share the swizzle of
// base (16*i only moves (row >> 1) & 7 by multiples of 8), so a lane's slot is
// fixed for a whole stage: slot = chunk ^ ((r16 >> 1) & 7) for wavefront
// tiles aligned to 16 rows.
__device__ __forceinline__ uint4 lds_read16(const uint8_t* lds, int row, int slot) {
  return *reinterpret_cast<const uint4*>(lds + row * kRowBytes + slot * 16);
}

// One stage: W tile rows [0, kBN) at lw, X tile rows [0, kBM) at lx.
template <bool MX>
__device__ __forceinline__ void compute_stage(const uint8_t* lw, const uint8_t* lx, const uint8_t* sw,
                                              const uint8_t* sx, f32x4_t (&acc)[kTN][kTM]) {
  const int wave = wave_id(), lane = threadIdx.x & 63;
  const int wn = wave / kWM, wm = wave % kWM;
  const int r16 = lane & 15, g4 = lane >> 4;
  const int slot0 = g4 ^ ((r16 >> 1) & 7);  // chunk g4 (bf16 k-step 0 / fp8 low half)
  const int wrow0 = wn * kWTN + r16, xrow0 = wm * kWTM + r16;
  if constexpr (!MX) {
#pragma unroll 1
    for (int s = 0; s < 2; ++s) {
      const int slot = slot0 ^ (s << 2);  // chunk s*4 + g4
      bf16x8_t wf[kTN], xf[kTM];
#pragma unroll
      for (int i = 0; i < kTN; ++i) wf[i] = __builtin_bit_cast(bf16x8_t, lds_read16(lw, wrow0 + i * 16, slot));
#pragma unroll
      for (int j = 0; j < kTM; ++j) xf[j] = __builtin_bit_cast(bf16x8_t, lds_read16(lx, xrow0 + j * 16, slot));
#pragma unroll
      for (int i = 0; i < kTN; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[i], xf[j], acc[i][j], 0, 0, 0);
    }
  } else {
    i32x8_t wf[kTN], xf[kTM];
    int wsc[kTN], xsc[kTM];
#pragma unroll
    for (int i = 0; i < kTN; ++i) {
      const int row = wrow0 + i * 16;
      const uint4 lo = lds_read16(lw, row, slot0), hi = lds_read16(lw, row, slot0 ^ 4);
      wf[i] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      wsc[i] = sw[row * 4 + g4];
    }
#pragma unroll
    for (int j = 0; j < kTM; ++j) {
      const int row = xrow0 + j * 16;
      const uint4 lo = lds_read16(lx, row, slot0), hi = lds_read16(lx, row, slot0 ^ 4);
      xf[j] = i32x8_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      xsc[j] = sx[row * 4 + g4];
    }
#pragma unroll
    for (int i = 0; i < kTN; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[i], xf[j], acc[i][j], 0, 0, 0, wsc[i], 0, xsc[j]);
  }
}

// ----------------------------------------------------------------- epilogue
// Writes the wavefront's accumulators.  Plain: column n0 + wn*kWTN + 16i + 4*g4.
// SwiGLU: subtiles i < kTN/2 are gate columns j = n0 + wn*kWTN/2 + 16i + 4*g4
// and subtiles i + kTN/2 the up columns of the same j; the pre-activations go
// to Caux first, then h = silu(g) * u is formed in place and stored.
template <int EPI, int OUT>
__device__ __forceinline__ void store_tile(const GGArgs& a, f32x4_t (&acc)[kTN][kTM], int64_t m0, int rows, int n0,
                                           int ncols, int64_t ldc, uint8_t* C, int f) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave / kWM, wm = wave % kWM;
  const int r16 = lane & 15, g4 = lane >> 4;
  if constexpr (EPI == MOE_EPI_SWIGLU) {
    const int jbase = n0 + wn * (kWTN / 2) + g4 * 4;
    if (a.Caux) {
      uint8_t* aux = a.Caux;
      const int64_t lda = 2 * (int64_t)f;
#pragma unroll
      for (int j = 0; j < kTM; ++j) {
        const int mr = wm * kWTM + j * 16 + r16;
#pragma unroll
        for (int i = 0; i < kTN / 2; ++i) {
          const int jc = jbase + i * 16;
          if (mr < rows && jc < f) {
            store_sub<MOE_OUT_BF16>(aux, lda, m0 + mr, jc, acc[i][j]);
            store_sub<MOE_OUT_BF16>(aux, lda, m0 + mr, f + jc, acc[i + kTN / 2][j]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kTN / 2; ++i)
#pragma unroll
      for (int j = 0; j < kTM; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][j][q] = silu_f32(acc[i][j][q]) * acc[i + kTN / 2][j][q];
#pragma unroll
    for (int j = 0; j < kTM; ++j) {
      const int mr = wm * kWTM + j * 16 + r16;
#pragma unroll
      for (int i = 0; i < kTN / 2; ++i) {
        const int jc = jbase + i * 16;
        if (mr < rows && jc < f) store_sub<MOE_OUT_BF16>(C, ldc, m0 + mr, jc, acc[i][j]);
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < kTM; ++j) {
      const int mr = wm * kWTM + j * 16 + r16;
#pragma unroll
      for (int i = 0; i < kTN; ++i) {
        const int n = n0 + wn * kWTN + i * 16 + g4 * 4;
        if (mr < rows && n < ncols) store_sub<OUT>(C, ldc, m0 + mr, n, acc[i][j]);
      }
    }
  }
}

template <int MODE, bool MX, int EPI, int OUT>
__global__ void __launch_bounds__(kThreads, 1) grouped_gemm_kernel(GGArgs a) {
  // Two named stage buffers: a stage reads one while the direct-to-LDS loads
  // of the next fill the other.  Distinct objects let the compiler see that
  // the in-flight LDS-DMA writes cannot alias the fragment reads, so it does
  // not wait for them before reading the current stage.
  __shared__ __align__(1024) uint8_t buf0[kStageBytes];
  __shared__ __align__(1024) uint8_t buf1[kStageBytes];
  __shared__ __align__(16) uint8_t sc0[MX ? (kBN + kBM) * 4 : 16];   // MXFP8: W scales [kBN][4], X scales [kBM][4]
  __shared__ __align__(16) uint8_t sc1[MX ? (kBN + kBM) * 4 : 16];
  __shared__ GroupInfo<kThreads> gi;

  build_groups<kThreads, kBM, MODE != MODE_K>(a, gi);

  const int wid = worker_id();
  const int f = a.N / 2;  // SwiGLU width

  if constexpr (MODE != MODE_K) {
    const int64_t total = (int64_t)gi.tpre[a.G] * a.n_tiles;
    const int elt = MX ? 1 : 2;
    const int64_t lda_b = (int64_t)a.K * elt;
    const int nk = a.K / (MX ? 128 : 64);
    for (int64_t tile = wid; tile < total; tile += gridDim.x) {
      const int mt = (int)(tile / a.n_tiles), nt = (int)(tile % a.n_tiles);
      const int g = find_group(gi.tpre, a.G, mt);
      const int64_t m0 = gi.roff[g] + (int64_t)(mt - gi.tpre[g]) * kBM;
      const int rows = (int)min<int64_t>(kBM, gi.roff[g + 1] - m0);
      const int n0 = (EPI == MOE_EPI_SWIGLU) ? nt * (kBN / 2) : nt * kBN;
      const int nrows_b = (EPI == MOE_EPI_SWIGLU) ? 2 * f : a.N;

      // rows relative to per-tile uniform bases (offsets stay 32-bit)
      auto xrow = [&](int r) -> int64_t { return min(r, rows - 1); };
      auto wrow = [&](int r) -> int64_t {
        if constexpr (EPI == MOE_EPI_SWIGLU) {
          const int wn = r / kWTN, q = r % kWTN;
          int jj = n0 + wn * (kWTN / 2) + (q % (kWTN / 2));
          jj = min(jj, f - 1);
          return q < kWTN / 2 ? jj : f + jj;
        } else {
          return min(n0 + r, a.N - 1);
        }
      };
      const uint8_t* xbase = a.A + m0 * lda_b;
      const uint8_t* wbase = a.B + (int64_t)g * nrows_b * lda_b;
      const uint8_t* xsbase = MX ? a.As + m0 * (a.K / 32) : nullptr;
      const uint8_t* wsbase = MX ? a.Bs + (int64_t)g * nrows_b * (a.K / 32) : nullptr;
      DirectRows<kBM> xl;
      DirectRows<kBN> wd;
      DirectScales<kBM> xs;
      DirectScales<kBN> ws;
      xl.init(lda_b, xrow);
      if constexpr (MODE == MODE_M_NK) wd.init(lda_b, wrow);
      if constexpr (MX) {
        xs.init(a.K / 32, xrow);
        ws.init(a.K / 32, wrow);
      }
      const uint16_t* Bkn = reinterpret_cast<const uint16_t*>(a.B) + (int64_t)g * a.K * a.N;
      KOuterLoad<kBN> wl;

      f32x4_t acc[kTN][kTM];
#pragma unroll
      for (int i = 0; i < kTN; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

      // issue the loads of stage kt into (buf, sc); the K-outer weight goes to registers
      auto load_stage = [&](uint8_t* buf, uint8_t* sc, int kt) {
        const int kb = kt * kRowBytes;
        xl.issue(buf + kBN * kRowBytes, xbase + kb);
        if constexpr (MODE == MODE_M_NK) {
          wd.issue(buf, wbase + kb);
        } else {
          wl.issue(Bkn, a.N, (int64_t)kt * 64, a.K, n0, a.N);
        }
        if constexpr (MX) {
          xs.issue(sc + kBN * 4, xsbase + kt * 4);
          ws.issue(sc, wsbase + kt * 4);
        }
      };
      // one stage: wait for (cur) to land, start (nxt) = stage kt + 1, compute (cur)
      auto body = [&](uint8_t* cur, uint8_t* sccur, uint8_t* nxt, uint8_t* scnxt, int kt) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const bool more = kt + 1 < nk;
        if (more) load_stage(nxt, scnxt, kt + 1);
        compute_stage<MX>(cur, cur + kBN * kRowBytes, sccur, sccur + kBN * 4, acc);
        if constexpr (MODE == MODE_M_KN) {
          if (more) wl.store(nxt);
        }
      };

      __syncthreads();  // the previous tile's last stage has been read by everyone
      load_stage(buf0, sc0, 0);
      if constexpr (MODE == MODE_M_KN) wl.store(buf0);
      for (int kt = 0; kt < nk; kt += 2) {
        body(buf0, sc0, buf1, sc1, kt);
        if (kt + 1 < nk) body(buf1, sc1, buf0, sc0, kt + 1);
      }
      store_tile<EPI, OUT>(a, acc, m0, rows, n0, EPI == MOE_EPI_SWIGLU ? f : a.N,
                           EPI == MOE_EPI_SWIGLU ? f : a.N, a.C, f);
    }
  } else {
    // ragged-K: C[g] [M, N] = sum over the group's rows r of A[r, p] * B[r, q]
    const int per_group = a.p_tiles * a.n_tiles;
    const int64_t total = (int64_t)a.G * per_group;
    const uint16_t* A16 = reinterpret_cast<const uint16_t*>(a.A);
    const uint16_t* B16 = reinterpret_cast<const uint16_t*>(a.B);
    for (int64_t tile = wid; tile < total; tile += gridDim.x) {
      const int rank = (int)(tile / per_group), rem = (int)(tile % per_group);
      const int g = gi.tpre[rank];
      const int pt = rem / a.n_tiles, qt = rem % a.n_tiles;
      const int p0 = pt * kBM, q0 = qt * kBN;
      const int64_t r0 = gi.roff[g], r1 = gi.roff[g + 1];
      const int nk = (int)((r1 - r0 + 63) / 64);
      KOuterLoad<kBM> xl;
      KOuterLoad<kBN> wl;
      f32x4_t acc[kTN][kTM];
#pragma unroll
      for (int i = 0; i < kTN; ++i)
#pragma unroll
        for (int j = 0; j < kTM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      auto body = [&](uint8_t* cur, uint8_t* nxt, int kt) {
        __syncthreads();
        const bool more = kt + 1 < nk;
        if (more) {
          xl.issue(A16, a.M, r0 + (int64_t)(kt + 1) * 64, r1, p0, a.M);
          wl.issue(B16, a.N, r0 + (int64_t)(kt + 1) * 64, r1, q0, a.N);
        }
        compute_stage<false>(cur, cur + kBN * kRowBytes, nullptr, nullptr, acc);
        if (more) {
          xl.store(nxt + kBN * kRowBytes);
          wl.store(nxt);
        }
      };
      __syncthreads();
      if (nk > 0) {
        xl.issue(A16, a.M, r0, r1, p0, a.M);
        wl.issue(B16, a.N, r0, r1, q0, a.N);
        xl.store(buf0 + kBN * kRowBytes);
        wl.store(buf0);
      }
      for (int kt = 0; kt < nk; kt += 2) {
        body(buf0, buf1, kt);
        if (kt + 1 < nk) body(buf1, buf0, kt + 1);
      }
      uint8_t* Cg = a.C + (int64_t)g * a.M * a.N * (OUT == MOE_OUT_F32 ? 4 : 2);
      store_tile<MOE_EPI_NONE, OUT>(a, acc, p0, min(kBM, a.M - p0), q0, a.N, a.N, Cg, 0);
    }
  }
}

template <int MODE, bool MX, int EPI, int OUT>
static moe_status_t launch(const GGArgs& a, hipStream_t s, int64_t max_tiles) {
  int64_t grid = moe_host::device_cu_count();
  if (max_tiles < grid) grid = max_tiles;
  if (grid <= 0) grid = 1;
  hipLaunchKernelGGL((grouped_gemm_kernel<MODE, MX, EPI, OUT>), dim3((unsigned)grid), dim3(kThreads), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t launch_fwd(const GGArgs& a, int epilogue, int out_f32, int b_layout, hipStream_t s);  // gg_fwd.hip
moe_status_t launch_fwd_mx(const GGArgs& a, int epilogue, int packed, hipStream_t s);  // gg_fwd_mx.hip

}  // namespace moe

extern "C" moe_status_t grouped_gemm_launch(const moe_gg_desc* d, const void* A, const uint8_t* As, const void* B,
                                            const uint8_t* Bs, const int32_t* sizes, void* C, void* Caux,
                                            uint32_t* flag, hipStream_t s) {
  using namespace moe;
  GGArgs a;
  a.A = reinterpret_cast<const uint8_t*>(A);
  a.B = reinterpret_cast<const uint8_t*>(B);
  a.As = As;
  a.Bs = Bs;
  a.sizes = sizes;
  a.C = reinterpret_cast<uint8_t*>(C);
  a.Caux = reinterpret_cast<uint8_t*>(Caux);
  a.flag = flag;
  a.m_cap = d->m_cap;
  a.G = d->G;
  a.M = d->M;
  a.N = d->N;
  a.K = d->K;
  if (d->ragged == MOE_RAGGED_M) {
    const int ncols = d->epilogue == MOE_EPI_SWIGLU ? d->N / 2 : d->N;
    const int bn = d->epilogue == MOE_EPI_SWIGLU ? kBN / 2 : kBN;
    a.n_tiles = (ncols + bn - 1) / bn;
    a.p_tiles = 0;
    const int64_t max_m_tiles = (d->m_cap + kBM - 1) / kBM + d->G;
    const int64_t max_tiles = max_m_tiles * a.n_tiles;
    if (d->dtype == MOE_DTYPE_MXFP8) return launch_fwd_mx(a, d->epilogue, d->b_layout == MOE_B_PACKED, s);
    (void)max_tiles;
    return launch_fwd(a, d->epilogue, d->out_dtype == MOE_OUT_F32, d->b_layout, s);
  }
  a.n_tiles = (d->N + kBN - 1) / kBN;
  a.p_tiles = (d->M + kBM - 1) / kBM;
  const int64_t max_tiles = (int64_t)d->G * a.n_tiles * a.p_tiles;
  if (d->out_dtype == MOE_OUT_F32) return launch<MODE_K, false, MOE_EPI_NONE, MOE_OUT_F32>(a, s, max_tiles);
  return launch<MODE_K, false, MOE_EPI_NONE, MOE_OUT_BF16>(a, s, max_tiles);
}
