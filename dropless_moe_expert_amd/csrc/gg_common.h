// Shared pieces of the grouped-GEMM kernels: arguments, the device-side
// group prefix (the tile scheduler's input), tile-order helpers, stores.
#pragma once
#include "common.h"

namespace moe {

constexpr int kMaxGroups = 1024;
enum { MODE_M_NK = 0, MODE_M_KN = 1, MODE_K = 2 };

struct GGArgs {
  const uint8_t* A;        // activations (bytes)
  const uint8_t* B;        // weights / second operand (bytes)
  const uint8_t* As;       // MXFP8 scales of A
  const uint8_t* Bs;       // MXFP8 scales of B
  const int32_t* sizes;    // device group sizes
  uint8_t* C;
  uint8_t* Caux;
  uint32_t* flag;
  int64_t m_cap;
  int G, M, N, K;
  int n_tiles;             // tiles along n (ragged-M) / q (ragged-K)
  int p_tiles;             // ragged-K: tiles along p (rows of C[g])
  int sched_slot;          // ragged-K: the launch's slot of tile-queue counters
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// wavefront index as a scalar (uniform) value
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ----------------------------------------------------------------- group prefix
template <int THREADS>
struct GroupInfo {
  int32_t roff[kMaxGroups + 1];   // row offsets: sizes clamped to >= 0, offsets to m_cap
  int32_t tpre[kMaxGroups];       // groups ranked by size, largest first
  int64_t scan[THREADS];
};

// exclusive scan of v over the workgroup (THREADS values), total in *tot
template <int THREADS>
__device__ __forceinline__ int64_t block_scan(int64_t v, int64_t* buf, int64_t* tot) {
  const int t = threadIdx.x;
  buf[t] = v;
  __syncthreads();
  for (int o = 1; o < THREADS; o <<= 1) {
    int64_t add = (t >= o) ? buf[t - o] : 0;
    __syncthreads();
    buf[t] += add;
    __syncthreads();
  }
  int64_t incl = buf[t];
  *tot = buf[THREADS - 1];
  __syncthreads();
  return incl - v;
}

// Row offsets of the ragged-K groups from the device sizes: each size
// clamped to >= 0, the running sum taken in 64 bits (1024 sizes of up to
// 2^31 - 1 each cannot wrap it) and every offset clamped to m_cap, so no
// group reaches outside the operands; then the groups ranked largest first
// (ties: lower index first), so the longest contractions start earliest.
// Raises the data-error flags from block 0.
template <int THREADS>
__device__ void build_groups(const GGArgs& a, GroupInfo<THREADS>& gi) {
  const int t = threadIdx.x;
  constexpr int per = kMaxGroups / THREADS;
  int64_t s[per];
  int64_t local = 0;
  bool neg = false;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    int g = t * per + i;
    int64_t v = (g < a.G) ? (int64_t)a.sizes[g] : 0;
    if (v < 0) { neg = true; v = 0; }
    s[i] = v;
    local += v;
  }
  int64_t tot;
  const int64_t base = block_scan<THREADS>(local, gi.scan, &tot);
  const int64_t cap = a.m_cap;
  int64_t o = base;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    int g = t * per + i;
    if (g <= a.G) gi.roff[g] = (int32_t)min<int64_t>(o, cap);
    o += s[i];
  }
  if (t == THREADS - 1 && a.G == kMaxGroups) gi.roff[kMaxGroups] = (int32_t)min<int64_t>(o, cap);
  if (blockIdx.x == 0 && t == 0 && tot > cap) raise_flag(a.flag, MOE_FLAG_ROWS_OVER_CAP);
  if (blockIdx.x == 0 && __any(neg) && (t & 63) == 0) raise_flag(a.flag, MOE_FLAG_NEGATIVE_SIZE);
  __syncthreads();
  for (int g = t; g < a.G; g += THREADS) {
    const int32_t sg = gi.roff[g + 1] - gi.roff[g];
    int rank = 0;
    for (int h = 0; h < a.G; ++h) {
      const int32_t sh = gi.roff[h + 1] - gi.roff[h];
      rank += (sh > sg) || (sh == sg && h < g);
    }
    gi.tpre[rank] = g;
  }
  __syncthreads();
}

__device__ __forceinline__ int worker_id() {
  // consecutive worker ids share an XCD (blocks are dealt round-robin to 8 XCDs)
  const int nb = gridDim.x;
  if (nb % 8) return blockIdx.x;
  return (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8;
}

// ----------------------------------------------------------------- kernel

// s_waitcnt that waits only for vector-memory count <= n (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4] = 7, lgkmcnt [11:8] = 15 = no wait)
#define MOE_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

template <int OUT>
__device__ __forceinline__ void store_sub(uint8_t* C, int64_t ldc, int64_t m, int n, const f32x4_t& v) {
  if constexpr (OUT == MOE_OUT_F32) {
    *reinterpret_cast<float4*>(C + (m * ldc + n) * 4) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    *reinterpret_cast<uint2*>(C + (m * ldc + n) * 2) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
}

}  // namespace moe
