// Shared pieces of the grouped-GEMM kernels: arguments, the device-side
// group prefix (the tile scheduler's input), tile-order helpers, stores.
#pragma once
#include "common.h"
#include "tile_queue.h"

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
  int sched_slot;          // the launch's slot of tile-queue (ragged-K) or split (ragged-M) words
  uint32_t sched_epoch;    // the launch's epoch (tile_queue.h)
  uint32_t sched_next;     // the epoch of the slot's next launch
  float* part;             // ragged-M bf16: workspace of the split tail's partial sums, or NULL
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// wavefront index as a scalar (uniform) value
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// ----------------------------------------------------------------- tile queues
// One tile-queue word in device memory, for tq::take / tq::finish.
struct DeviceWord {
  uint32_t* p;
  __device__ uint32_t add1() { return atomicAdd(p, 1u); }
  __device__ uint32_t cas(uint32_t expected, uint32_t desired) { return atomicCAS(p, expected, desired); }
};

// One workgroup's walk over a launch's tile queues (per_group tiles per
// group, G groups dealt to the queues in a snake over the size ranks: queue
// q holds ranks k nq + q for even k and k nq + nq - 1 - q for odd k, so
// every queue gets a share of large and small groups).  Its own queue
// blockIdx % nq first - blocks are dealt round-robin to the 8 XCDs, so a
// queue's tiles share one XCD's L2 - and then the others, so no workgroup
// idles while tiles remain.  process(rank, tile) runs with the whole
// workgroup.  Thread 0 takes; the two s_tile entries alternate, so one is
// rewritten only after the barrier that follows every thread's read of it.
// Thread 0 of the last workgroup to finish presets the slot for its next
// launch (tile_queue.h).
template <class F>
__device__ __forceinline__ void tq_walk(uint32_t* slot, uint32_t epoch, uint32_t next_epoch, int G,
                                        int per_group, F&& process) {
  __shared__ int32_t s_tile[2];
  const int nq = min(tq::kQueues, (int)gridDim.x);
  const int myq = (int)(blockIdx.x % nq);
  int parity = 0;
  for (int qq = 0; qq < nq; ++qq) {
    const int q = (myq + qq) % nq;
    const int rounds = G / nq, left = G % nq;
    const int ngroups = rounds + (((rounds & 1) ? nq - 1 - q : q) < left ? 1 : 0);
    const int64_t ntiles = (int64_t)ngroups * per_group;
    for (;;) {
      if (threadIdx.x == 0) {
        DeviceWord w{slot + q};
        s_tile[parity] = (int32_t)tq::take(w, epoch);
      }
      __syncthreads();
      const int64_t t = s_tile[parity];
      parity ^= 1;
      if (t >= ntiles) break;
      const int k = (int)(t / per_group), rem = (int)(t - (int64_t)k * per_group);
      process(k * nq + ((k & 1) ? nq - 1 - q : q), rem);
    }
  }
  if (threadIdx.x == 0) {
    DeviceWord done{slot + tq::kQueues};
    if (tq::finish(done, epoch, gridDim.x)) {
#pragma unroll
      for (int i = 0; i < tq::kWords; ++i) atomicExch(slot + i, tq::word(next_epoch, 0u));
    }
  }
}

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
