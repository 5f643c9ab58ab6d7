// Permute = dispatch, local part: a stable counting sort of (token, expert)
// pairs into expert-contiguous rows, then the row copy of x.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", section "Optimization 2": dispatch reorders tokens locally by
// expert before the exchange; Figure 3: combine restores the original order.
//
// Three launches, no atomics deciding any order:
//   1. rank:    one wavefront per chunk of kChunk pairs, its ids loaded at
//               once.  Pairs are taken 64 at
//               a time in pair order; a lane's rank among equal experts in
//               the chunk = running count + lanes below it with the same
//               expert (found with 8 ballots over the id bits).  Writes the
//               local rank of every pair and the chunk's per-expert counts.
//   2. scan:    one workgroup: each expert's chunks split over 1024 / E
//               threads (a thread's loads all in flight, kept in registers);
//               one workgroup-wide scan of the parts' sums in expert-major
//               order gives every part's absolute first row, hence
//               group_offsets, group_sizes and the chunk bases.
//   3. scatter: one wavefront per token: row r = base[chunk][e] + local rank
//               for each of its K pairs; writes perm_dst / perm_src and copies
//               the token's row once from HBM to its K destinations (16-byte
//               vector loads and stores, all of a lane's loads of the row in
//               flight before its stores when K is a compile-time value).
#include <mutex>

#include "common.h"

namespace moe {

constexpr int kChunk = 256;  // pairs per rank wavefront

__global__ __launch_bounds__(64) void permute_rank_kernel(const int32_t* __restrict__ ids, int64_t M, int E,
                                                          int32_t* __restrict__ local_rank,
                                                          int32_t* __restrict__ chunk_counts, uint32_t* flag) {
  __shared__ int32_t running[256];
  const int lane = threadIdx.x;
  for (int e = lane; e < E; e += 64) running[e] = 0;
  __syncthreads();
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  const int64_t c1 = min(M, c0 + kChunk);
  // the chunk's ids, all loads in flight at once (the ranking below is a
  // serial walk over the chunk's 64-pair steps)
  constexpr int kSteps = kChunk / 64;
  int ev[kSteps];
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int64_t i = c0 + 64 * s + lane;
    ev[s] = i < c1 ? ids[i] : 0;
  }
  bool bad = false;
#pragma unroll
  for (int s = 0; s < kSteps; ++s) {
    const int64_t base = c0 + 64 * s;
    if (base >= c1) break;   // uniform
    const int64_t i = base + lane;
    const bool valid = i < c1;
    int e = valid ? ev[s] : 0;
    if (valid && (e < 0 || e >= E)) { bad = true; e = E - 1; }
    // lanes with the same expert: AND over the 8 id bits of (ballot or its complement)
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      uint64_t ones = __ballot(valid && ((e >> b) & 1));
      same &= ((e >> b) & 1) ? ones : ~ones;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int before = __popcll(same & below);
    const int total = __popcll(same);
    int r = 0;
    if (valid) r = running[e] + before;
    __syncthreads();  // all lanes read running[] before the update
    if (valid) {
      local_rank[i] = r;
      if (before == total - 1) running[e] += total;  // highest lane of the class updates
    }
    __syncthreads();
  }
  if (__any(bad) && lane == 0) raise_flag(flag, MOE_FLAG_BAD_EXPERT_ID);
  for (int e = lane; e < E; e += 64) chunk_counts[(int64_t)blockIdx.x * E + e] = running[e];
}

// Scan: thread t owns part p = t / E of expert e = t % E (its loads of a
// chunk row are then consecutive), P = NT / E parts per expert, each a
// contiguous range of chunks.  The parts' sums, laid out expert-major
// (e P + p), go through one workgroup-wide exclusive scan: in that order
// expert e's rows follow every smaller expert's, so the scan at (e, p) is
// directly the absolute row of the part's first pair (group_offsets[e] +
// the rows of the expert's earlier parts), and at (e, 0) the expert's
// offset.  A thread's chunk counts (at most kScanRegs of them) stay in
// registers between the sum and the write-back of the chunk bases, all of
// its loads in flight at once.
constexpr int kScanRegs = 64;

template <int NT>
__device__ __forceinline__ int32_t block_excl_scan(int32_t v, int32_t* wsum, int32_t* total) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  constexpr int NW = NT / 64;
  int32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    int32_t x = lane < NW ? wsum[lane] : 0, xi = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int32_t u = __shfl_up(xi, o, 64);
      if (lane >= o) xi += u;
    }
    if (lane < NW) wsum[lane] = xi - x;   // exclusive prefix of the wavefront totals
    if (lane == NW - 1) wsum[NW] = xi;    // the grand total
  }
  __syncthreads();
  *total = wsum[NW];
  return wsum[w] + incl - v;
}

template <int NT>
__global__ __launch_bounds__(NT) void permute_scan_kernel(int32_t* __restrict__ chunk_counts, int nchunk, int E,
                                                           int32_t* __restrict__ group_sizes,
                                                           int32_t* __restrict__ group_offsets) {
  __shared__ int32_t part[NT];
  __shared__ int32_t wsum[NT / 64 + 1];
  const int tid = threadIdx.x;
  const int P = NT / E;
  const int e = tid % E, p = tid / E;
  const bool active = p < P;
  const int per = (nchunk + P - 1) / P;
  const int c0 = min(nchunk, p * per), c1 = min(nchunk, c0 + per);
  const int n = active ? c1 - c0 : 0;
  int32_t* const col = chunk_counts + (int64_t)c0 * E + e;   // this thread's chunk counts, E apart
  const bool in_regs = per <= kScanRegs;                      // uniform
  int32_t v[kScanRegs];
  int32_t sum = 0;
  if (in_regs) {
#pragma unroll
    for (int b = 0; b < kScanRegs; ++b) v[b] = b < n ? col[(int64_t)b * E] : 0;
#pragma unroll
    for (int b = 0; b < kScanRegs; ++b) sum += v[b];
  } else {
    for (int b = 0; b < n; ++b) sum += col[(int64_t)b * E];
  }
  // expert-major slot of this part; the threads past E P hold zeros at the end
  const int slot = active ? e * P + p : tid;
  part[slot] = sum;
  __syncthreads();
  const int32_t mine = part[tid];
  int32_t total;
  const int32_t excl = block_excl_scan<NT>(mine, wsum, &total);
  __syncthreads();
  part[tid] = excl;   // exclusive scan at each expert-major slot
  __syncthreads();
  if (!active) return;
  const int32_t base = part[slot];   // the row of this part's first pair
  if (p == 0) {
    const int32_t next = e + 1 < E ? part[(e + 1) * P] : total;
    group_offsets[e] = base;
    group_sizes[e] = next - base;
    if (e == E - 1) group_offsets[E] = total;
  }
  int32_t run = base;
  if (in_regs) {
#pragma unroll
    for (int b = 0; b < kScanRegs; ++b) {
      if (b < n) col[(int64_t)b * E] = run;   // absolute base of the chunk
      run += v[b];
    }
  } else {
    for (int b = 0; b < n; ++b) {
      const int32_t c = col[(int64_t)b * E];
      col[(int64_t)b * E] = run;
      run += c;
    }
  }
}

// one wavefront per token
template <int KT>
__global__ __launch_bounds__(256) void permute_scatter_kernel(const uint16_t* __restrict__ x,
                                                              const int32_t* __restrict__ ids,
                                                              const int32_t* __restrict__ local_rank,
                                                              const int32_t* __restrict__ chunk_base, int chunk_pairs,
                                                              int64_t T,
                                                              int d, int E, int K, int32_t* __restrict__ perm_src,
                                                              int32_t* __restrict__ perm_dst,
                                                              uint16_t* __restrict__ x_perm) {
  constexpr int KM = KT > 0 ? KT : 32;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (KT > 0) K = KT;
  // lane k < K resolves pair k
  int32_t my_row = 0;
  if (lane < K) {
    const int64_t i = t * K + lane;
    int e = ids[i];
    if (e < 0 || e >= E) e = E - 1;
    my_row = chunk_base[(i / chunk_pairs) * E + e] + local_rank[i];
    perm_dst[i] = my_row;
    perm_src[my_row] = (int32_t)i;
  }
  if (x == nullptr) return;
  // broadcast the K destination rows while every lane is active
  int32_t rows[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) rows[k] = (k < K) ? __shfl(my_row, k, 64) : 0;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * d);
  const int nvec = d / 8;
  constexpr int VB = 4;   // vectors of the row a lane loads before storing them
  for (int v0 = lane; v0 < nvec; v0 += 64 * VB) {
    uint4 val[VB];
#pragma unroll
    for (int b = 0; b < VB; ++b) val[b] = (v0 + 64 * b < nvec) ? src[v0 + 64 * b] : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int b = 0; b < VB; ++b) {
      const int v = v0 + 64 * b;
      if (v < nvec) {
#pragma unroll
        for (int k = 0; k < KM; ++k)
          if (k < K) reinterpret_cast<uint4*>(x_perm + (int64_t)rows[k] * d)[v] = val[b];
      }
    }
  }
}

// The scatter writing MXFP8: each 32-element block of the token row (four
// consecutive lanes' 16-byte vectors) gets one E8M0 scale and E4M3 codes by
// the same rule and helpers as mxfp8_group_quantize (axis 0), then goes to
// the token's K rows; equal to moe_permute followed by the quantiser.
template <int KT>
__global__ __launch_bounds__(256) void permute_scatter_mx_kernel(const uint16_t* __restrict__ x,
                                                                 const int32_t* __restrict__ ids,
                                                                 const int32_t* __restrict__ local_rank,
                                                                 const int32_t* __restrict__ chunk_base, int chunk_pairs,
                                                                 int64_t T,
                                                                 int d, int E, int K, int32_t* __restrict__ perm_src,
                                                                 int32_t* __restrict__ perm_dst,
                                                                 uint8_t* __restrict__ xq, uint8_t* __restrict__ xs) {
  constexpr int KM = KT > 0 ? KT : 32;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (KT > 0) K = KT;
  int32_t my_row = 0;
  if (lane < K) {
    const int64_t i = t * K + lane;
    int e = ids[i];
    if (e < 0 || e >= E) e = E - 1;
    my_row = chunk_base[(i / chunk_pairs) * E + e] + local_rank[i];
    perm_dst[i] = my_row;
    perm_src[my_row] = (int32_t)i;
  }
  int32_t rows[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) rows[k] = (k < K) ? __shfl(my_row, k, 64) : 0;
  const uint4* src = reinterpret_cast<const uint4*>(x + t * d);
  const int nvec = d / 8;   // a multiple of 4: blocks never straddle lanes of different iterations
  for (int v = lane; v - (lane & 3) < nvec; v += 64) {
    const bool live = v < nvec;
    float f[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (live) unpack8(src[v], f);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = mx_absmax(amax, f[j]);
    amax = mx_absmax(amax, __shfl_xor(amax, 1, 64));
    amax = mx_absmax(amax, __shfl_xor(amax, 2, 64));
    const int e = mx_exponent(amax);
    if (live) {
      uint2 q;
      q.x = mx_codes4(f[0], f[1], f[2], f[3], e);
      q.y = mx_codes4(f[4], f[5], f[6], f[7], e);
#pragma unroll
      for (int k = 0; k < KM; ++k) {
        if (k < K) {
          reinterpret_cast<uint2*>(xq + (int64_t)rows[k] * d)[v] = q;
          if ((lane & 3) == 0) xs[(int64_t)rows[k] * (d / 32) + (v >> 2)] = (uint8_t)(e + 127);
        }
      }
    }
  }
}

}  // namespace moe

// ------------------------------------------------------------------ no-allocation variant
// moe_permute_noalloc runs the same three kernels with their workspace (the
// per-pair ranks and per-chunk counts) in this file-scope device array
// instead of a caller buffer.  Every GPU the library runs on holds its own
// copy at its own address until the process ends.  In host code the array's
// name is not a device address: its address on the current device comes from
// hipGetSymbolAddress, taken once per device on the first call there and
// kept.  Nothing in it needs clearing: the rank kernel writes every entry
// the later kernels read.  Calls that overlap on one GPU share the array and
// race.
namespace {
constexpr size_t kScratchBytes = MOE_PERMUTE_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// device address of the current device's scratch, or nullptr
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" moe_status_t moe_permute_launch(const uint16_t*, const int32_t*, int64_t, int32_t, int32_t, int32_t,
                                           int32_t*, int32_t*, int32_t*, int32_t*, uint16_t*, void*, uint32_t*,
                                           hipStream_t);

extern "C" moe_status_t moe_permute_noalloc_launch(const uint16_t* x, const int32_t* ids, int64_t T, int32_t d,
                                                   int32_t E, int32_t K, int32_t* group_sizes,
                                                   int32_t* group_offsets, int32_t* perm_src, int32_t* perm_dst,
                                                   uint16_t* x_perm, uint32_t* flag, hipStream_t s) {
  void* ws = scratch_ptr();
  if (!ws) return MOE_ERR_HIP;
  return moe_permute_launch(x, ids, T, d, E, K, group_sizes, group_offsets, perm_src, perm_dst, x_perm, ws, flag, s);
}

extern "C" size_t moe_permute_ws_bytes_impl(int64_t T, int32_t E, int32_t K) {
  const int64_t M = T * K;
  const int64_t nchunk = (M + moe::kChunk - 1) / moe::kChunk;
  size_t a = (size_t)M * 4;
  a = (a + 255) & ~(size_t)255;
  size_t b = (size_t)nchunk * E * 4;
  return a + ((b + 255) & ~(size_t)255);
}

extern "C" moe_status_t moe_permute_launch(const uint16_t* x, const int32_t* ids, int64_t T, int32_t d, int32_t E,
                                           int32_t K, int32_t* group_sizes, int32_t* group_offsets,
                                           int32_t* perm_src, int32_t* perm_dst, uint16_t* x_perm, void* ws,
                                           uint32_t* flag, hipStream_t s) {
  const int64_t M = T * K;
  const int64_t nchunk = (M + moe::kChunk - 1) / moe::kChunk;
  int32_t* local_rank = reinterpret_cast<int32_t*>(ws);
  size_t a = ((size_t)M * 4 + 255) & ~(size_t)255;
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + a);
  if (M > 0) {
    hipLaunchKernelGGL(moe::permute_rank_kernel, dim3((unsigned)nchunk), dim3(64), 0, s, ids, M, E, local_rank,
                       chunk_counts, flag);
  }
  hipLaunchKernelGGL(moe::permute_scan_kernel<1024>, dim3(1), dim3(1024), 0, s, chunk_counts, (int)nchunk, E, group_sizes,
                     group_offsets);
  if (T > 0) {
    const dim3 g((unsigned)((T + 3) / 4)), b(256);
    switch (K) {
      case 1: hipLaunchKernelGGL((moe::permute_scatter_kernel<1>), g, b, 0, s, x, ids, local_rank, chunk_counts,
                                 moe::kChunk, T, d, E, K, perm_src, perm_dst, x_perm); break;
      case 2: hipLaunchKernelGGL((moe::permute_scatter_kernel<2>), g, b, 0, s, x, ids, local_rank, chunk_counts,
                                 moe::kChunk, T, d, E, K, perm_src, perm_dst, x_perm); break;
      case 4: hipLaunchKernelGGL((moe::permute_scatter_kernel<4>), g, b, 0, s, x, ids, local_rank, chunk_counts,
                                 moe::kChunk, T, d, E, K, perm_src, perm_dst, x_perm); break;
      case 8: hipLaunchKernelGGL((moe::permute_scatter_kernel<8>), g, b, 0, s, x, ids, local_rank, chunk_counts,
                                 moe::kChunk, T, d, E, K, perm_src, perm_dst, x_perm); break;
      default: hipLaunchKernelGGL((moe::permute_scatter_kernel<0>), g, b, 0, s, x, ids, local_rank, chunk_counts,
                                  moe::kChunk, T, d, E, K, perm_src, perm_dst, x_perm);
    }
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status_t moe_permute_mxfp8_launch(const uint16_t* x, const int32_t* ids, int64_t T, int32_t d, int32_t E,
                                                 int32_t K, int32_t* group_sizes, int32_t* group_offsets,
                                                 int32_t* perm_src, int32_t* perm_dst, uint8_t* xq, uint8_t* xs,
                                                 void* ws, uint32_t* flag, hipStream_t s) {
  const int64_t M = T * K;
  const int64_t nchunk = (M + moe::kChunk - 1) / moe::kChunk;
  int32_t* local_rank = reinterpret_cast<int32_t*>(ws);
  size_t a = ((size_t)M * 4 + 255) & ~(size_t)255;
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + a);
  if (M > 0) {
    hipLaunchKernelGGL(moe::permute_rank_kernel, dim3((unsigned)nchunk), dim3(64), 0, s, ids, M, E, local_rank,
                       chunk_counts, flag);
  }
  hipLaunchKernelGGL(moe::permute_scan_kernel<1024>, dim3(1), dim3(1024), 0, s, chunk_counts, (int)nchunk, E, group_sizes,
                     group_offsets);
  if (T > 0) {
    const dim3 g((unsigned)((T + 3) / 4)), b(256);
    switch (K) {
      case 2: hipLaunchKernelGGL((moe::permute_scatter_mx_kernel<2>), g, b, 0, s, x, ids, local_rank, chunk_counts,
                                 moe::kChunk, T, d, E, K, perm_src, perm_dst, xq, xs); break;
      case 8: hipLaunchKernelGGL((moe::permute_scatter_mx_kernel<8>), g, b, 0, s, x, ids, local_rank, chunk_counts,
                                 moe::kChunk, T, d, E, K, perm_src, perm_dst, xq, xs); break;
      default: hipLaunchKernelGGL((moe::permute_scatter_mx_kernel<0>), g, b, 0, s, x, ids, local_rank, chunk_counts,
                                  moe::kChunk, T, d, E, K, perm_src, perm_dst, xq, xs);
    }
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

// The permute after moe_route_fused: the router already wrote each pair's
// rank within its token block and the blocks' per-expert counts (chunks of
// chunk_tokens tokens), so only the scan and the scatter run.
extern "C" moe_status_t moe_permute_routed_launch(const uint16_t* x, const int32_t* ids, int64_t T, int32_t d,
                                                  int32_t E, int32_t K, int32_t chunk_tokens, int32_t* group_sizes,
                                                  int32_t* group_offsets, int32_t* perm_src, int32_t* perm_dst,
                                                  uint16_t* x_perm, void* ws, hipStream_t s) {
  const int64_t M = T * K;
  const int64_t nchunk = (T + chunk_tokens - 1) / chunk_tokens;
  const int chunk_pairs = chunk_tokens * K;
  int32_t* local_rank = reinterpret_cast<int32_t*>(ws);
  size_t a = ((size_t)M * 4 + 255) & ~(size_t)255;
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + a);
  hipLaunchKernelGGL(moe::permute_scan_kernel<1024>, dim3(1), dim3(1024), 0, s, chunk_counts, (int)nchunk, E, group_sizes,
                     group_offsets);
  if (T > 0) {
    const dim3 g((unsigned)((T + 3) / 4)), b(256);
    switch (K) {
      case 2: hipLaunchKernelGGL((moe::permute_scatter_kernel<2>), g, b, 0, s, x, ids, local_rank, chunk_counts,
                                 chunk_pairs, T, d, E, K, perm_src, perm_dst, x_perm); break;
      case 8: hipLaunchKernelGGL((moe::permute_scatter_kernel<8>), g, b, 0, s, x, ids, local_rank, chunk_counts,
                                 chunk_pairs, T, d, E, K, perm_src, perm_dst, x_perm); break;
      default: hipLaunchKernelGGL((moe::permute_scatter_kernel<0>), g, b, 0, s, x, ids, local_rank, chunk_counts,
                                  chunk_pairs, T, d, E, K, perm_src, perm_dst, x_perm);
    }
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
