// Router top-K with softmax gating: one wavefront per token.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", intro: a learned router picks each token's Top-K experts.
// "AI Systems Performance Engineering" ch. 1, §4.1 softmax worked example:
// exponentials of (score - row max) divided by their sum.
//
// A token's E <= 256 logits sit in registers (E/64 per lane).  K rounds of a
// wavefront argmax pick the experts; the comparison is on raw fp32 logits,
// larger wins and equal logits go to the lower expert index, so the ids are
// exact.  Weights: exp(l - l_max) over the sum (the K picks, or all E).
#include "common.h"

namespace moe {

constexpr int kRouteMaxPerLane = 4;  // E <= 256

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int64_t T, int E, int K,
                                                         int renorm, int32_t* __restrict__ ids,
                                                         float* __restrict__ w, uint32_t* flag) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + t * E;
  float v[kRouteMaxPerLane];
  bool nan_seen = false;
#pragma unroll
  for (int j = 0; j < kRouteMaxPerLane; ++j) {
    int e = lane + 64 * j;
    float x = (e < E) ? row[e] : -INFINITY;
    if (x != x) { nan_seen = true; x = -INFINITY; }
    v[j] = x;
  }
  if (__any(nan_seen) && lane == 0) raise_flag(flag, MOE_FLAG_NAN_LOGIT);
  unsigned taken = 0;  // bit j: expert lane + 64j already picked
  float my_logit = -INFINITY;  // lane k keeps the k-th pick
  int my_id = 0;
  for (int k = 0; k < K; ++k) {
    // lane-local best among untaken (index order within a lane is ascending)
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < kRouteMaxPerLane; ++j) {
      int e = lane + 64 * j;
      if (e < E && !((taken >> j) & 1u) && better(v[j], e, bv, bi)) { bv = v[j]; bi = e; }
    }
    // wavefront argmax
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      float ov = __shfl_xor(bv, o, 64);
      int oi = __shfl_xor(bi, o, 64);
      if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    if (lane == k) { my_logit = bv; my_id = bi; }
  }
  const float lmax = __shfl(my_logit, 0, 64);  // the first pick is the row maximum
  const float a = (lane < K) ? expf(my_logit - lmax) : 0.f;
  float denom;
  if (renorm) {
    denom = wave_sum(a);
  } else {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kRouteMaxPerLane; ++j) {
      int e = lane + 64 * j;
      if (e < E) s += expf(v[j] - lmax);
    }
    denom = wave_sum(s);
  }
  if (lane < K) {
    ids[t * K + lane] = my_id;
    w[t * K + lane] = a / denom;
  }
}

}  // namespace moe

extern "C" moe_status_t moe_route_topk_launch(const float* logits, int64_t T, int32_t E, int32_t K, int32_t renorm,
                                              int32_t* ids, float* w, uint32_t* flag, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const int tokens_per_block = 4;
  dim3 grid((unsigned)((T + tokens_per_block - 1) / tokens_per_block));
  hipLaunchKernelGGL(moe::route_topk_kernel, grid, dim3(256), 0, s, logits, T, E, K, renorm, ids, w, flag);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
