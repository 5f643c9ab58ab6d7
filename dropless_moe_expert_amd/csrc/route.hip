// Router top-K with softmax gating: a group of LPT lanes per token.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", intro: a learned router picks each token's Top-K experts.
// "AI Systems Performance Engineering" ch. 1, §4.1 softmax worked example:
// exponentials of (score - row max) divided by their sum.
//
// A token's E <= 256 logits are spread over LPT = 2..16 lanes (inside one DPP
// row), VPL of them per lane, so one wavefront serves 64 / LPT tokens.  Lane
// `sub` holds the experts (c * LPT + sub) * VW + i, i < VW, for its chunks c
// of VW = min(VPL, 4) consecutive logits: ascending in the lane's own order,
// and one chunk per lane is one vector load, contiguous over the group.
//
// Selection and weights: route_select.h (branch-free integer keys, DPP
// butterflies within the group; the ids are exact).
//
// Measured on 16384 tokens x 128 experts, top 8: the previous form of this
// kernel (float compares with the index tie-break written as a short-circuit
// condition per logit) compiled to exec-mask branches around every compare
// and took 11.6 us.
#include "route_select.h"

namespace moe {

// VEC: E is a multiple of VW and the logits 4-byte aligned per row start of a
// vector (the launcher checks), so a chunk is one load; else one per logit.
// SLOTS: picks kept per lane, pick k in lane k % LPT, slot k / LPT.
template <int LPT, int VPL, int SLOTS, bool VEC>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int64_t T, int E, int K,
                                                         int renorm, int32_t* __restrict__ ids,
                                                         float* __restrict__ w, uint32_t* flag) {
  using G = topk::Group<LPT, VPL>;
  constexpr int VW = G::VW;
  constexpr int TPW = 64 / LPT;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPT;
  const int64_t t = ((int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)) * TPW + lane / LPT;
  const bool live = t < T;
  const float* row = logits + (live ? t : T - 1) * E;
  auto expert = [&](int j) { return G::expert(sub, j); };

  float v[VPL];
  if constexpr (VEC) {
    using vec_t = float __attribute__((ext_vector_type(VW)));
#pragma unroll
    for (int c = 0; c < VPL / VW; ++c) {
      const int e0 = expert(c * VW);
      const vec_t x = *reinterpret_cast<const vec_t*>(row + (e0 < E ? e0 : 0));
#pragma unroll
      for (int i = 0; i < VW; ++i) v[c * VW + i] = x[i];
    }
  } else {
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int e = expert(j);
      v[j] = row[e < E ? e : 0];
    }
  }
  bool nan_seen = false;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const bool in = G::expert(sub, j) < E;
    const bool nan = v[j] != v[j];
    nan_seen |= in && nan;
    v[j] = (!in || nan) ? -INFINITY : v[j];
  }
  if (__any(live && nan_seen) && lane == 0) raise_flag(flag, MOE_FLAG_NAN_LOGIT);

  int pk[SLOTS], pi[SLOTS], kmax;
  G::template select<SLOTS>(v, E, K, sub, pk, pi, kmax);
  float a[SLOTS];
  const float part = G::template weights<SLOTS>(v, E, K, renorm, sub, pk, kmax, a);
  if (live) {
#pragma unroll
    for (int q = 0; q < SLOTS; ++q) {
      const int k = q * LPT + sub;
      if (k < K) {
        ids[t * K + k] = pi[q];
        w[t * K + k] = a[q] / part;
      }
    }
  }
}

template <int LPT, int VPL>
void route_launch(const float* logits, int64_t T, int E, int K, int renorm, int32_t* ids, float* w,
                  uint32_t* flag, hipStream_t s) {
  constexpr int VW = VPL < 4 ? VPL : 4;
  const bool vec = E % VW == 0 && reinterpret_cast<uintptr_t>(logits) % (4 * VW) == 0;
  const int64_t tokens_per_block = 4 * (64 / LPT);
  const dim3 grid((unsigned)((T + tokens_per_block - 1) / tokens_per_block));
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, logits, T, E, K, renorm, ids, w, flag); };
  constexpr int MAXS = (32 + LPT - 1) / LPT;
  if (K <= LPT) {
    vec ? go(route_topk_kernel<LPT, VPL, 1, true>) : go(route_topk_kernel<LPT, VPL, 1, false>);
  } else {
    vec ? go(route_topk_kernel<LPT, VPL, MAXS, true>) : go(route_topk_kernel<LPT, VPL, MAXS, false>);
  }
}

}  // namespace moe

extern "C" moe_status_t moe_route_topk_launch(const float* logits, int64_t T, int32_t E, int32_t K, int32_t renorm,
                                              int32_t* ids, float* w, uint32_t* flag, hipStream_t s) {
  if (T == 0) return MOE_OK;
  // lanes per token and logits per lane: LPT * VPL >= E, VPL <= 16
  if (E <= 8) {
    moe::route_launch<2, 4>(logits, T, E, K, renorm, ids, w, flag, s);
  } else if (E <= 16) {
    moe::route_launch<4, 4>(logits, T, E, K, renorm, ids, w, flag, s);
  } else if (E <= 32) {
    moe::route_launch<4, 8>(logits, T, E, K, renorm, ids, w, flag, s);
  } else if (E <= 64) {
    moe::route_launch<8, 8>(logits, T, E, K, renorm, ids, w, flag, s);
  } else if (E <= 128) {
    moe::route_launch<8, 16>(logits, T, E, K, renorm, ids, w, flag, s);
  } else {
    moe::route_launch<16, 16>(logits, T, E, K, renorm, ids, w, flag, s);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
