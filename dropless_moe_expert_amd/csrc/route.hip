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
// Selection is branch-free integer work.  Each logit becomes a key, the
// signed integer whose order is the float order (-0 is first made +0, NaN
// was made -inf); a taken or absent expert holds INT_MIN, below every key.
// A round is: the lane's maximum key (max3 chains), the group's maximum M
// (DPP butterfly), the lowest expert holding M in the lane, the group's
// lowest such expert W (the pick: larger logit first, ties to the lower
// index), and W's key set to INT_MIN by the lane that holds it.  The ids are
// exact.  Weights: exp(l - l_max) over the sum (the K picks, or all E).
//
// Measured on 16384 tokens x 128 experts, top 8: the previous form of this
// kernel (float compares with the index tie-break written as a short-circuit
// condition per logit) compiled to exec-mask branches around every compare
// and took 11.6 us.
#include <climits>

#include "common.h"

namespace moe {

// Lane exchanges inside a row of 16 lanes by DPP (a VALU move, no trip
// through the LDS crossbar): level 0 swaps neighbours (quad_perm 1,0,3,2),
// level 1 pairs of neighbours (quad_perm 2,3,0,1), level 2 the two quads of a
// half row (row_half_mirror), level 3 the two half rows (row_mirror).  After
// levels 0..log2(n)-1 every lane of an aligned group of n lanes has met all
// of them, so a max or a sum over the levels reaches every lane of the group
// (a sum bit-identically: each level adds the same two values in either
// order).
template <int LEVEL>
__device__ __forceinline__ int dpp_xchg(int v) {
  constexpr int ctrl = LEVEL == 0 ? 0xB1 : LEVEL == 1 ? 0x4E : LEVEL == 2 ? 0x141 : 0x140;
  return __builtin_amdgcn_mov_dpp(v, ctrl, 0xF, 0xF, false);
}
template <int LEVEL>
__device__ __forceinline__ float dpp_xchg(float v) {
  return __int_as_float(dpp_xchg<LEVEL>(__float_as_int(v)));
}

// The same exchanges with the partner value in the position an unfused DPP
// max or min can take (old value = the operation's identity), so the move
// and the operation can issue as one DPP instruction.
template <int LEVEL>
__device__ __forceinline__ int dpp_xchg_or(int identity, int v) {
  constexpr int ctrl = LEVEL == 0 ? 0xB1 : LEVEL == 1 ? 0x4E : LEVEL == 2 ? 0x141 : 0x140;
  return __builtin_amdgcn_update_dpp(identity, v, ctrl, 0xF, 0xF, false);
}
template <int LPT>
__device__ __forceinline__ int group_max(int v) {
  v = max(dpp_xchg_or<0>(INT_MIN, v), v);
  if constexpr (LPT >= 4) v = max(dpp_xchg_or<1>(INT_MIN, v), v);
  if constexpr (LPT >= 8) v = max(dpp_xchg_or<2>(INT_MIN, v), v);
  if constexpr (LPT >= 16) v = max(dpp_xchg_or<3>(INT_MIN, v), v);
  return v;
}
template <int LPT>
__device__ __forceinline__ int group_min(int v) {
  v = min(dpp_xchg_or<0>(INT_MAX, v), v);
  if constexpr (LPT >= 4) v = min(dpp_xchg_or<1>(INT_MAX, v), v);
  if constexpr (LPT >= 8) v = min(dpp_xchg_or<2>(INT_MAX, v), v);
  if constexpr (LPT >= 16) v = min(dpp_xchg_or<3>(INT_MAX, v), v);
  return v;
}
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp_xchg<0>(v);
  if constexpr (LPT >= 4) v += dpp_xchg<1>(v);
  if constexpr (LPT >= 8) v += dpp_xchg<2>(v);
  if constexpr (LPT >= 16) v += dpp_xchg<3>(v);
  return v;
}

// order-preserving integer key of a non-NaN float (equal floats, equal keys)
__device__ __forceinline__ int order_key(float x) {
  const int b = x == 0.f ? 0 : __float_as_int(x);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key_value(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

// VEC: E is a multiple of VW and the logits 4-byte aligned per row start of a
// vector (the launcher checks), so a chunk is one load; else one per logit.
// SLOTS: picks kept per lane, pick k in lane k % LPT, slot k / LPT.
template <int LPT, int VPL, int SLOTS, bool VEC>
__global__ __launch_bounds__(256) void route_topk_kernel(const float* __restrict__ logits, int64_t T, int E, int K,
                                                         int renorm, int32_t* __restrict__ ids,
                                                         float* __restrict__ w, uint32_t* flag) {
  static_assert(LPT == 2 || LPT == 4 || LPT == 8 || LPT == 16, "groups inside one DPP row");
  constexpr int VW = VPL < 4 ? VPL : 4;
  static_assert(VPL % VW == 0, "whole chunks");
  constexpr int TPW = 64 / LPT;
  const int lane = threadIdx.x & 63;
  const int sub = lane % LPT;
  const int64_t t = ((int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)) * TPW + lane / LPT;
  const bool live = t < T;
  const float* row = logits + (live ? t : T - 1) * E;
  auto expert = [&](int j) { return ((j / VW) * LPT + sub) * VW + j % VW; };

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
  int key[VPL];
  bool nan_seen = false;
#pragma unroll
  for (int j = 0; j < VPL; ++j) {
    const bool in = expert(j) < E;
    const bool nan = v[j] != v[j];
    nan_seen |= in && nan;
    v[j] = (!in || nan) ? -INFINITY : v[j];
    key[j] = in ? order_key(v[j]) : INT_MIN;
  }
  if (__any(live && nan_seen) && lane == 0) raise_flag(flag, MOE_FLAG_NAN_LOGIT);

  int pk[SLOTS], pi[SLOTS];
#pragma unroll
  for (int q = 0; q < SLOTS; ++q) { pk[q] = INT_MIN; pi[q] = 0; }
  int kmax = 0;
  for (int k = 0; k < K; ++k) {
    int m = key[0];
#pragma unroll
    for (int j = 1; j < VPL; ++j) m = max(m, key[j]);
    m = group_max<LPT>(m);
    // the lane's lowest expert holding m, then the group's
    int li = INT_MAX;
    bool first[VPL];
    bool seen = false;
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const bool eq = key[j] == m;
      first[j] = eq && !seen;
      seen = seen || eq;
      li = first[j] ? expert(j) : li;
    }
    const int wi = group_min<LPT>(li);
    const bool owner = li == wi;
#pragma unroll
    for (int j = 0; j < VPL; ++j) key[j] = (owner && first[j]) ? INT_MIN : key[j];
    if (k == 0) kmax = m;   // the first pick is the row maximum
#pragma unroll
    for (int q = 0; q < SLOTS; ++q)
      if (k == q * LPT + sub) { pk[q] = m; pi[q] = wi; }
  }
  const float lmax = key_value(kmax);
  float a[SLOTS];
  float part = 0.f;
#pragma unroll
  for (int q = 0; q < SLOTS; ++q) {
    a[q] = (q * LPT + sub < K) ? expf(key_value(pk[q]) - lmax) : 0.f;
    part += a[q];
  }
  if (!renorm) {
    part = 0.f;
#pragma unroll
    for (int j = 0; j < VPL; ++j)
      if (expert(j) < E) part += expf(v[j] - lmax);
  }
  part = group_sum<LPT>(part);
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
