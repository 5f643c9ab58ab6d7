// Top-K selection of a token's logits spread over a group of LPT lanes, and
// the softmax weights of the picks: shared by the router and the fused
// router, so both return the same ids and weights for the same logits.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", intro: a learned router picks each token's Top-K experts.
// "AI Systems Performance Engineering" ch. 1, §4.1 softmax worked example:
// exponentials of (score - row max) divided by their sum.
//
// Lane `sub` of a group holds VPL logits, experts (c * LPT + sub) * VW + i,
// i < VW, of its chunks c of VW = min(VPL, 4) consecutive experts
// (ascending in the lane's own order).  Each logit becomes a key, the signed
// integer whose order is the float order (-0 folded into +0; NaN must have
// been made -inf), and a taken or absent expert (>= E) holds INT_MIN, below
// every key.  A round is branch-free integer work: the lane's maximum key
// (max3 chains), the group's maximum M (DPP butterfly fused into max), the
// lowest expert holding M in the lane, the group's lowest such expert W (the
// pick: larger logit first, ties to the lower index), and W's key set to
// INT_MIN by the lane that holds it.  Weights: exp(l - l_max) over the sum
// of the K picks (renormalised) or of all E.
#pragma once
#include <climits>

#include "common.h"

namespace moe {
namespace topk {

// Lane exchanges inside a row of 16 lanes by DPP: level 0 swaps neighbours
// (quad_perm 1,0,3,2), level 1 pairs of neighbours (quad_perm 2,3,0,1),
// level 2 the two quads of a half row (row_half_mirror), level 3 the two
// half rows (row_mirror).  After levels 0..log2(n)-1 every lane of an
// aligned group of n lanes has met all of them, so a max, min or sum over
// the levels reaches every lane of the group (a sum bit-identically: each
// level adds the same two values in either order).  The identity as the
// old value lets the move fuse into the DPP form of max and min.
template <int LEVEL>
__device__ __forceinline__ int xchg(int identity, int v) {
  constexpr int ctrl = LEVEL == 0 ? 0xB1 : LEVEL == 1 ? 0x4E : LEVEL == 2 ? 0x141 : 0x140;
  return __builtin_amdgcn_update_dpp(identity, v, ctrl, 0xF, 0xF, false);
}
template <int LEVEL>
__device__ __forceinline__ float xchg(float v) {
  constexpr int ctrl = LEVEL == 0 ? 0xB1 : LEVEL == 1 ? 0x4E : LEVEL == 2 ? 0x141 : 0x140;
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), ctrl, 0xF, 0xF, false));
}
template <int LPT>
__device__ __forceinline__ int group_max(int v) {
  v = max(xchg<0>(INT_MIN, v), v);
  if constexpr (LPT >= 4) v = max(xchg<1>(INT_MIN, v), v);
  if constexpr (LPT >= 8) v = max(xchg<2>(INT_MIN, v), v);
  if constexpr (LPT >= 16) v = max(xchg<3>(INT_MIN, v), v);
  return v;
}
template <int LPT>
__device__ __forceinline__ int group_min(int v) {
  v = min(xchg<0>(INT_MAX, v), v);
  if constexpr (LPT >= 4) v = min(xchg<1>(INT_MAX, v), v);
  if constexpr (LPT >= 8) v = min(xchg<2>(INT_MAX, v), v);
  if constexpr (LPT >= 16) v = min(xchg<3>(INT_MAX, v), v);
  return v;
}
template <int LPT>
__device__ __forceinline__ float group_sum(float v) {
  v += xchg<0>(v);
  if constexpr (LPT >= 4) v += xchg<1>(v);
  if constexpr (LPT >= 8) v += xchg<2>(v);
  if constexpr (LPT >= 16) v += xchg<3>(v);
  return v;
}

// order-preserving integer key of a non-NaN float (equal floats, equal keys)
__device__ __forceinline__ int order_key(float x) {
  const int b = x == 0.f ? 0 : __float_as_int(x);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}
__device__ __forceinline__ float key_value(int k) { return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF)); }

template <int LPT, int VPL>
struct Group {
  static_assert(LPT == 2 || LPT == 4 || LPT == 8 || LPT == 16, "groups inside one DPP row");
  static constexpr int VW = VPL < 4 ? VPL : 4;
  static_assert(VPL % VW == 0, "whole chunks");
  static constexpr int SLOTS_MAX = (32 + LPT - 1) / LPT;   // K <= 32
  // expert of the lane's value j
  __device__ static __forceinline__ int expert(int sub, int j) { return ((j / VW) * LPT + sub) * VW + j % VW; }

  // The K picks of the group's token, pick k kept by lane k % LPT in slot
  // k / LPT (pk: its key, pi: its expert); kmax: the key of the first pick
  // (the row maximum).  v: the lane's logits, NaN already -inf; experts >= E
  // are absent.  K <= E.
  template <int SLOTS>
  __device__ static __forceinline__ void select(const float (&v)[VPL], int E, int K, int sub, int (&pk)[SLOTS],
                                                int (&pi)[SLOTS], int& kmax) {
    int key[VPL];
#pragma unroll
    for (int j = 0; j < VPL; ++j) key[j] = expert(sub, j) < E ? order_key(v[j]) : INT_MIN;
#pragma unroll
    for (int q = 0; q < SLOTS; ++q) { pk[q] = INT_MIN; pi[q] = 0; }
    kmax = 0;
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
        li = first[j] ? expert(sub, j) : li;
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
  }

  // a[q]: exp(pick - max) of the lane's slots (0 past K); returns the
  // group's sum of them (renorm) or of exp(l - max) over all E experts
  template <int SLOTS>
  __device__ static __forceinline__ float weights(const float (&v)[VPL], int E, int K, int renorm, int sub,
                                                  const int (&pk)[SLOTS], int kmax, float (&a)[SLOTS]) {
    const float lmax = key_value(kmax);
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
        if (expert(sub, j) < E) part += expf(v[j] - lmax);
    }
    return group_sum<LPT>(part);
  }
};

}  // namespace topk
}  // namespace moe
