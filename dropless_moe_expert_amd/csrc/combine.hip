// Unpermute-and-combine, its backward, and the SwiGLU backward.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", Figure 3 and section "Optimization 2": combine brings expert
// outputs back to the original token order and accumulates them;
// "AI Systems Performance Engineering" ch. 1, §2.3.2 dispatch/combine table:
// the accumulation is a weighted sum by the routing weights.
//
// All three are HBM-bound: one wavefront per token (or row), 16-byte vector
// loads/stores, fp32 arithmetic, bf16 storage.
#include "common.h"

namespace moe {

// y[t] = bf16(sum_k w[t,k] * y_perm[perm_dst[t*K+k]]), k ascending.
// KT > 0: K known at compile time, so all KT row loads of a vector (and of
// VB vectors) are issued before the first is used; KT = 0: any K <= 32.
template <int KT, int VB>
__global__ __launch_bounds__(256) void unpermute_combine_kernel(const uint16_t* __restrict__ y_perm,
                                                                const float* __restrict__ w,
                                                                const int32_t* __restrict__ perm_dst, int64_t T,
                                                                int d, int K, uint16_t* __restrict__ y) {
  constexpr int KM = KT > 0 ? KT : 32;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (KT > 0) K = KT;
  int32_t my_row = 0;
  float my_w = 1.f;
  if (lane < K) {
    my_row = perm_dst[t * K + lane];
    if (w) my_w = w[t * K + lane];
  }
  // broadcast the K rows and weights while every lane is active
  int32_t rows[KM];
  float ws[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    rows[k] = (k < K) ? __shfl(my_row, k, 64) : 0;
    ws[k] = (k < K) ? __shfl(my_w, k, 64) : 0.f;
  }
  const int nvec = d / 8;
  if constexpr (KT > 0) {
    for (int v0 = lane; v0 < nvec; v0 += 64 * VB) {
      uint4 in[VB][KT];
#pragma unroll
      for (int b = 0; b < VB; ++b) {
        const int v = v0 + 64 * b;
#pragma unroll
        for (int k = 0; k < KT; ++k)
          in[b][k] = v < nvec ? reinterpret_cast<const uint4*>(y_perm + (int64_t)rows[k] * d)[v] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int b = 0; b < VB; ++b) {
        const int v = v0 + 64 * b;
        float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
        for (int k = 0; k < KT; ++k) {
          float f[8];
          unpack8(in[b][k], f);
#pragma unroll
          for (int j = 0; j < 8; ++j) acc[j] = fmaf(ws[k], f[j], acc[j]);
        }
        if (v < nvec) reinterpret_cast<uint4*>(y + t * d)[v] = pack8(acc);
      }
    }
  } else {
    for (int v = lane; v < nvec; v += 64) {
      float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
      for (int k = 0; k < 32; ++k) {
        if (k >= K) break;
        float f[8];
        unpack8(reinterpret_cast<const uint4*>(y_perm + (int64_t)rows[k] * d)[v], f);
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(ws[k], f[j], acc[j]);
      }
      reinterpret_cast<uint4*>(y + t * d)[v] = pack8(acc);
    }
  }
}

// dy_perm[perm_dst[t,k]] = bf16(w[t,k] * dy[t]);  dw[t,k] = <dy[t], y_perm[perm_dst[t,k]]>
// MX: dy_perm leaves as MXFP8 along its rows instead (xq codes, xs scales):
// each 32-element block, four neighbouring lanes' vectors, gets its amax
// across those lanes by DPP and the codes of the transposed quantiser's
// row part, the same rule bit for bit.
template <int KT, bool MX>
__global__ __launch_bounds__(256) void combine_backward_kernel(const uint16_t* __restrict__ dy,
                                                               const uint16_t* __restrict__ y_perm,
                                                               const float* __restrict__ w,
                                                               const int32_t* __restrict__ perm_dst, int64_t T,
                                                               int d, int K, uint16_t* __restrict__ dy_perm,
                                                               float* __restrict__ dw, uint8_t* __restrict__ xq,
                                                               uint8_t* __restrict__ xs) {
  constexpr int KM = KT > 0 ? KT : 32;
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  if (KT > 0) K = KT;
  int32_t my_row = 0;
  float my_w = 0.f;
  if (lane < K) {
    my_row = perm_dst[t * K + lane];
    my_w = w[t * K + lane];
  }
  float dot[KM];
  int32_t rows[KM];
  float ws[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    dot[k] = 0.f;
    rows[k] = (k < K) ? __shfl(my_row, k, 64) : 0;
    ws[k] = (k < K) ? __shfl(my_w, k, 64) : 0.f;
  }
  const int nvec = d / 8;
  for (int v = lane; v < nvec; v += 64) {
    float g[8];
    unpack8(reinterpret_cast<const uint4*>(dy + t * d)[v], g);
    uint4 in[KM];
    if constexpr (KT > 0) {
      // every row load of this vector in flight before the first is used
#pragma unroll
      for (int k = 0; k < KT; ++k) in[k] = reinterpret_cast<const uint4*>(y_perm + (int64_t)rows[k] * d)[v];
    }
#pragma unroll
    for (int k = 0; k < KM; ++k) {
      if (k < K) {
        const int32_t r = rows[k];
        float yv[8];
        if constexpr (KT > 0) {
          unpack8(in[k], yv);
        } else {
          unpack8(reinterpret_cast<const uint4*>(y_perm + (int64_t)r * d)[v], yv);
        }
        float sacc = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) sacc = fmaf(g[j], yv[j], sacc);
        dot[k] += sacc;
        if constexpr (MX) {
          const uint4 o = mul8_bf16(ws[k], g);
          uint32_t m = max_u16x2(max_u16x2(mag_pair(o.x), mag_pair(o.y)), max_u16x2(mag_pair(o.z), mag_pair(o.w)));
          m = max_u16x2(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0xB1, 0xF, 0xF, false));   // lane ^ 1
          m = max_u16x2(m, (uint32_t)__builtin_amdgcn_mov_dpp((int)m, 0x4E, 0xF, 0xF, false));   // lane ^ 2
          const int e = mx_exponent(amax_of_pair(m));
          uint2 q;
          if (e != kMxNaN) {
            const float sc = mx_scale_operand(e);
            const uint32_t lim2 = mx_clamp_pair(e);
            q = make_uint2(mx_codes4_pairs(o.x, o.y, sc, lim2), mx_codes4_pairs(o.z, o.w, sc, lim2));
          } else {
            q = make_uint2(mx_nan_codes4_pairs(o.x, o.y), mx_nan_codes4_pairs(o.z, o.w));
          }
          reinterpret_cast<uint2*>(xq + (int64_t)r * d)[v] = q;
          if ((lane & 3) == 0) xs[(int64_t)r * (d / 32) + (v >> 2)] = (uint8_t)(e + 127);
        } else {
          if (dy_perm) reinterpret_cast<uint4*>(dy_perm + (int64_t)r * d)[v] = mul8_bf16(ws[k], g);
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k < K) {
      const float sum = wave_sum(dot[k]);
      if (lane == 0) dw[t * K + k] = sum;
    }
  }
}

// dgu = [dg | du] from gu = [g | u], dh; rows < sum(group_sizes) (or all rows)
__global__ __launch_bounds__(256) void swiglu_backward_kernel(const uint16_t* __restrict__ gu,
                                                              const uint16_t* __restrict__ dh, int64_t m_cap, int f,
                                                              const int32_t* __restrict__ group_sizes, int G,
                                                              uint16_t* __restrict__ dgu) {
  __shared__ int64_t s_rows;
  if (threadIdx.x < kWave) {
    const int64_t tot = group_sizes ? rows_in_use(group_sizes, G, m_cap) : m_cap;
    if (threadIdx.x == 0) s_rows = tot;
  }
  __syncthreads();
  const int64_t rows = s_rows;
  const int nvec = f / 8;
  const int64_t total = rows * nvec;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = idx / nvec;
    const int v = (int)(idx - r * nvec);
    float g[8], u[8], d[8], dg[8], du[8];
    unpack8(reinterpret_cast<const uint4*>(gu + r * 2 * f)[v], g);
    unpack8(reinterpret_cast<const uint4*>(gu + r * 2 * f + f)[v], u);
    unpack8(reinterpret_cast<const uint4*>(dh + r * f)[v], d);
#pragma unroll
    for (int j = 0; j < 8; ++j) swiglu_grad(g[j], u[j], d[j], dg[j], du[j]);
    reinterpret_cast<uint4*>(dgu + r * 2 * f)[v] = pack8(dg);
    reinterpret_cast<uint4*>(dgu + r * 2 * f + f)[v] = pack8(du);
  }
}

}  // namespace moe

extern "C" moe_status_t moe_unpermute_combine_launch(const uint16_t* y_perm, const float* w, const int32_t* perm_dst,
                                                     int64_t T, int32_t d, int32_t K, uint16_t* y, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const dim3 g((unsigned)((T + 3) / 4)), b(256);
  switch (K) {
    case 1: hipLaunchKernelGGL((moe::unpermute_combine_kernel<1, 8>), g, b, 0, s, y_perm, w, perm_dst, T, d, K, y); break;
    case 2: hipLaunchKernelGGL((moe::unpermute_combine_kernel<2, 4>), g, b, 0, s, y_perm, w, perm_dst, T, d, K, y); break;
    case 4: hipLaunchKernelGGL((moe::unpermute_combine_kernel<4, 2>), g, b, 0, s, y_perm, w, perm_dst, T, d, K, y); break;
    case 8: hipLaunchKernelGGL((moe::unpermute_combine_kernel<8, 2>), g, b, 0, s, y_perm, w, perm_dst, T, d, K, y); break;
    default: hipLaunchKernelGGL((moe::unpermute_combine_kernel<0, 1>), g, b, 0, s, y_perm, w, perm_dst, T, d, K, y);
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status_t moe_combine_backward_launch(const uint16_t* dy, const uint16_t* y_perm, const float* w,
                                                    const int32_t* perm_dst, int64_t T, int32_t d, int32_t K,
                                                    uint16_t* dy_perm, float* dw, uint8_t* xq, uint8_t* xs,
                                                    hipStream_t s) {
  if (T == 0) return MOE_OK;
  const dim3 g((unsigned)((T + 3) / 4)), b(256);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, g, b, 0, s, dy, y_perm, w, perm_dst, T, d, K, dy_perm, dw, xq, xs);
  };
  if (xq) {
    switch (K) {
      case 2: go(moe::combine_backward_kernel<2, true>); break;
      case 8: go(moe::combine_backward_kernel<8, true>); break;
      default: go(moe::combine_backward_kernel<0, true>);
    }
  } else {
    switch (K) {
      case 2: go(moe::combine_backward_kernel<2, false>); break;
      case 8: go(moe::combine_backward_kernel<8, false>); break;
      default: go(moe::combine_backward_kernel<0, false>);
    }
  }
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status_t moe_swiglu_backward_launch(const uint16_t* gu, const uint16_t* dh, int64_t m_cap, int32_t f,
                                                   const int32_t* group_sizes, int32_t G, uint16_t* dgu,
                                                   hipStream_t s) {
  if (m_cap == 0) return MOE_OK;
  const int64_t work = m_cap * (f / 8);
  const int64_t blocks = std::min<int64_t>((work + 255) / 256, (int64_t)moe_host::device_cu_count() * 16);
  hipLaunchKernelGGL(moe::swiglu_backward_kernel, dim3((unsigned)std::max<int64_t>(blocks, 1)), dim3(256), 0, s, gu,
                     dh, m_cap, f, group_sizes, G, dgu);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
