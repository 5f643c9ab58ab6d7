// Measurement kernel: the MFMA ceiling of the grouped GEMM's inner loop.
//
// Not a step of the layer.  It runs the bf16 GEMM's compute pattern with no
// global memory traffic: one 8-wavefront workgroup per CU (all of LDS), a
// ping-pong schedule in which each wavefront reads 12 fragments (16 bytes per
// lane) from LDS, meets a barrier, issues 32 independent
// v_mfma_f32_16x16x32_bf16 from registers (in the GEMMs' serpentine order)
// and meets a barrier, with the second wavefront of every SIMD one phase
// behind the first.  LDS holds either random bf16 values (random mantissas and signs, exponents 2^-4..2^3) or
// constant ones.  On MI355X the random case runs well below the nominal MFMA
// rate (power-limited clocks); its rate is the practical ceiling against
// which the GEMMs' MFMA utilisation is read.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"
#include "moe_bench.h"

namespace moe {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr int kLdsBytes = 160 * 1024;
constexpr int kFragRows = 64;   // LDS rows of 1 KB (64 lanes x 16 bytes) that the fragments cycle through

__global__ void __launch_bounds__(512, 1) mfma_ceiling_kernel(float* sink, int iters, int random_operands) {
  __shared__ __align__(16) uint4 lds[kLdsBytes / 16];
  for (int i = threadIdx.x; i < kFragRows * 64; i += blockDim.x) {
    uint32_t h[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t v = (uint32_t)(i * 4 + q + 12345) * 2654435761u;
      v ^= v >> 13;
      v *= 0x5bd1e995u;
      v ^= v >> 15;
      const uint32_t lo = (0x3d80u + (v & 0x3ffu)) | (((v >> 10) & 1u) << 15);
      const uint32_t hi = (0x3d80u + ((v >> 11) & 0x3ffu)) | (((v >> 21) & 1u) << 15);
      h[q] = random_operands ? ((lo & 0xffffu) | ((hi & 0xffffu) << 16)) : 0x3f803f80u;
    }
    lds[i] = make_uint4(h[0], h[1], h[2], h[3]);
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const bool second = wave >= 4;
  f32x4_t acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bf16x8_t w[8], x[4];
  if (second) __syncthreads();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = __builtin_bit_cast(bf16x8_t, lds[((it + i + wave) & (kFragRows - 1)) * 64 + lane]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x[j] = __builtin_bit_cast(bf16x8_t, lds[((it * 3 + j + 16) & (kFragRows - 1)) * 64 + lane]);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int j = (i & 1) ? 3 - jj : jj;   // serpentine, as the GEMMs issue them
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(w[i], x[j], acc[i][j], 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!second) __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) s += acc[i][j][0] + acc[i][j][3];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace moe

extern "C" int64_t moe_bench_mfma_flops(int64_t blocks, int32_t iters) {
  return blocks * 8 * (int64_t)iters * 32 * (2 * 16 * 16 * 32);
}

extern "C" moe_status_t moe_bench_mfma_ceiling(int32_t random_operands, int32_t iters, float* sink, int64_t blocks,
                                               void* stream) {
  if (!sink || blocks < 1 || blocks > (1 << 20) || iters < 1) return MOE_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(sink) & 3u) return MOE_ERR_ALIGNMENT;
  hipLaunchKernelGGL(moe::mfma_ceiling_kernel, dim3((unsigned)blocks), dim3(512), 0,
                     reinterpret_cast<hipStream_t>(stream), sink, iters, random_operands);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
