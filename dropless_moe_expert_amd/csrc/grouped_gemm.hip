// Dispatch of grouped_gemm to its kernels.
//
// Page "NVIDIA Accelerates Dropless MoE Training in JAX Using Transformer
// Engine", section "Optimization 1: Grouped GEMM": every expert's matmul in
// one kernel call, each with its true token count, computing only the
// regions with valid tokens, with no device-to-host copy of the counts
// (which would break graph capture); MXFP8 block scaling for the expert
// matmuls.  Section "What specialized optimizations are required for
// dropless MoE?": the counts may be invisible to the CPU.
//
//  * ragged M, bf16 (forward with B [G, N, K] rows or packed, data gradient
//    with B [G, K, N]): gg_bf16.hip, gg_fwd_kernel (with the caller's
//    workspace, the tiles of a short last round split along K);
//  * ragged K, bf16 (weight gradients): gg_bf16.hip, gg_wgrad_kernel;
//  * ragged M, MXFP8: gg_fwd_mx.hip, gg_fwd_mx_kernel (split tail as bf16);
//  * ragged K, MXFP8 (operands from mxfp8_quantize_transposed): gg_fwd_mx.hip,
//    gg_wgrad_mx_kernel.
// Every grid is a function of host arguments only (CU count, m_cap, G, N, K).
#include "gg_common.h"

namespace moe {
moe_status_t launch_fwd(const GGArgs& a, int epilogue, int out_f32, int b_layout, hipStream_t s);  // gg_bf16.hip
moe_status_t launch_wgrad(const GGArgs& a, int out_f32, hipStream_t s);                             // gg_bf16.hip
moe_status_t launch_fwd_mx(const GGArgs& a, int epilogue, int packed, hipStream_t s);              // gg_fwd_mx.hip
moe_status_t launch_wgrad_mx(const GGArgs& a, hipStream_t s);                                       // gg_fwd_mx.hip
moe_status_t launch_fwd_mx4(const GGArgs& a, int epilogue, hipStream_t s);                          // gg_mx4.hip
size_t fwd_split_workspace_bytes();                                                                  // gg_bf16.hip
}  // namespace moe

// The workspace a call can use: the bf16 and MXFP8 ragged-M kernels' split tail
extern "C" size_t grouped_gemm_ws_bytes_impl(const moe_gg_desc* d) {
  if (d->ragged == MOE_RAGGED_M && (d->dtype == MOE_DTYPE_BF16 || d->dtype == MOE_DTYPE_MXFP8))
    return moe::fwd_split_workspace_bytes();
  return 0;
}

extern "C" moe_status_t grouped_gemm_launch(const moe_gg_desc* d, const void* A, const uint8_t* As, const void* B,
                                            const uint8_t* Bs, const int32_t* sizes, void* C, void* Caux,
                                            void* ws, size_t ws_bytes, uint32_t* flag, hipStream_t s) {
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
  a.n_tiles = 0;
  a.p_tiles = 0;
  a.sched_slot = 0;
  a.sched_epoch = a.sched_next = 0;
  // the split tail runs only with the whole workspace, 256-byte aligned
  const size_t need = grouped_gemm_ws_bytes_impl(d);
  a.part = (need && ws && ws_bytes >= need && !(reinterpret_cast<uintptr_t>(ws) & 255u)) ? reinterpret_cast<float*>(ws)
                                                                                         : nullptr;
  if (d->ragged == MOE_RAGGED_M) {
    if (d->dtype == MOE_DTYPE_MXFP8) return launch_fwd_mx(a, d->epilogue, d->b_layout == MOE_B_PACKED, s);
    if (d->dtype == MOE_DTYPE_MXFP4) return launch_fwd_mx4(a, d->epilogue, s);
    return launch_fwd(a, d->epilogue, d->out_dtype == MOE_OUT_F32, d->b_layout, s);
  }
  if (d->dtype == MOE_DTYPE_MXFP8) return launch_wgrad_mx(a, s);
  return launch_wgrad(a, d->out_dtype == MOE_OUT_F32, s);
}
