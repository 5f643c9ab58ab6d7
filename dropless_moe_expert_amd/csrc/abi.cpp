// C-ABI entry points of libmoe.so: host-side argument checks, then the
// kernel launches.  No allocation, no host<->device copies, no sync.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>

#include "moe.h"

// launchers (one per kernel family)
extern "C" {
moe_status_t moe_route_topk_launch(const float*, int64_t, int32_t, int32_t, int32_t, int32_t*, float*, uint32_t*,
                                   hipStream_t);
size_t moe_permute_ws_bytes_impl(int64_t, int32_t, int32_t);
int moe_route_fused_tokens(int32_t);
moe_status_t moe_route_fused_launch(const uint16_t*, const uint16_t*, const float*, int64_t, int32_t, int32_t, int32_t,
                                    int32_t, int32_t*, float*, float*, int32_t*, int32_t*, uint32_t*, hipStream_t);
moe_status_t moe_permute_routed_launch(const uint16_t*, const int32_t*, int64_t, int32_t, int32_t, int32_t, int32_t,
                                       int32_t*, int32_t*, int32_t*, int32_t*, uint16_t*, void*, hipStream_t);
moe_status_t moe_permute_launch(const uint16_t*, const int32_t*, int64_t, int32_t, int32_t, int32_t, int32_t*,
                                int32_t*, int32_t*, int32_t*, uint16_t*, void*, uint32_t*, hipStream_t);
moe_status_t moe_permute_noalloc_launch(const uint16_t*, const int32_t*, int64_t, int32_t, int32_t, int32_t, int32_t*,
                                        int32_t*, int32_t*, int32_t*, uint16_t*, uint32_t*, hipStream_t);
moe_status_t moe_permute_mxfp8_launch(const uint16_t*, const int32_t*, int64_t, int32_t, int32_t, int32_t, int32_t*,
                                      int32_t*, int32_t*, int32_t*, uint8_t*, uint8_t*, void*, uint32_t*, hipStream_t);
moe_status_t moe_unpermute_combine_launch(const uint16_t*, const float*, const int32_t*, int64_t, int32_t, int32_t,
                                          uint16_t*, hipStream_t);
moe_status_t moe_combine_backward_launch(const uint16_t*, const uint16_t*, const float*, const int32_t*, int64_t,
                                         int32_t, int32_t, uint16_t*, float*, uint8_t*, uint8_t*, hipStream_t);
moe_status_t moe_swiglu_backward_launch(const uint16_t*, const uint16_t*, int64_t, int32_t, const int32_t*, int32_t,
                                        uint16_t*, hipStream_t);
moe_status_t mxfp8_quantize_transposed_launch(const uint16_t*, const uint16_t*, int64_t, int32_t, const int32_t*,
                                              int32_t, int64_t, uint8_t*, uint8_t*, uint8_t*, uint8_t*, uint32_t*,
                                              hipStream_t);
moe_status_t mxfp8_gather_quantize_launch(const uint16_t*, const int32_t*, const float*, int32_t, int64_t, int32_t,
                                          const int32_t*, int32_t, int64_t, uint8_t*, uint8_t*, uint8_t*, uint8_t*,
                                          uint32_t*, hipStream_t);
moe_status_t mxfp4_quantize_launch(const uint16_t*, int64_t, int32_t, uint8_t*, uint8_t*, hipStream_t);
moe_status_t mxfp8_group_quantize_launch(const uint16_t*, int64_t, int32_t, int32_t, const int32_t*, int32_t,
                                         uint8_t*, uint8_t*, uint32_t*, hipStream_t);
moe_status_t grouped_gemm_launch(const moe_gg_desc*, const void*, const uint8_t*, const void*, const uint8_t*,
                                 const int32_t*, void*, void*, void*, size_t, uint32_t*, hipStream_t);
size_t grouped_gemm_ws_bytes_impl(const moe_gg_desc*);
}

namespace moe {  // gg_fwd.hip
size_t packed_weight_bytes(int G, int N, int K, int epilogue);
moe_status_t launch_pack_weights(const uint16_t* w, int G, int N, int K, int epilogue, void* out, hipStream_t s);
size_t packed_mx_weight_bytes(int G, int N, int K, int epilogue);   // gg_fwd_mx.hip
moe_status_t launch_pack_mx_weights(const uint8_t* q, const uint8_t* sc, int G, int N, int K, int epilogue, void* out,
                                    hipStream_t s);
}  // namespace moe

namespace moe_host {

// CU count per device, read once per device (the only global state).
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

}  // namespace moe_host

namespace {

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// T * K <= INT32_MAX (T >= 0, K >= 1), without forming a product that could overflow
inline bool pairs_fit(int64_t T, int32_t K) { return T <= INT32_MAX / K; }
// k_cap >= rows + 63 G, without forming a sum that could overflow (G <= 1024)
inline bool kcap_fits(int64_t k_cap, int64_t rows, int32_t G) { return k_cap - 63 * (int64_t)G >= rows; }
inline hipStream_t S(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape, dtype or layout";
    case MOE_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

moe_status_t moe_route_topk(const float* logits, int64_t T, int32_t E, int32_t K, int32_t renormalize,
                            int32_t* topk_ids, float* topk_w, uint32_t* err_flag, void* stream) {
  if (T < 0 || E < 1 || E > 256 || K < 1 || K > E || K > 32) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!logits || !topk_ids || !topk_w)) return MOE_ERR_INVALID_ARG;
  return moe_route_topk_launch(logits, T, E, K, renormalize, topk_ids, topk_w, err_flag, S(stream));
}

size_t moe_permute_workspace_bytes(int64_t T, int32_t E, int32_t K) {
  if (T < 0 || E < 1 || E > 256 || K < 1 || K > 32 || !pairs_fit(T, K)) return 0;
  return moe_permute_ws_bytes_impl(T, E, K);
}

moe_status_t moe_permute(const uint16_t* x, const int32_t* topk_ids, int64_t T, int32_t d, int32_t E, int32_t K,
                         int32_t* group_sizes, int32_t* group_offsets, int32_t* perm_src, int32_t* perm_dst,
                         uint16_t* x_perm, void* ws, size_t ws_bytes, uint32_t* err_flag, void* stream) {
  if (T < 0 || E < 1 || E > 256 || K < 1 || K > 32 || K > E) return MOE_ERR_INVALID_ARG;
  if (!pairs_fit(T, K)) return MOE_ERR_UNSUPPORTED;
  if (!group_sizes || !group_offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !perm_src || !perm_dst)) return MOE_ERR_INVALID_ARG;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARG;
  if (x) {
    if (d < 8 || d % 8) return MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_ALIGNMENT;
  }
  const size_t need = moe_permute_ws_bytes_impl(T, E, K);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return MOE_ERR_ALIGNMENT;
  return moe_permute_launch(x, topk_ids, T, d, E, K, group_sizes, group_offsets, perm_src, perm_dst, x_perm, ws,
                            err_flag, S(stream));
}

moe_status_t moe_permute_noalloc(const uint16_t* x, const int32_t* topk_ids, int64_t T, int32_t d, int32_t E,
                                 int32_t K, int32_t* group_sizes, int32_t* group_offsets, int32_t* perm_src,
                                 int32_t* perm_dst, uint16_t* x_perm, uint32_t* err_flag, void* stream) {
  if (T < 0 || E < 1 || E > 256 || K < 1 || K > 32 || K > E) return MOE_ERR_INVALID_ARG;
  if (!pairs_fit(T, K)) return MOE_ERR_UNSUPPORTED;
  if (!group_sizes || !group_offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !perm_src || !perm_dst)) return MOE_ERR_INVALID_ARG;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARG;
  if (x) {
    if (d < 8 || d % 8) return MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_ALIGNMENT;
  }
  if (moe_permute_ws_bytes_impl(T, E, K) > MOE_PERMUTE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  return moe_permute_noalloc_launch(x, topk_ids, T, d, E, K, group_sizes, group_offsets, perm_src, perm_dst, x_perm,
                                    err_flag, S(stream));
}

moe_status_t moe_permute_mxfp8(const uint16_t* x, const int32_t* topk_ids, int64_t T, int32_t d, int32_t E,
                               int32_t K, int32_t* group_sizes, int32_t* group_offsets, int32_t* perm_src,
                               int32_t* perm_dst, uint8_t* x_q, uint8_t* x_scale, void* ws, size_t ws_bytes,
                               uint32_t* err_flag, void* stream) {
  if (T < 0 || E < 1 || E > 256 || K < 1 || K > 32 || K > E) return MOE_ERR_INVALID_ARG;
  if (!pairs_fit(T, K)) return MOE_ERR_UNSUPPORTED;
  if (!group_sizes || !group_offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !perm_src || !perm_dst || !x || !x_q || !x_scale)) return MOE_ERR_INVALID_ARG;
  if (d < 32 || d % 32) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!aligned16(x) || !aligned16(x_q))) return MOE_ERR_ALIGNMENT;
  const size_t need = moe_permute_ws_bytes_impl(T, E, K);
  if (!ws || ws_bytes < need) return MOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return MOE_ERR_ALIGNMENT;
  return moe_permute_mxfp8_launch(x, topk_ids, T, d, E, K, group_sizes, group_offsets, perm_src, perm_dst, x_q,
                                  x_scale, ws, err_flag, S(stream));
}

static size_t route_fused_ws_bytes(int64_t T, int32_t E, int32_t K) {
  const int64_t tw = moe_route_fused_tokens(E);
  const int64_t nchunk = (T + tw - 1) / tw;
  const size_t a = ((size_t)(T * K) * 4 + 255) & ~(size_t)255;
  return a + ((((size_t)nchunk * E * 4) + 255) & ~(size_t)255);
}

size_t moe_route_fused_workspace_bytes(int64_t T, int32_t E, int32_t K) {
  if (T < 0 || E < 1 || E > 256 || K < 1 || K > 32 || !pairs_fit(T, K)) return 0;
  return route_fused_ws_bytes(T, E, K);
}

moe_status_t moe_route_fused(const uint16_t* x, const uint16_t* w_router, const float* bias, int64_t T, int32_t d,
                             int32_t E, int32_t K, int32_t renormalize, int32_t* topk_ids, float* topk_w,
                             float* logits, void* ws, size_t ws_bytes, uint32_t* err_flag, void* stream) {
  if (T < 0 || E < 1 || E > 256 || K < 1 || K > E || K > 32) return MOE_ERR_INVALID_ARG;
  if (!pairs_fit(T, K)) return MOE_ERR_UNSUPPORTED;
  if (d < 32 || d % 32 || (int64_t)d * 2 * 255 > (int64_t)UINT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!x || !w_router || !topk_ids || !topk_w)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(x) || !aligned16(w_router) || (logits && !aligned16(logits)))) return MOE_ERR_ALIGNMENT;
  int32_t* lr = nullptr;
  int32_t* cc = nullptr;
  if (ws) {
    if (ws_bytes < route_fused_ws_bytes(T, E, K)) return MOE_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return MOE_ERR_ALIGNMENT;
    lr = reinterpret_cast<int32_t*>(ws);
    cc = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + (((size_t)(T * K) * 4 + 255) & ~(size_t)255));
  }
  return moe_route_fused_launch(x, w_router, bias, T, d, E, K, renormalize, topk_ids, topk_w, logits, lr, cc,
                                err_flag, S(stream));
}

moe_status_t moe_permute_routed(const uint16_t* x, const int32_t* topk_ids, int64_t T, int32_t d, int32_t E,
                                int32_t K, int32_t* group_sizes, int32_t* group_offsets, int32_t* perm_src,
                                int32_t* perm_dst, uint16_t* x_perm, void* ws, size_t ws_bytes, uint32_t* err_flag,
                                void* stream) {
  (void)err_flag;
  if (T < 0 || E < 1 || E > 256 || K < 1 || K > 32 || K > E) return MOE_ERR_INVALID_ARG;
  if (!pairs_fit(T, K)) return MOE_ERR_UNSUPPORTED;
  if (!group_sizes || !group_offsets) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!topk_ids || !perm_src || !perm_dst)) return MOE_ERR_INVALID_ARG;
  if ((x == nullptr) != (x_perm == nullptr)) return MOE_ERR_INVALID_ARG;
  if (x) {
    if (d < 8 || d % 8) return MOE_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(x_perm)) return MOE_ERR_ALIGNMENT;
  }
  if (!ws || ws_bytes < route_fused_ws_bytes(T, E, K)) return MOE_ERR_WORKSPACE;
  if (reinterpret_cast<uintptr_t>(ws) & 255u) return MOE_ERR_ALIGNMENT;
  return moe_permute_routed_launch(x, topk_ids, T, d, E, K, moe_route_fused_tokens(E), group_sizes, group_offsets,
                                   perm_src, perm_dst, x_perm, ws, S(stream));
}

moe_status_t mxfp4_quantize(const uint16_t* x, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                            void* stream) {
  if (rows < 0 || cols < 128 || cols % 128) return rows < 0 ? MOE_ERR_INVALID_ARG : MOE_ERR_UNSUPPORTED;
  if (rows == 0) return MOE_OK;
  if (!x || !codes || !scales) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(codes)) return MOE_ERR_ALIGNMENT;
  return mxfp4_quantize_launch(x, rows, cols, codes, scales, S(stream));
}

size_t grouped_gemm_workspace_bytes(const moe_gg_desc* desc) {
  if (!desc) return 0;
  return grouped_gemm_ws_bytes_impl(desc);
}

moe_status_t grouped_gemm(const moe_gg_desc* d, const void* A, const uint8_t* A_scale, const void* B,
                          const uint8_t* B_scale, const int32_t* group_sizes, void* C, void* C_aux, void* ws,
                          size_t ws_bytes, uint32_t* err_flag, void* stream) {
  if (!d) return MOE_ERR_INVALID_ARG;
  if (d->G < 1 || d->G > 1024 || d->N < 1 || d->m_cap < 0) return MOE_ERR_INVALID_ARG;
  if (d->m_cap > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  // a 256-row output tile is addressed by 32-bit offsets from its first row
  if (d->N > (1 << 22)) return MOE_ERR_UNSUPPORTED;
  if (!A || !B || !C || !group_sizes) return MOE_ERR_INVALID_ARG;
  if (!aligned16(A) || !aligned16(B) || !aligned16(C)) return MOE_ERR_ALIGNMENT;
  if (C_aux && d->epilogue != MOE_EPI_SWIGLU_MXFP8 && !aligned16(C_aux)) return MOE_ERR_ALIGNMENT;
  if (d->dtype != MOE_DTYPE_BF16 && d->dtype != MOE_DTYPE_MXFP8 && d->dtype != MOE_DTYPE_MXFP4)
    return MOE_ERR_UNSUPPORTED;
  if (d->dtype == MOE_DTYPE_MXFP4) {
    if (d->ragged != MOE_RAGGED_M || d->b_layout != MOE_B_NK || d->out_dtype != MOE_OUT_BF16) return MOE_ERR_UNSUPPORTED;
    if (d->epilogue != MOE_EPI_NONE && d->epilogue != MOE_EPI_SWIGLU) return MOE_ERR_UNSUPPORTED;
    if (d->K < 128 || d->K % 128) return MOE_ERR_UNSUPPORTED;
    if (d->epilogue == MOE_EPI_SWIGLU && (d->N / 2) % 8) return MOE_ERR_UNSUPPORTED;
    if (C_aux || !A_scale || !B_scale) return MOE_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(A_scale) & 3u) || (reinterpret_cast<uintptr_t>(B_scale) & 3u))
      return MOE_ERR_ALIGNMENT;
    if (d->N % 8) return MOE_ERR_UNSUPPORTED;
    if (d->m_cap == 0) return MOE_OK;
    return grouped_gemm_launch(d, A, A_scale, B, B_scale, group_sizes, C, C_aux, ws, ws_bytes, err_flag, S(stream));
  }
  if (d->out_dtype != MOE_OUT_BF16 && d->out_dtype != MOE_OUT_F32) return MOE_ERR_UNSUPPORTED;
  if (d->epilogue != MOE_EPI_NONE && d->epilogue != MOE_EPI_SWIGLU && d->epilogue != MOE_EPI_SWIGLU_MXFP8 &&
      d->epilogue != MOE_EPI_SWIGLU_BWD)
    return MOE_ERR_UNSUPPORTED;
  if (d->N % 8) return MOE_ERR_UNSUPPORTED;
  if (d->ragged == MOE_RAGGED_M) {
    if (d->K < 1) return MOE_ERR_INVALID_ARG;
    if (d->b_layout != MOE_B_NK && d->b_layout != MOE_B_KN && d->b_layout != MOE_B_PACKED) return MOE_ERR_UNSUPPORTED;
    if (d->epilogue == MOE_EPI_SWIGLU) {
      if (d->b_layout == MOE_B_KN || d->out_dtype != MOE_OUT_BF16 || (d->N / 2) % 8) return MOE_ERR_UNSUPPORTED;
    } else if (d->epilogue == MOE_EPI_SWIGLU_MXFP8) {
      // codes to C, scales to C_aux (1-byte elements: 4-byte aligned rows of codes)
      if (d->dtype != MOE_DTYPE_MXFP8 || d->out_dtype != MOE_OUT_BF16 || (d->N / 2) % 32) return MOE_ERR_UNSUPPORTED;
      if (!C_aux) return MOE_ERR_INVALID_ARG;
    } else if (d->epilogue == MOE_EPI_SWIGLU_BWD) {
      // dgu to C [m_cap, 2N] from the pre-activations in C_aux [m_cap, 2N]
      // (its row pitch is 2N: 256 rows of it stay within 32-bit byte offsets)
      if (d->dtype != MOE_DTYPE_BF16 || d->b_layout != MOE_B_KN || d->out_dtype != MOE_OUT_BF16 ||
          d->N > (1 << 21))
        return MOE_ERR_UNSUPPORTED;
      if (!C_aux) return MOE_ERR_INVALID_ARG;
    } else if (C_aux) {
      return MOE_ERR_INVALID_ARG;
    }
    if (d->dtype == MOE_DTYPE_MXFP8) {
      if (d->K % 128 || d->b_layout == MOE_B_KN || d->out_dtype != MOE_OUT_BF16) return MOE_ERR_UNSUPPORTED;
      const bool packed = d->b_layout == MOE_B_PACKED;   // the weight scales travel inside the packed B
      if (!A_scale || (!packed && !B_scale)) return MOE_ERR_INVALID_ARG;
      if ((reinterpret_cast<uintptr_t>(A_scale) & 3u) || (!packed && (reinterpret_cast<uintptr_t>(B_scale) & 3u)))
        return MOE_ERR_ALIGNMENT;
    } else {
      if (d->K % 64) return MOE_ERR_UNSUPPORTED;
      if (d->b_layout == MOE_B_KN && d->N < 8) return MOE_ERR_UNSUPPORTED;
    }
    if (d->m_cap == 0) return MOE_OK;
  } else if (d->ragged == MOE_RAGGED_K) {
    if (d->epilogue != MOE_EPI_NONE || C_aux) return MOE_ERR_UNSUPPORTED;
    if (d->M < 8 || d->M % 8) return MOE_ERR_UNSUPPORTED;
    if (d->dtype == MOE_DTYPE_MXFP8) {
      // operands laid out by mxfp8_quantize_transposed: K = its k_cap
      if (d->out_dtype != MOE_OUT_BF16) return MOE_ERR_UNSUPPORTED;
      if (d->K < 64 || d->K % 64 || !kcap_fits(d->K, d->m_cap, d->G)) return MOE_ERR_INVALID_ARG;
      if (!A_scale || !B_scale) return MOE_ERR_INVALID_ARG;
      if ((reinterpret_cast<uintptr_t>(A_scale) & 3u) || (reinterpret_cast<uintptr_t>(B_scale) & 3u))
        return MOE_ERR_ALIGNMENT;
    }
  } else {
    return MOE_ERR_UNSUPPORTED;
  }
  return grouped_gemm_launch(d, A, A_scale, B, B_scale, group_sizes, C, C_aux, ws, ws_bytes, err_flag, S(stream));
}

size_t moe_pack_weights_bytes(int32_t G, int32_t N, int32_t K, int32_t epilogue) {
  if (G < 1 || G > 1024 || N < 8 || N % 8 || K < 64 || K % 64) return 0;
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SWIGLU) return 0;
  if (epilogue == MOE_EPI_SWIGLU && (N / 2) % 8) return 0;
  return moe::packed_weight_bytes(G, N, K, epilogue);
}

moe_status_t moe_pack_weights(const uint16_t* w, int32_t G, int32_t N, int32_t K, int32_t epilogue, void* out,
                              size_t out_bytes, void* stream) {
  const size_t need = moe_pack_weights_bytes(G, N, K, epilogue);
  if (need == 0) return MOE_ERR_UNSUPPORTED;
  if (!w || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(out)) return MOE_ERR_ALIGNMENT;
  if (out_bytes < need) return MOE_ERR_WORKSPACE;
  return moe::launch_pack_weights(w, G, N, K, epilogue, out, S(stream));
}

size_t moe_pack_weights_mxfp8_bytes(int32_t G, int32_t N, int32_t K, int32_t epilogue) {
  if (G < 1 || G > 1024 || N < 8 || N % 8 || K < 128 || K % 128) return 0;
  if (epilogue != MOE_EPI_NONE && epilogue != MOE_EPI_SWIGLU) return 0;
  if (epilogue == MOE_EPI_SWIGLU && (N / 2) % 8) return 0;
  return moe::packed_mx_weight_bytes(G, N, K, epilogue);
}

moe_status_t moe_pack_weights_mxfp8(const uint8_t* q, const uint8_t* scale, int32_t G, int32_t N, int32_t K,
                                    int32_t epilogue, void* out, size_t out_bytes, void* stream) {
  const size_t need = moe_pack_weights_mxfp8_bytes(G, N, K, epilogue);
  if (need == 0) return MOE_ERR_UNSUPPORTED;
  if (!q || !scale || !out) return MOE_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || (reinterpret_cast<uintptr_t>(scale) & 1u)) return MOE_ERR_ALIGNMENT;
  if (out_bytes < need) return MOE_ERR_WORKSPACE;
  return moe::launch_pack_mx_weights(q, scale, G, N, K, epilogue, out, S(stream));
}

moe_status_t moe_unpermute_combine(const uint16_t* y_perm, const float* topk_w, const int32_t* perm_dst, int64_t T,
                                   int32_t d, int32_t K, uint16_t* y, void* stream) {
  if (T < 0 || K < 1 || K > 32 || d < 8 || d % 8) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!y_perm || !perm_dst || !y)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(y_perm) || !aligned16(y))) return MOE_ERR_ALIGNMENT;
  return moe_unpermute_combine_launch(y_perm, topk_w, perm_dst, T, d, K, y, S(stream));
}

moe_status_t moe_combine_backward(const uint16_t* dy, const uint16_t* y_perm, const float* topk_w,
                                  const int32_t* perm_dst, int64_t T, int32_t d, int32_t K, uint16_t* dy_perm,
                                  float* d_topk_w, void* stream) {
  if (T < 0 || K < 1 || K > 32 || d < 8 || d % 8) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!dy || !y_perm || !topk_w || !perm_dst || !d_topk_w)) return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(dy) || !aligned16(y_perm) || (dy_perm && !aligned16(dy_perm)))) return MOE_ERR_ALIGNMENT;
  return moe_combine_backward_launch(dy, y_perm, topk_w, perm_dst, T, d, K, dy_perm, d_topk_w, nullptr, nullptr,
                                     S(stream));
}

moe_status_t moe_combine_backward_mxfp8(const uint16_t* dy, const uint16_t* y_perm, const float* topk_w,
                                        const int32_t* perm_dst, int64_t T, int32_t d, int32_t K, uint8_t* q_rows,
                                        uint8_t* scale_rows, float* d_topk_w, void* stream) {
  if (T < 0 || K < 1 || K > 32 || d < 32) return MOE_ERR_INVALID_ARG;
  if (d % 32) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!dy || !y_perm || !topk_w || !perm_dst || !q_rows || !scale_rows || !d_topk_w))
    return MOE_ERR_INVALID_ARG;
  if (T > 0 && (!aligned16(dy) || !aligned16(y_perm) || (reinterpret_cast<uintptr_t>(q_rows) & 7u)))
    return MOE_ERR_ALIGNMENT;
  return moe_combine_backward_launch(dy, y_perm, topk_w, perm_dst, T, d, K, nullptr, d_topk_w, q_rows, scale_rows,
                                     S(stream));
}

moe_status_t moe_swiglu_backward(const uint16_t* gu, const uint16_t* dh, int64_t m_cap, int32_t f,
                                 const int32_t* group_sizes, int32_t G, uint16_t* dgu, void* stream) {
  if (m_cap < 0 || f < 8 || f % 8) return MOE_ERR_INVALID_ARG;
  if (group_sizes && (G < 1 || G > 1024)) return MOE_ERR_INVALID_ARG;
  if (m_cap > 0 && (!gu || !dh || !dgu)) return MOE_ERR_INVALID_ARG;
  if (m_cap > 0 && (!aligned16(gu) || !aligned16(dh) || !aligned16(dgu))) return MOE_ERR_ALIGNMENT;
  return moe_swiglu_backward_launch(gu, dh, m_cap, f, group_sizes, G, dgu, S(stream));
}

moe_status_t mxfp8_group_quantize(const uint16_t* x, int64_t rows, int32_t cols, int32_t axis,
                                  const int32_t* group_sizes, int32_t G, uint8_t* q, uint8_t* scale,
                                  uint32_t* err_flag, void* stream) {
  if (rows < 0 || cols < 8) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!x || !q || !scale)) return MOE_ERR_INVALID_ARG;
  if (axis == 0) {
    if (cols % 32) return MOE_ERR_UNSUPPORTED;
    if (group_sizes && (G < 1 || G > 1024)) return MOE_ERR_INVALID_ARG;
    if (rows > 0 && (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u))) return MOE_ERR_ALIGNMENT;
  } else if (axis == 1) {
    if (!group_sizes || G < 1 || G > 1024) return MOE_ERR_INVALID_ARG;
    if (cols % 8) return MOE_ERR_UNSUPPORTED;
    if (rows > 0 && (!aligned16(x) || (reinterpret_cast<uintptr_t>(q) & 7u) ||
                     (reinterpret_cast<uintptr_t>(scale) & 7u)))
      return MOE_ERR_ALIGNMENT;
  } else {
    return MOE_ERR_INVALID_ARG;
  }
  return mxfp8_group_quantize_launch(x, rows, cols, axis, group_sizes, G, q, scale, err_flag, S(stream));
}

moe_status_t mxfp8_quantize_transposed(const uint16_t* x, int64_t rows, int32_t cols, const int32_t* group_sizes,
                                       int32_t G, int64_t k_cap, uint8_t* qT, uint8_t* scaleT, uint8_t* q_rows,
                                       uint8_t* scale_rows, uint32_t* err_flag, void* stream) {
  if (rows < 0 || cols < 8 || G < 1 || G > 1024) return MOE_ERR_INVALID_ARG;
  if (cols % 8) return MOE_ERR_UNSUPPORTED;
  if (group_sizes) {
    if (k_cap < 0 || k_cap % 64 || !kcap_fits(k_cap, rows, G)) return MOE_ERR_INVALID_ARG;
  } else if (rows % 64) {
    return MOE_ERR_UNSUPPORTED;
  }
  if (rows > 0 && (!x || !qT || !scaleT)) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!aligned16(x) || !aligned16(qT) || (reinterpret_cast<uintptr_t>(scaleT) & 1u)))
    return MOE_ERR_ALIGNMENT;
  if (!q_rows != !scale_rows) return MOE_ERR_INVALID_ARG;
  if (q_rows) {
    if (cols % 32) return MOE_ERR_UNSUPPORTED;
    if (rows > 0 && !aligned16(q_rows)) return MOE_ERR_ALIGNMENT;
  }
  if (rows == 0) return MOE_OK;
  return mxfp8_quantize_transposed_launch(x, nullptr, rows, cols, group_sizes, G, k_cap, qT, scaleT, q_rows,
                                          scale_rows, err_flag, S(stream));
}

moe_status_t mxfp8_quantize_gathered(const uint16_t* x, const int32_t* perm_src, const float* topk_w, int64_t T,
                                     int32_t K, int32_t cols, const int32_t* group_sizes, int32_t G, int64_t k_cap,
                                     uint8_t* qT, uint8_t* scaleT, uint8_t* q_rows, uint8_t* scale_rows,
                                     uint32_t* err_flag, void* stream) {
  if (T < 0 || K < 1 || K > 32 || !pairs_fit(T, K) || cols < 8 || !group_sizes || G < 1 || G > 1024)
    return MOE_ERR_INVALID_ARG;
  if (cols % 8) return MOE_ERR_UNSUPPORTED;
  const int64_t rows = T * K;
  if (k_cap < 0 || k_cap % 64 || !kcap_fits(k_cap, rows, G)) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!x || !perm_src || !qT || !scaleT)) return MOE_ERR_INVALID_ARG;
  if (rows > 0 && (!aligned16(x) || !aligned16(qT) || (reinterpret_cast<uintptr_t>(scaleT) & 1u)))
    return MOE_ERR_ALIGNMENT;
  if (!q_rows != !scale_rows) return MOE_ERR_INVALID_ARG;
  if (q_rows) {
    if (cols % 32) return MOE_ERR_UNSUPPORTED;
    if (rows > 0 && !aligned16(q_rows)) return MOE_ERR_ALIGNMENT;
  }
  if (rows == 0) return MOE_OK;
  return mxfp8_gather_quantize_launch(x, perm_src, topk_w, K, rows, cols, group_sizes, G, k_cap, qT, scaleT, q_rows,
                                      scale_rows, err_flag, S(stream));
}

moe_status_t moe_swiglu_backward_mxfp8(const uint16_t* gu, const uint16_t* dh, int64_t m_cap, int32_t f,
                                       const int32_t* group_sizes, int32_t G, int64_t k_cap, uint8_t* qT,
                                       uint8_t* scaleT, uint8_t* q_rows, uint8_t* scale_rows, uint32_t* err_flag,
                                       void* stream) {
  if (m_cap < 0 || f < 16 || f % 16 || !group_sizes || G < 1 || G > 1024) return MOE_ERR_INVALID_ARG;
  if (k_cap < 0 || k_cap % 64 || !kcap_fits(k_cap, m_cap, G)) return MOE_ERR_INVALID_ARG;
  if (m_cap > 0 && (!gu || !dh || !qT || !scaleT || !q_rows || !scale_rows)) return MOE_ERR_INVALID_ARG;
  if (m_cap > 0 && (!aligned16(gu) || !aligned16(dh) || !aligned16(qT) || !aligned16(q_rows) ||
                    (reinterpret_cast<uintptr_t>(scaleT) & 1u)))
    return MOE_ERR_ALIGNMENT;
  if (m_cap == 0) return MOE_OK;
  return mxfp8_quantize_transposed_launch(gu, dh, m_cap, 2 * f, group_sizes, G, k_cap, qT, scaleT, q_rows,
                                          scale_rows, err_flag, S(stream));
}

}  // extern "C"
