// Host-side checks of the C ABI under AddressSanitizer and
// UndefinedBehaviorSanitizer, on the CPU: abi.cpp linked against stub
// launchers, so that every argument check runs and no kernel is launched.
// Each call states the status it must return; a valid call must reach its
// launcher exactly once, an invalid one never.  Sizes at the ends of their
// types check that no size arithmetic overflows.
#include <cinttypes>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include <hip/hip_runtime.h>

#include "moe.h"

static int g_launches = 0;
static moe_status_t launched() {
  ++g_launches;
  return MOE_OK;
}

extern "C" {
moe_status_t moe_route_topk_launch(const float*, int64_t, int32_t, int32_t, int32_t, int32_t*, float*, uint32_t*,
                                   hipStream_t) { return launched(); }
size_t moe_permute_ws_bytes_impl(int64_t T, int32_t E, int32_t K) {
  // the library's formula (per-pair ranks, per-chunk counts, 256-byte aligned)
  const int64_t M = T * K, nchunk = (M + 255) / 256;
  return (((size_t)M * 4 + 255) & ~(size_t)255) + (((size_t)nchunk * E * 4 + 255) & ~(size_t)255);
}
int moe_route_fused_tokens(int32_t E) { return E <= 32 ? 16 : E <= 64 ? 32 : 64; }
moe_status_t moe_route_fused_launch(const uint16_t*, const uint16_t*, const float*, int64_t, int32_t, int32_t, int32_t,
                                    int32_t, int32_t*, float*, float*, int32_t*, int32_t*, uint32_t*,
                                    hipStream_t) { return launched(); }
moe_status_t moe_permute_routed_launch(const uint16_t*, const int32_t*, int64_t, int32_t, int32_t, int32_t, int32_t,
                                       int32_t*, int32_t*, int32_t*, int32_t*, uint16_t*, void*,
                                       hipStream_t) { return launched(); }
moe_status_t moe_permute_launch(const uint16_t*, const int32_t*, int64_t, int32_t, int32_t, int32_t, int32_t*,
                                int32_t*, int32_t*, int32_t*, uint16_t*, void*, uint32_t*,
                                hipStream_t) { return launched(); }
moe_status_t moe_permute_noalloc_launch(const uint16_t*, const int32_t*, int64_t, int32_t, int32_t, int32_t, int32_t*,
                                        int32_t*, int32_t*, int32_t*, uint16_t*, uint32_t*,
                                        hipStream_t) { return launched(); }
moe_status_t moe_permute_mxfp8_launch(const uint16_t*, const int32_t*, int64_t, int32_t, int32_t, int32_t, int32_t*,
                                      int32_t*, int32_t*, int32_t*, uint8_t*, uint8_t*, void*, uint32_t*,
                                      hipStream_t) { return launched(); }
moe_status_t moe_unpermute_combine_launch(const uint16_t*, const float*, const int32_t*, int64_t, int32_t, int32_t,
                                          uint16_t*, hipStream_t) { return launched(); }
moe_status_t moe_combine_backward_launch(const uint16_t*, const uint16_t*, const float*, const int32_t*, int64_t,
                                         int32_t, int32_t, uint16_t*, float*, uint8_t*, uint8_t*, hipStream_t) {
  return launched();
}
moe_status_t moe_swiglu_backward_launch(const uint16_t*, const uint16_t*, int64_t, int32_t, const int32_t*, int32_t,
                                        uint16_t*, hipStream_t) { return launched(); }
moe_status_t mxfp8_quantize_transposed_launch(const uint16_t*, const uint16_t*, int64_t, int32_t, const int32_t*,
                                              int32_t, int64_t, uint8_t*, uint8_t*, uint8_t*, uint8_t*, uint32_t*,
                                              hipStream_t) { return launched(); }
moe_status_t mxfp8_gather_quantize_launch(const uint16_t*, const int32_t*, const float*, int32_t, int64_t, int32_t,
                                          const int32_t*, int32_t, int64_t, uint8_t*, uint8_t*, uint8_t*, uint8_t*,
                                          uint32_t*, hipStream_t) { return launched(); }
moe_status_t mxfp4_quantize_launch(const uint16_t*, int64_t, int32_t, uint8_t*, uint8_t*, hipStream_t) {
  return launched();
}
moe_status_t mxfp8_group_quantize_launch(const uint16_t*, int64_t, int32_t, int32_t, const int32_t*, int32_t, uint8_t*,
                                         uint8_t*, uint32_t*, hipStream_t) { return launched(); }
moe_status_t grouped_gemm_launch(const moe_gg_desc*, const void*, const uint8_t*, const void*, const uint8_t*,
                                 const int32_t*, void*, void*, void*, size_t, uint32_t*, hipStream_t) {
  return launched();
}
// the library's rule: bf16 and MXFP8 ragged-M calls can use one fp32 256 x 256 tile per CU (256 CUs here)
size_t grouped_gemm_ws_bytes_impl(const moe_gg_desc* d) {
  return d->ragged == MOE_RAGGED_M && (d->dtype == MOE_DTYPE_BF16 || d->dtype == MOE_DTYPE_MXFP8)
             ? (size_t)256 * 256 * 256 * 4
             : 0;
}
}

namespace moe {
size_t packed_weight_bytes(int G, int N, int K, int) { return (size_t)G * N * K * 2; }
moe_status_t launch_pack_weights(const uint16_t*, int, int, int, int, void*, hipStream_t) { return launched(); }
size_t packed_mx_weight_bytes(int G, int N, int K, int) { return (size_t)G * N * K + (size_t)G * N * (K / 32); }
moe_status_t launch_pack_mx_weights(const uint8_t*, const uint8_t*, int, int, int, int, void*, hipStream_t) {
  return launched();
}
}  // namespace moe

static int g_fail = 0;
#define EXPECT(call, want)                                                                     \
  do {                                                                                         \
    const int before = g_launches;                                                             \
    const int got = (int)(call);                                                               \
    const bool launched_ok = (want) == MOE_OK ? g_launches == before + 1 : g_launches == before; \
    if (got != (int)(want) || !launched_ok) {                                                  \
      std::printf("FAIL line %d: %s -> %d (want %d), launches %d\n", __LINE__, #call, got, (int)(want), \
                  g_launches - before);                                                       \
      ++g_fail;                                                                                \
    }                                                                                          \
  } while (0)

int main() {
  // aligned stand-ins for device pointers (never dereferenced by the checks)
  alignas(256) static uint8_t buf[1 << 12];
  void* p = buf;
  auto* f = reinterpret_cast<float*>(buf);
  auto* i32 = reinterpret_cast<int32_t*>(buf);
  auto* u16 = reinterpret_cast<uint16_t*>(buf);
  auto* u8 = buf;
  auto* odd16 = reinterpret_cast<uint16_t*>(buf + 2);
  const int64_t BIG = INT64_MAX, HUGE_T = (int64_t)1 << 60;

  // router top-K
  EXPECT(moe_route_topk(f, 10, 8, 2, 1, i32, f, nullptr, nullptr), MOE_OK);
  EXPECT(moe_route_topk(f, 10, 8, 9, 1, i32, f, nullptr, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_topk(f, -1, 8, 2, 1, i32, f, nullptr, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_route_topk(f, BIG, 256, 32, 1, i32, f, nullptr, nullptr), MOE_OK);   // T is only a count here
  // permute: sizes at the ends of their types
  EXPECT(moe_permute(u16, i32, 16, 64, 8, 2, i32, i32, i32, i32, u16, p, 1 << 12, nullptr, nullptr), MOE_OK);
  EXPECT(moe_permute(u16, i32, HUGE_T, 64, 64, 32, i32, i32, i32, i32, u16, p, 1 << 12, nullptr, nullptr),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_permute(u16, i32, BIG, 64, 8, 8, i32, i32, i32, i32, u16, p, 1 << 12, nullptr, nullptr),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_permute(odd16, i32, 16, 64, 8, 2, i32, i32, i32, i32, u16, p, 1 << 12, nullptr, nullptr),
         MOE_ERR_ALIGNMENT);
  EXPECT(moe_permute(u16, i32, 16, 64, 8, 2, i32, i32, i32, i32, u16, p, 16, nullptr, nullptr), MOE_ERR_WORKSPACE);
  if (moe_permute_workspace_bytes(BIG, 256, 32) != 0 || moe_permute_workspace_bytes(HUGE_T, 8, 8) != 0) {
    std::printf("FAIL: workspace query of an unsupported size is not 0\n");
    ++g_fail;
  }
  if (moe_permute_workspace_bytes(16384, 128, 8) < 16384 * 8 * 4) {
    std::printf("FAIL: workspace query too small\n");
    ++g_fail;
  }
  EXPECT(moe_permute_noalloc(u16, i32, 16, 64, 8, 2, i32, i32, i32, i32, u16, nullptr, nullptr), MOE_OK);
  EXPECT(moe_permute_noalloc(u16, i32, BIG, 64, 8, 8, i32, i32, i32, i32, u16, nullptr, nullptr),
         MOE_ERR_UNSUPPORTED);
  EXPECT(moe_permute_noalloc(nullptr, i32, (1 << 17) + 32, 0, 256, 8, i32, i32, i32, i32, nullptr, nullptr, nullptr),
         MOE_ERR_WORKSPACE);
  EXPECT(moe_permute_mxfp8(u16, i32, 16, 64, 8, 2, i32, i32, i32, i32, u8, u8, p, 1 << 12, nullptr, nullptr), MOE_OK);
  EXPECT(moe_permute_mxfp8(u16, i32, BIG, 64, 8, 2, i32, i32, i32, i32, u8, u8, p, 1 << 12, nullptr, nullptr),
         MOE_ERR_UNSUPPORTED);
  // fused router and its permute
  const size_t rws = moe_route_fused_workspace_bytes(16, 8, 2);
  EXPECT(moe_route_fused(u16, u16, f, 16, 64, 8, 2, 1, i32, f, nullptr, p, rws, nullptr, nullptr), MOE_OK);
  EXPECT(moe_route_fused(u16, u16, f, HUGE_T, 64, 8, 2, 1, i32, f, nullptr, nullptr, 0, nullptr, nullptr),
         MOE_ERR_UNSUPPORTED);
  if (moe_route_fused_workspace_bytes(BIG, 256, 32) != 0) {
    std::printf("FAIL: fused-router workspace query of an unsupported size is not 0\n");
    ++g_fail;
  }
  EXPECT(moe_permute_routed(u16, i32, 16, 64, 8, 2, i32, i32, i32, i32, u16, p, rws, nullptr, nullptr), MOE_OK);
  EXPECT(moe_permute_routed(u16, i32, BIG, 64, 8, 2, i32, i32, i32, i32, u16, p, rws, nullptr, nullptr),
         MOE_ERR_UNSUPPORTED);
  // grouped GEMM descriptors
  moe_gg_desc d{};
  d = {MOE_DTYPE_BF16, MOE_RAGGED_M, MOE_B_NK, MOE_EPI_NONE, MOE_OUT_BF16, 4, 0, 64, 64, 100};
  EXPECT(grouped_gemm(&d, p, nullptr, p, nullptr, i32, p, nullptr, nullptr, 0, nullptr, nullptr), MOE_OK);
  d.m_cap = BIG;
  EXPECT(grouped_gemm(&d, p, nullptr, p, nullptr, i32, p, nullptr, nullptr, 0, nullptr, nullptr), MOE_ERR_UNSUPPORTED);
  d.m_cap = 100;
  d.N = 1 << 22;   // the widest output the 32-bit tile offsets address
  EXPECT(grouped_gemm(&d, p, nullptr, p, nullptr, i32, p, nullptr, nullptr, 0, nullptr, nullptr), MOE_OK);
  d.N = (1 << 22) + 8;
  EXPECT(grouped_gemm(&d, p, nullptr, p, nullptr, i32, p, nullptr, nullptr, 0, nullptr, nullptr), MOE_ERR_UNSUPPORTED);
  // SwiGLU backward in the data gradient's epilogue: bf16, B_KN, bf16 out, the pre-activations required
  d = {MOE_DTYPE_BF16, MOE_RAGGED_M, MOE_B_KN, MOE_EPI_SWIGLU_BWD, MOE_OUT_BF16, 4, 0, 1 << 21, 64, 100};
  EXPECT(grouped_gemm(&d, p, nullptr, p, nullptr, i32, p, p, nullptr, 0, nullptr, nullptr), MOE_OK);
  EXPECT(grouped_gemm(&d, p, nullptr, p, nullptr, i32, p, nullptr, nullptr, 0, nullptr, nullptr), MOE_ERR_INVALID_ARG);
  d.N = (1 << 21) + 8;   // a 2N row pitch past the 32-bit tile offsets
  EXPECT(grouped_gemm(&d, p, nullptr, p, nullptr, i32, p, p, nullptr, 0, nullptr, nullptr), MOE_ERR_UNSUPPORTED);
  d.N = 64;
  d.b_layout = MOE_B_NK;
  EXPECT(grouped_gemm(&d, p, nullptr, p, nullptr, i32, p, p, nullptr, 0, nullptr, nullptr), MOE_ERR_UNSUPPORTED);
  d.b_layout = MOE_B_KN;
  d.out_dtype = MOE_OUT_F32;
  EXPECT(grouped_gemm(&d, p, nullptr, p, nullptr, i32, p, p, nullptr, 0, nullptr, nullptr), MOE_ERR_UNSUPPORTED);
  d.out_dtype = MOE_OUT_BF16;
  d.dtype = MOE_DTYPE_MXFP8;
  EXPECT(grouped_gemm(&d, p, u8, p, u8, i32, p, p, nullptr, 0, nullptr, nullptr), MOE_ERR_UNSUPPORTED);
  d = {MOE_DTYPE_MXFP8, MOE_RAGGED_K, MOE_B_NK, MOE_EPI_NONE, MOE_OUT_BF16, 1024, 64, 64, INT32_MAX - 63, INT32_MAX};
  EXPECT(grouped_gemm(&d, p, u8, p, u8, i32, p, nullptr, nullptr, 0, nullptr, nullptr), MOE_ERR_INVALID_ARG);
  d = {MOE_DTYPE_BF16, MOE_RAGGED_K, MOE_B_NK, MOE_EPI_NONE, MOE_OUT_BF16, 4, 64, 64, 0, 100};
  EXPECT(grouped_gemm(&d, p, nullptr, p, nullptr, i32, p, nullptr, nullptr, 0, nullptr, nullptr), MOE_OK);
  if (grouped_gemm_workspace_bytes(&d) != 0) { std::printf("FAIL: gemm workspace\n"); ++g_fail; }
  d.ragged = MOE_RAGGED_M;
  d.K = 64;
  if (grouped_gemm_workspace_bytes(&d) == 0) { std::printf("FAIL: ragged-M gemm workspace\n"); ++g_fail; }
  if (grouped_gemm_workspace_bytes(nullptr) != 0) { std::printf("FAIL: null desc workspace\n"); ++g_fail; }
  d.ragged = MOE_RAGGED_K;
  EXPECT(moe_pack_weights(u16, 4, 64, 64, MOE_EPI_NONE, p, 4 * 64 * 64 * 2, nullptr), MOE_OK);
  EXPECT(moe_pack_weights(u16, 4, 64, 64, MOE_EPI_NONE, p, 16, nullptr), MOE_ERR_WORKSPACE);
  EXPECT(moe_pack_weights(u16, INT32_MAX, 64, 64, MOE_EPI_NONE, p, 1 << 12, nullptr), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_pack_weights_mxfp8(u8, u8, 4, 64, 128, MOE_EPI_NONE, p, 1 << 20, nullptr), MOE_OK);
  // combine, backward helpers, quantisers
  EXPECT(moe_unpermute_combine(u16, f, i32, 16, 64, 2, u16, nullptr), MOE_OK);
  EXPECT(moe_unpermute_combine(u16, f, i32, BIG, 64, 2, u16, nullptr), MOE_OK);   // T only counts tokens
  EXPECT(moe_combine_backward(u16, u16, f, i32, 16, 64, 2, u16, f, nullptr), MOE_OK);
  EXPECT(moe_combine_backward(u16, u16, f, i32, 16, 64, 2, nullptr, f, nullptr), MOE_OK);   // weights only
  EXPECT(moe_combine_backward(u16, u16, f, i32, 16, 64, 2, u16, nullptr, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine_backward_mxfp8(u16, u16, f, i32, 16, 64, 2, u8, u8, f, nullptr), MOE_OK);
  EXPECT(moe_combine_backward_mxfp8(u16, u16, f, i32, 16, 48, 2, u8, u8, f, nullptr), MOE_ERR_UNSUPPORTED);
  EXPECT(moe_combine_backward_mxfp8(u16, u16, f, i32, 16, 64, 2, nullptr, u8, f, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_combine_backward_mxfp8(u16, u16, f, i32, 16, 64, 40, u8, u8, f, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(moe_swiglu_backward(u16, u16, 16, 64, i32, 4, u16, nullptr), MOE_OK);
  EXPECT(moe_swiglu_backward(u16, u16, 16, 64, i32, 0, u16, nullptr), MOE_ERR_INVALID_ARG);
  EXPECT(mxfp8_group_quantize(u16, 16, 64, 0, nullptr, 0, u8, u8, nullptr, nullptr), MOE_OK);
  EXPECT(mxfp8_group_quantize(u16, 16, 64, 1, i32, 4, u8, u8, nullptr, nullptr), MOE_OK);
  EXPECT(mxfp8_quantize_transposed(u16, 64, 64, i32, 4, 64 * 6, u8, u8, nullptr, nullptr, nullptr, nullptr), MOE_OK);
  EXPECT(mxfp8_quantize_transposed(u16, BIG, 64, i32, 4, 64 * 6, u8, u8, nullptr, nullptr, nullptr, nullptr),
         MOE_ERR_INVALID_ARG);
  EXPECT(mxfp8_quantize_gathered(u16, i32, f, 16, 4, 64, i32, 4, 64 * 6, u8, u8, u8, u8, nullptr, nullptr), MOE_OK);
  EXPECT(mxfp8_quantize_gathered(u16, i32, nullptr, 16, 4, 64, i32, 4, 64 * 6, u8, u8, nullptr, nullptr, nullptr,
                                 nullptr),
         MOE_OK);
  EXPECT(mxfp8_quantize_gathered(u16, i32, f, 16, 33, 64, i32, 4, 64 * 6, u8, u8, u8, u8, nullptr, nullptr),
         MOE_ERR_INVALID_ARG);   // K > 32
  EXPECT(mxfp8_quantize_gathered(u16, i32, f, BIG, 4, 64, i32, 4, 64 * 6, u8, u8, u8, u8, nullptr, nullptr),
         MOE_ERR_INVALID_ARG);   // T * K past int32
  EXPECT(mxfp8_quantize_gathered(u16, i32, f, 16, 4, 64, i32, 4, 64, u8, u8, u8, u8, nullptr, nullptr),
         MOE_ERR_INVALID_ARG);   // k_cap below rows + 63 G
  EXPECT(mxfp8_quantize_gathered(u16, i32, f, 16, 4, 48, i32, 4, 64 * 6, u8, u8, u8, u8, nullptr, nullptr),
         MOE_ERR_UNSUPPORTED);   // row codes need cols % 32 == 0
  EXPECT(mxfp8_quantize_gathered(u16, nullptr, f, 16, 4, 64, i32, 4, 64 * 6, u8, u8, u8, u8, nullptr, nullptr),
         MOE_ERR_INVALID_ARG);
  EXPECT(moe_swiglu_backward_mxfp8(u16, u16, 64, 64, i32, 4, 64 * 6, u8, u8, u8, u8, nullptr, nullptr), MOE_OK);
  EXPECT(moe_swiglu_backward_mxfp8(u16, u16, BIG, 64, i32, 4, 64 * 6, u8, u8, u8, u8, nullptr, nullptr),
         MOE_ERR_INVALID_ARG);
  EXPECT(mxfp4_quantize(u16, 16, 128, u8, u8, nullptr), MOE_OK);
  EXPECT(mxfp4_quantize(u16, 16, 96, u8, u8, nullptr), MOE_ERR_UNSUPPORTED);
  for (int s = -1; s <= 6; ++s)
    if (!moe_status_string(s)) { std::printf("FAIL: status string %d\n", s); ++g_fail; }
  std::printf("%s: %d checks failed, %d launches reached\n", g_fail ? "FAIL" : "ok", g_fail, g_launches);
  return g_fail ? 1 : 0;
}
