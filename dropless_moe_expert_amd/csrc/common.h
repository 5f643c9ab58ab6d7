// Shared device-side helpers of the dropless-MoE library (gfx950 only).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "moe.h"

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4_t;

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// round-to-nearest-even f32 -> bf16 bits (NaN stays NaN)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return ((u >> 16) | 0x40u) & 0xFFFFu;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

typedef float f32x2_v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even; one v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

// 8 bf16 in a uint4 -> 8 floats
__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xFFFF0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}

__device__ __forceinline__ uint4 pack8(const float* f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                    pack_bf16x2(f[6], f[7]));
}

// bf16(w * g[j]) for 8 values, each the exact product rounded to nearest even
// once.  The fp32 product p can only round differently from the exact one
// when p lies exactly halfway between two bf16 values (low 16 bits 0x8000):
// then its exact error e = fma(w, g, -p) says on which side the product
// lies (e == 0: a true tie, to even).  Exact for products in the normal
// fp32 range; NaN and infinity as the plain conversion gives them.
__device__ __forceinline__ uint4 mul8_bf16(float w, const float* g) {
  float p[8];
  uint32_t fix[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = w * g[j];
    const float e = fmaf(w, g[j], -p[j]);
    const uint32_t b = __float_as_uint(p[j]);
    const bool mid = (b & 0xFFFFu) == 0x8000u && e != 0.f && (b & 0x7F800000u) != 0x7F800000u;
    // the bf16 bits toward the exact product: magnitude up when e has p's sign
    fix[j] = mid ? (b >> 16) + (((__float_as_uint(e) ^ b) >> 31) ^ 1u) : 0xFFFFFFFFu;
  }
  const uint4 v = pack8(p);
  uint32_t h[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (fix[2 * q] != 0xFFFFFFFFu) h[q] = (h[q] & 0xFFFF0000u) | fix[2 * q];
    if (fix[2 * q + 1] != 0xFFFFFFFFu) h[q] = (h[q] & 0xFFFFu) | (fix[2 * q + 1] << 16);
  }
  return make_uint4(h[0], h[1], h[2], h[3]);
}

// ---------------------------------------------------------------- error flag
__device__ __forceinline__ void raise_flag(uint32_t* flag, uint32_t bits) {
  if (flag) atomicOr(flag, bits);
}

// ---------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Rows in use of a ragged operand: the sum of the G device group sizes
// (negative sizes count as 0), at most cap.  Called by a whole wavefront,
// which reads the sizes 64 at a time; every lane gets the result.
__device__ __forceinline__ int64_t rows_in_use(const int32_t* sizes, int G, int64_t cap) {
  int64_t t = 0;
  for (int g = (int)(threadIdx.x & 63); g < G; g += kWave) t += max(sizes[g], 0);
  return min(wave_sum(t), cap);
}

// SwiGLU backward of one element, from the pre-activations g, u and dh:
// with s = sigmoid(g), dg = dh*u*s*(1 + g*(1-s)), du = dh*g*s.  Shared by
// the bf16 SwiGLU backward and the one that quantises its output, so both
// round the same values.
__device__ __forceinline__ void swiglu_grad(float g, float u, float d, float& dg, float& du) {
#pragma clang fp contract(off)   // the same roundings wherever it is inlined
  const float s = 1.0f / (1.0f + __expf(-g));
  dg = d * u * s * (1.0f + g * (1.0f - s));
  du = d * g * s;
}

// ---------------------------------------------------------------- MXFP8 rounding
// Shared by the quantisation kernels and the GEMM epilogue that quantises its
// output, so both apply the same rule bit for bit.  Scale rule (OCP MX v1.0):
// e = floor(log2 amax) - 8 (8 = largest E4M3 exponent) clamped to
// [-127, 127], byte = e + 127; codes are the E4M3FN round-to-nearest-even of
// v * 2^-e clamped to +-448.  v * 2^-e is exact in fp32 for bf16 inputs;
// v_cvt_pk_fp8_f32 rounds to nearest even and keeps the sign of zero.
// A block holding a NaN or an infinity has no finite shared exponent: its
// scale is the E8M0 NaN (byte 0xFF = kMxNaN + 127), which makes every element
// of the block NaN, and each code is the element format's NaN with the
// value's sign (E2M1, which has none, saturates to its largest code).
constexpr int kMxNaN = 128;

// running amax of a block: |v| compared as integer bits, so that every
// finite value < +inf < NaN and a non-finite element is never dropped
__device__ __forceinline__ float mx_absmax(float m, float v) {
  return __uint_as_float(max(__float_as_uint(m), __float_as_uint(v) & 0x7FFFFFFFu));
}

// floor(log2(amax)) - 8 from the fp32 bits of a bf16 amax; clamped;
// kMxNaN for a NaN or infinite amax
__device__ __forceinline__ int mx_exponent(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  if (ef == 0) return -127;  // zero or subnormal amax: floor(log2) <= -127
  if (ef == 255) return kMxNaN;
  return max(-127, min(127, ef - 127 - 8));
}

__device__ __forceinline__ float pow2i(int e) {  // 2^e for e in [-126, 127]
  return __uint_as_float((uint32_t)(e + 127) << 23);
}

__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  int hi = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
  return (uint32_t)hi;
}

// multiply by 2^-e with e in [-127, 127]: 2^127 is one step outside the
// normal-exponent helper, so scale in two exact steps
__device__ __forceinline__ float scale_pow2(float v, int e) {
  const int ne = -e;  // in [-127, 127]
  if (ne >= -126) return v * pow2i(ne);
  return (v * pow2i(-63)) * pow2i(-64);
}

// E4M3 codes of four values of one block with shared exponent e (byte 0 =
// a ... byte 3 = d)
__device__ __forceinline__ uint32_t mx_codes4(float a, float b, float c, float d, int e) {
  if (e == kMxNaN)
    return 0x7F7F7F7Fu | ((__float_as_uint(a) >> 31) << 7) | ((__float_as_uint(b) >> 31) << 15) |
           ((__float_as_uint(c) >> 31) << 23) | ((__float_as_uint(d) >> 31) << 31);
  return cvt4_e4m3(scale_pow2(a, e), scale_pow2(b, e), scale_pow2(c, e), scale_pow2(d, e));
}

// the same with a shared exponent per value (four blocks, one value each)
__device__ __forceinline__ uint32_t mx_nan_byte(uint32_t q, float v, int e, int sh) {
  return e == kMxNaN ? ((q & ~(0xFFu << sh)) | ((0x7Fu | ((__float_as_uint(v) >> 31) << 7)) << sh)) : q;
}
__device__ __forceinline__ uint32_t mx_codes4(float a, float b, float c, float d, int ea, int eb, int ec, int ed) {
  uint32_t q = cvt4_e4m3(scale_pow2(a, ea), scale_pow2(b, eb), scale_pow2(c, ec), scale_pow2(d, ed));
  q = mx_nan_byte(q, a, ea, 0);
  q = mx_nan_byte(q, b, eb, 8);
  q = mx_nan_byte(q, c, ec, 16);
  return mx_nan_byte(q, d, ed, 24);
}

// ------------------------------------------- MXFP8 codes of packed bf16 pairs
// The same rule on bf16 data by gfx950's scaled conversion
// (v_cvt_scalef32_pk_fp8_bf16: two bf16 times 2^-e, rounded to nearest even
// into E4M3, sign of zero kept, subnormals kept).  Checked on the hardware
// against cvt4_e4m3(scale_pow2(v, e)) for every finite bf16 v with
// |v| < 2^(e+9) and every e in [-127, 127]: identical, except that the
// conversion does not saturate (a value that rounds past 448 becomes NaN).
// So each magnitude is first clamped to 448 * 2^e, which is exact: every
// value in (448, 480) * 2^e rounds to 448 anyway.  Element 0 of a pair is its
// low half; a code word holds elements 0..3 in bytes 0..3.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// the conversion's scale operand for 2^e: the E8M0 byte in the f32 exponent
// field (byte 0, e = -127, reads as 2^-127)
__device__ __forceinline__ float mx_scale_operand(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// bf16 bits of 448 * 2^e in both halves: above e = 119 no finite bf16
// reaches 464 * 2^e, and the +inf bound leaves every finite value alone
__device__ __forceinline__ uint32_t mx_clamp_pair(int e) {
  const uint32_t l = e >= 120 ? 0x7F80u : ((uint32_t)(e + 8 + 127) << 7) | 0x60u;
  return l | (l << 16);
}

__device__ __forceinline__ uint32_t min_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2_t, a),
                                                                __builtin_bit_cast(u16x2_t, b)));
}
__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                __builtin_bit_cast(u16x2_t, b)));
}
__device__ __forceinline__ uint32_t min_i16x2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(i16x2_t, a),
                                                                __builtin_bit_cast(i16x2_t, b)));
}

// |bf16| of both halves as unsigned 16-bit integers (the amax order)
__device__ __forceinline__ uint32_t mag_pair(uint32_t p) { return p & 0x7FFF7FFFu; }
// fp32 bits of the larger half of a magnitude pair (an amax for mx_exponent)
__device__ __forceinline__ float amax_of_pair(uint32_t m) { return __uint_as_float(max(m & 0xFFFFu, m >> 16) << 16); }

// both halves' magnitudes clamped to the bound l (lim2 = l in both halves,
// l <= 0x7F80), signs kept: as unsigned 16-bit a negative half 0x8000 | m
// is min'd with 0x8000 | l and a positive one is below that; as signed
// 16-bit a positive half is min'd with l and a negative one is below it
__device__ __forceinline__ uint32_t clamp_pair(uint32_t p, uint32_t lim2) {
  return min_i16x2(min_u16x2(p, lim2 | 0x80008000u), lim2);
}

// codes of elements 0..3 (p01 = elements 0 and 1, p23 = 2 and 3) of a block
// with finite exponent e: sc = mx_scale_operand(e), lim2 = mx_clamp_pair(e).
// Each conversion writes one half of its destination and keeps the other
// (here the clamped word's, overwritten by the second conversion).
__device__ __forceinline__ uint32_t mx_codes4_pairs(uint32_t p01, uint32_t p23, float sc, uint32_t lim2) {
  const uint32_t c01 = clamp_pair(p01, lim2), c23 = clamp_pair(p23, lim2);
  i16x2_t r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(__builtin_bit_cast(i16x2_t, c01),
                                                        __builtin_bit_cast(bf16x2_t, c01), sc, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(r, __builtin_bit_cast(bf16x2_t, c23), sc, true);
  return __builtin_bit_cast(uint32_t, r);
}
// the NaN block's codes of the same four elements (0x7F with each sign)
__device__ __forceinline__ uint32_t mx_nan_codes4_pairs(uint32_t p01, uint32_t p23) {
  return 0x7F7F7F7Fu | ((p01 >> 8) & 0x80u) | ((p01 >> 16) & 0x8000u) | ((p23 << 8) & 0x800000u) |
         (p23 & 0x80000000u);
}

// silu(g) = g * sigmoid(g); hardware exp and reciprocal (about 1 ulp each)
__device__ __forceinline__ float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

}  // namespace moe

// Host-side launch helpers shared by the entry points (defined in abi.cpp).
namespace moe_host {
int device_cu_count();
}
