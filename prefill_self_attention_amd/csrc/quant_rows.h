// quant_rows.h -- INT8 and FP8 (E4M3) rows of the KV cache: one float scale
// per (token, K/V head) row and its codes, computed the same way by every
// kernel that writes a quantised cache (prefill_fwd.hip and fwd64.hip), so
// the codes and scales are bit-identical whichever kernel runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {
namespace qrow {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- INT8 rows
// Symmetric INT8 cache rows, one float scale per (token, K/V head) row of D
// values ["大模型推理优化：Prefill、Decode与KV Cache的工程实践" §4.3: K and V
// quantised, Q kept; INT8 halves the cache; per-token scales are one of the
// granularities it lists]: scale = amax / 127, code = rint(x * (127 / amax))
// with ties to even, both in float32; rows with amax < 2^-100 are stored as
// scale 0 and codes 0.
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xF, 0xF, false));
}
// maximum over aligned groups of N (4, 8 or 16) lanes, in every lane
template <int N>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));                            // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_f<0x4E>(x));                            // quad_perm [2,3,0,1]
  if constexpr (N >= 8) x = fmaxf(x, dpp_f<0x141>(x));     // row_half_mirror
  if constexpr (N >= 16) x = fmaxf(x, dpp_f<0x140>(x));    // row_mirror
  return x;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float absmax8(const u32x4_t w) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) m = fmaxf(m, fmaxf(fabsf(bf16_lo(w[i])), fabsf(bf16_hi(w[i]))));
  return m;
}
constexpr float kInt8MinAmax = 0x1p-100f;
__device__ __forceinline__ float int8_scale(float amax) { return amax >= kInt8MinAmax ? amax / 127.0f : 0.0f; }
__device__ __forceinline__ uint32_t int8_code(float x, float inv) {
  const float t = fminf(fmaxf(__builtin_rintf(x * inv), -127.0f), 127.0f);
  return (uint32_t)(int32_t)t & 0xffu;
}
__device__ __forceinline__ u32x2_t quantize8(const u32x4_t w, float amax) {
  const float inv = amax >= kInt8MinAmax ? 127.0f / amax : 0.0f;
  u32x2_t r;
#pragma unroll
  for (int i = 0; i < 2; ++i)
    r[i] = int8_code(bf16_lo(w[2 * i]), inv) | int8_code(bf16_hi(w[2 * i]), inv) << 8 |
           int8_code(bf16_lo(w[2 * i + 1]), inv) << 16 | int8_code(bf16_hi(w[2 * i + 1]), inv) << 24;
  return r;
}

// FP8 rows: the OCP 8-bit E4M3 format (sign, 4 exponent bits with bias 7, 3
// mantissa bits, subnormals, no infinities, largest finite 448), one float
// scale per row as for INT8: scale = amax / 448, code = E4M3(x * (448 /
// amax)), the product in float32 and the conversion rounding to nearest with
// ties to even (v_cvt_pk_fp8_f32 on this part); rows with amax < 2^-100 get
// scale 0 and the codes of x * 0 (zeros keeping x's sign).
__device__ __forceinline__ float fp8_scale(float amax) { return amax >= kInt8MinAmax ? amax / 448.0f : 0.0f; }
__device__ __forceinline__ u32x2_t quantize_fp8(const u32x4_t w, float amax) {
  const float inv = amax >= kInt8MinAmax ? 448.0f / amax : 0.0f;
  u32x2_t r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w[2 * i]) * inv, bf16_hi(w[2 * i]) * inv, 0, false);
    r[i] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w[2 * i + 1]) * inv, bf16_hi(w[2 * i + 1]) * inv, lo,
                                                     true);
  }
  return r;
}

// cache formats of the varlen kernel's cache write
constexpr int kCacheBf16 = 0;
constexpr int kCacheInt8 = 1;
constexpr int kCacheFp8 = 2;

}  // namespace qrow
}  // namespace pa
