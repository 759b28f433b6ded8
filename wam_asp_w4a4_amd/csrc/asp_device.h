// Device-side helpers shared by the gfx950 translation units of libasp:
// vector types, the NVFP4 lane-pair quantiser, operand decoding for MFMA,
// launch/argument checks, and the internal launchers each unit exports.
#pragma once

#include <hip/hip_runtime.h>

#include "asp.h"
#include "asp_internal.h"
#include "nvfp4_codec.h"

namespace asp {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kInvSqrt128 = 0.08838834764831845f;  // 1/sqrt(128), rounded to float32

// Quantise the 8 consecutive values a lane holds; lanes (2j, 2j+1) hold one
// 16-element block.  Returns the 8 packed 4-bit codes (element e in bits
// 4e..4e+3) and the block's E4M3 scale code.  Every lane of the wave calls it.
__device__ __forceinline__ uint32_t quantize8_pair(const float (&v)[8], uint32_t& scale) {
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  scale = block_scale_code(amax);
  const float sd = e4m3_decode(scale);
  uint32_t word = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) word |= e2m1_code(v[e], sd) << (4 * e);
  return word;
}

__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

__device__ __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
  const uint4 a = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[2 * e] = bits_f32(w[e] << 16);
    v[2 * e + 1] = bits_f32(w[e] & 0xFFFF0000u);
  }
}

// 8 packed E2M1 codes (one K-step's worth for one MFMA lane) times their
// block scale, as exact fp16.  The hardware conversion applies only the
// power-of-two part of a scale, so it runs with scale 1 and the E4M3 scale
// (exact in fp16) is applied by a packed fp16 multiply: every product of an
// E2M1 value and an E4M3 value is an fp16 number, so nothing rounds.
__device__ __forceinline__ half8_t decode8(uint32_t w, _Float16 sc) {
  const half2_t s2 = {sc, sc};
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ _Float16 scale_f16(uint32_t code) {
  return (_Float16)e4m3_decode(code);  // exact: every E4M3 value is an fp16 normal
}

__device__ __forceinline__ __bf16 bf16_from_bits(uint16_t b) { return __builtin_bit_cast(__bf16, b); }

// ------------------------------------------------------------- host helpers

inline int32_t launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ASP_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return ASP_OK;
}

inline int32_t check_ptr(const void* p, const char* name, bool required) {
  if (!p) return required ? fail(ASP_ERR_ARG, "%s is NULL", name) : ASP_OK;
  if (!aligned16(p)) return fail(ASP_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return ASP_OK;
}

#define ASP_TRY(expr)                      \
  do {                                     \
    if (int32_t st_ = (expr)) return st_;  \
  } while (0)

constexpr int64_t kMaxK = 1 << 20;

inline int32_t check_mk(int64_t M, int64_t K) {
  ASP_TRY(check_k(K));
  if (K > kMaxK) return fail(ASP_ERR_SHAPE, "K=%lld above %lld", (long long)K, (long long)kMaxK);
  if (M < 0 || M > INT32_MAX) return fail(ASP_ERR_SHAPE, "M=%lld outside [0, 2^31)", (long long)M);
  return ASP_OK;
}

// Internal launchers (validate, then enqueue on `stream`).
size_t act_prep_scratch_bytes(int64_t M, int64_t K, int32_t r);
int32_t act_prep_impl(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                      const uint8_t* prep_pack, uint8_t* x_codes, uint8_t* x_scales, float* u,
                      float* prequant, void* scratch, size_t scratch_bytes, hipStream_t stream);
int32_t gemm_check(int64_t M, int64_t N, int64_t K, int32_t r, int32_t y_dtype);
int32_t gemm_impl(const uint8_t* x_codes, const uint8_t* x_scales, const float* u, int64_t M,
                  int64_t N, int64_t K, int32_t r, const uint8_t* w_codes,
                  const uint8_t* w_scales, const uint16_t* wv, const float* bias, void* y,
                  int32_t y_dtype, hipStream_t stream);

}  // namespace asp
