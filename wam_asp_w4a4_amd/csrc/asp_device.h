// Device-side helpers shared by the gfx950 translation units of libasp:
// vector types, the NVFP4 block quantiser, operand decoding for MFMA,
// launch/argument checks, and the internal launchers each unit exports.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "asp.h"
#include "asp_internal.h"
#include "nvfp4_codec.h"

namespace asp {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
// 16 bytes as a native vector: unlike HIP's uint4 (a struct of unions), it
// stays in registers when carried around a loop
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef double f64x2_t __attribute__((ext_vector_type(2)));

constexpr float kInvSqrt128 = 0.08838834764831845f;  // 1/sqrt(128), rounded to float32

// A float32 quotient of v by the decoded block scale sd that falls on the same
// side of every E2M1 grid midpoint as the exact v/sd, and on a midpoint exactly
// when v/sd is one.  q0 = v * rinv (rinv = 1/sd to within an ulp) is within a
// few ulps of v/sd, so the remainder q0*sd - v is exactly representable (sd has
// 4 significant bits) and one fma gives it exactly; q1 = q0 - e*rinv is then
// v/sd to far less than an ulp.  A v/sd that is not a midpoint lies more than
// half an ulp from every midpoint (a midpoint times sd has at most 7
// significant bits, so v differs from it by at least an ulp of v), hence q1 is
// on the same side.  q1 keeps v's sign, -0 included (-0 - +0 = -0), so the
// hardware conversion copies the sign bit as the format requires; rinv == 0
// (a zero scale) gives magnitude 0.  Valid for |v| <= ~6.4 sd, which a block's
// own scale guarantees (larger quotients only arise with the saturated scale
// 448, where q0 stays finite and the conversion saturates).
__device__ __forceinline__ float e2m1_quotient(float v, float sd, float rinv) {
  const float q0 = v * rinv;
  const float e = __builtin_fmaf(q0, sd, -v);
  return __builtin_fmaf(-e, rinv, q0);
}

// NVFP4 block of 16 values held by one lane in column order: its E4M3 scale
// code and the 8 bytes of packed codes.  v_cvt_scalef32_pk_fp4_f32 with scale
// 1 rounds to nearest, ties to the even code, and saturates at 6; it writes
// the code of its first operand into the low nibble of the selected byte.
__device__ __forceinline__ uint2 quantize_block(const float (&v)[16], uint32_t& scale) {
  float amax = 0.0f;
#pragma unroll
  for (int c = 0; c < 16; ++c) amax = fmaxf(amax, fabsf(v[c]));
  scale = block_scale_code(amax);
  const float sd = e4m3_decode(scale);
  const float rinv = sd > 0.0f ? __builtin_amdgcn_rcpf(sd) : 0.0f;
  auto pk = [&](uint32_t w, int c, auto sel) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, e2m1_quotient(v[c], sd, rinv),
                                                    e2m1_quotient(v[c + 1], sd, rinv), 1.0f,
                                                    decltype(sel)::value);
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  uint32_t w0 = 0, w1 = 0;
  w0 = pk(w0, 0, S0{}); w0 = pk(w0, 2, S1{}); w0 = pk(w0, 4, S2{}); w0 = pk(w0, 6, S3{});
  w1 = pk(w1, 8, S0{}); w1 = pk(w1, 10, S1{}); w1 = pk(w1, 12, S2{}); w1 = pk(w1, 14, S3{});
  return make_uint2(w0, w1);
}

// Direct global-to-LDS copy of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's bytes land at lds_base + 16*l; lds_base must be wave-uniform.  No
// registers are involved, so many copies can be in flight at once; they count
// as vector-memory operations for s_waitcnt.
__device__ __forceinline__ void lds_copy16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds(src, lds_base, 16, 0, 0);
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

// float -> bf16 rounded to nearest even by the hardware conversion
// (v_cvt_pk_bf16_f32, two values per instruction; finite inputs)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t bf16_rne(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ bf16x8_t bf16x8_rne(const float (&f)[8]) {
  const uint32_t w[4] = {bf16x2_rne(f[0], f[1]), bf16x2_rne(f[2], f[3]), bf16x2_rne(f[4], f[5]),
                         bf16x2_rne(f[6], f[7])};
  return __builtin_bit_cast(bf16x8_t, w);
}

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

// Internal launchers (validate, then enqueue on `stream`).  A call covers one
// layer or a group of up to kMaxGroup layers with the same M, K, r and dtypes:
// each launch then spans every layer of the group (one more grid dimension),
// so small layers fill more of the chip and pay one launch between them.
constexpr int kMaxGroup = 8;

struct PrepCall {
  const void* x;
  const uint8_t* prep_pack;
  uint8_t* x_codes;
  uint8_t* x_scales;
  float* u;
  float* prequant;
  void* scratch;  // the partial sums of u
  size_t scratch_bytes;
};

struct GemmCall {
  const uint8_t* x_codes;
  const uint8_t* x_scales;
  const float* u;
  const uint8_t* w_codes;
  const uint8_t* w_scales;
  const uint16_t* wv;
  const float* bias;
  void* y;
  int64_t N;
};

size_t act_prep_scratch_bytes(int64_t M, int64_t K, int32_t r);
// stages: 1 = partial sums of u (k_prep_u), 2 = the rest (k_prep_q), 3 = both
int32_t act_prep_impl(int stages, int n, const PrepCall* calls, int32_t x_dtype, int64_t M,
                      int64_t K, int32_t r, hipStream_t stream);
int32_t gemm_check(int64_t M, int64_t N, int64_t K, int32_t r, int32_t y_dtype);
int32_t gemm_impl(int n, const GemmCall* calls, int64_t M, int64_t K, int32_t r, int32_t y_dtype,
                  hipStream_t stream);

}  // namespace asp
