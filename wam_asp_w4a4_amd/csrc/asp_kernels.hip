// gfx950 (CDNA4) kernels of libasp and their C entry points.
//
//   k_quantize      NVFP4 quantiser (float32 rows -> codes + E4M3 scales)
//   k_dequantize    NVFP4 dequantiser
//   k_act_prep      fused activation prep: x/s, block Hadamard, u = x_tilde V,
//                   deflation x_tilde - u V^T, NVFP4 quantise + pack
//   k_gemm          4-bit GEMM on MFMA with in-register dequantisation and a
//                   fused bf16 low-rank + bias epilogue
//
// The layer (model card "FastWAM UR3 3-task -- 4-bit quantisations", section
// "What ASP is, and what the deflated form means"):
//   y = (x_tilde V)(W_tilde V)^T + NVFP4GEMM((I - V V^T) x_tilde, W_tilde (I - V V^T)) + b.
//
// NVFP4 has 16-element blocks with E4M3 scales, while gfx950's scaled FP4
// MFMA takes one power-of-two (E8M0) scale per 32 elements, so the operands
// are instead decoded in registers: an E2M1 value times an E4M3 scale has at
// most 6 significant bits and lies in [2^-10, 2688], so it is an exact normal
// fp16 number and the fp16 MFMA (fp32 accumulation) sees exactly the values
// the format encodes.
#include <hip/hip_runtime.h>

#include "asp.h"
#include "asp_internal.h"
#include "nvfp4_codec.h"

using namespace asp;

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr float kInvSqrt128 = 0.08838834764831845f;  // 1/sqrt(128), rounded to float32

// ---------------------------------------------------------------------------
// Quantise the 8 consecutive values a lane holds; the lane pair (2j, 2j+1)
// holds one 16-block.  Returns the 8 packed codes (element e in bits 4e..4e+3)
// and the block's scale code.  Every lane of the wave must call this.
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

// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) k_quantize(const float* __restrict__ in, int64_t n_half,
                                                  uint32_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // one lane per 8 elements
  const bool ok = i < n_half;
  float v[8];
  if (ok) {
    const float4 a = reinterpret_cast<const float4*>(in)[2 * i];
    const float4 b = reinterpret_cast<const float4*>(in)[2 * i + 1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = 0.0f;
  }
  uint32_t sc;
  const uint32_t word = quantize8_pair(v, sc);
  if (ok) {
    codes[i] = word;
    if ((i & 1) == 0) scales[i >> 1] = (uint8_t)sc;
  }
}

__global__ void __launch_bounds__(256) k_dequantize(const uint32_t* __restrict__ codes,
                                                    const uint8_t* __restrict__ scales,
                                                    int64_t n_half, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_half) return;
  const uint32_t w = codes[i];
  const float sd = e4m3_decode(scales[i >> 1]);
  float v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = e2m1_decode((w >> (4 * e)) & 15u) * sd;
  reinterpret_cast<float4*>(out)[2 * i] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(out)[2 * i + 1] = make_float4(v[4], v[5], v[6], v[7]);
}

// ---------------------------------------------------------------------------
// Activation prep.  One workgroup (256 lanes) per row of x.  Lane t holds 8
// consecutive channels per 2048-channel chunk; the 16 lanes of a 128-channel
// Hadamard block are a contiguous, aligned lane group, so the transform is
// 3 in-register butterfly stages plus 4 cross-lane stages (lane xor 1,2,4,8).

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

// Sylvester-ordered Walsh-Hadamard transform of the 128 values held by a
// 16-lane group (8 per lane, lane-major), scaled by 1/sqrt(128).
__device__ __forceinline__ void fwht128_group(float (&v)[8], int lane) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if ((e & h) == 0) {
        const float a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
#pragma unroll
  for (int mask = 1; mask < 16; mask <<= 1) {
    const bool upper = lane & mask;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float o = __shfl_xor(v[e], mask);
      v[e] = upper ? o - v[e] : v[e] + o;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] *= kInvSqrt128;
}

template <typename XT>
__global__ void __launch_bounds__(256) k_act_prep(const XT* __restrict__ x, int K, int r,
                                                  const float* __restrict__ s,
                                                  const float* __restrict__ V,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales,
                                                  float* __restrict__ u_out,
                                                  float* __restrict__ pre) {
  extern __shared__ float smem[];  // r > 0: x_tilde[K], partial sums[256], u[64]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t row = blockIdx.x;
  const XT* xr = x + row * K;
  uint8_t* crow = codes + row * (K / 2);
  uint8_t* srow = scales + row * (K / 16);
  float* prow = pre ? pre + row * K : nullptr;

  float* xt = smem;
  float* part = smem + K;
  float* us = part + 256;

  for (int c0 = tid * 8; c0 < K; c0 += 2048) {
    float v[8], sv[8];
    load8(xr + c0, v);
    load8(s + c0, sv);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = v[e] / sv[e];
    fwht128_group(v, lane);
    if (r == 0) {
      uint32_t sc;
      const uint32_t word = quantize8_pair(v, sc);
      *reinterpret_cast<uint32_t*>(crow + c0 / 2) = word;
      if ((tid & 1) == 0) srow[c0 / 16] = (uint8_t)sc;
      if (prow) {
        reinterpret_cast<float4*>(prow + c0)[0] = make_float4(v[0], v[1], v[2], v[3]);
        reinterpret_cast<float4*>(prow + c0)[1] = make_float4(v[4], v[5], v[6], v[7]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) xt[c0 + e] = v[e];
    }
  }
  if (r == 0) return;
  __syncthreads();

  // u = x_tilde V: lane t sums column c = t % r over channels seg, seg+nseg, ...
  const int nseg = 256 / r;
  {
    const int c = tid % r, seg = tid / r;
    float acc = 0.0f;
    if (seg < nseg)
      for (int k = seg; k < K; k += nseg) acc = fmaf(xt[k], V[(int64_t)k * r + c], acc);
    part[tid] = acc;
  }
  __syncthreads();
  if (tid < r) {
    float acc = 0.0f;
    for (int g = 0; g < nseg; ++g) acc += part[g * r + tid];
    us[tid] = acc;
    u_out[row * r + tid] = acc;
  }
  __syncthreads();

  // deflate and quantise
  for (int c0 = tid * 8; c0 < K; c0 += 2048) {
    float v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float* vr = V + (int64_t)(c0 + e) * r;
      float d = xt[c0 + e];
      for (int c = 0; c < r; ++c) d = fmaf(-us[c], vr[c], d);
      v[e] = d;
    }
    uint32_t sc;
    const uint32_t word = quantize8_pair(v, sc);
    *reinterpret_cast<uint32_t*>(crow + c0 / 2) = word;
    if ((tid & 1) == 0) srow[c0 / 16] = (uint8_t)sc;
    if (prow) {
      reinterpret_cast<float4*>(prow + c0)[0] = make_float4(v[0], v[1], v[2], v[3]);
      reinterpret_cast<float4*>(prow + c0)[1] = make_float4(v[4], v[5], v[6], v[7]);
    }
  }
}

// ---------------------------------------------------------------------------
// 4-bit GEMM.  Workgroup tile 128 x 128 (M x N), 4 waves as 2 x 2, each wave
// 64 x 64 = 2 x 2 tiles of v_mfma_f32_32x32x16_f16.  K advances 128 elements
// (8 NVFP4 blocks) per stage through double-buffered LDS.
//
// MFMA 32x32x16 operand layout: lane l supplies row (A) / column (B) l % 32
// and 8 K-elements selected by l / 32; a lane's 8 codes of one K-step are one
// 32-bit word of packed nibbles (8 consecutive elements of one 16-block).
// LDS keeps each tile row's 128 elements permuted so that the 8 words a lane
// needs for the 8 K-steps are contiguous: word g of the row (elements
// 8g..8g+7) sits at position (g % 2) * 8 + g / 2.
constexpr int BM = 128, BN = 128, BK = 128;
constexpr int ROWB = 80;  // LDS bytes per tile row: 64 code bytes + 16 pad

struct GemmSmem {
  uint8_t a[2][BM * ROWB];
  uint8_t b[2][BN * ROWB];
  uint8_t as[2][BM * 8];
  uint8_t bs[2][BN * 8];
};

__device__ __forceinline__ half8_t decode8(uint32_t w, uint32_t scale_code) {
  const _Float16 sc = (_Float16)e4m3_decode(scale_code);  // exact
  const half2_t s2 = {sc, sc};
  const half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
  const half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
  const half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
  const half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

__device__ __forceinline__ __bf16 bf16_from_bits(uint16_t b) {
  return __builtin_bit_cast(__bf16, b);
}

__global__ void __launch_bounds__(256) k_gemm(const uint8_t* __restrict__ xc,
                                              const uint8_t* __restrict__ xs,
                                              const float* __restrict__ u, int M, int N, int K,
                                              int r, const uint8_t* __restrict__ wc,
                                              const uint8_t* __restrict__ ws,
                                              const uint16_t* __restrict__ wv,
                                              const float* __restrict__ bias, void* __restrict__ y,
                                              int y_bf16) {
  __shared__ GemmSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int64_t KB = K / 2, KS = K / 16;

  // global -> register staging coordinates: rows lrow and lrow + 64, 16 bytes
  // at segment lseg of the stage's 64 code bytes; one 8-byte scale row per lane.
  const int lrow = tid >> 2, lseg = tid & 3;
  const int64_t ar0 = min(m0 + lrow, M - 1), ar1 = min(m0 + lrow + 64, M - 1);
  const int64_t br0 = min(n0 + lrow, N - 1), br1 = min(n0 + lrow + 64, N - 1);
  const uint8_t* srow = tid < 128 ? xs + (int64_t)min(m0 + tid, M - 1) * KS
                                  : ws + (int64_t)min(n0 + tid - 128, N - 1) * KS;

  uint4 ra0, ra1, rb0, rb1;
  uint2 rsc;
  auto gload = [&](int kc) {
    const int64_t off = (int64_t)kc * 64 + lseg * 16;
    ra0 = *reinterpret_cast<const uint4*>(xc + ar0 * KB + off);
    ra1 = *reinterpret_cast<const uint4*>(xc + ar1 * KB + off);
    rb0 = *reinterpret_cast<const uint4*>(wc + br0 * KB + off);
    rb1 = *reinterpret_cast<const uint4*>(wc + br1 * KB + off);
    rsc = *reinterpret_cast<const uint2*>(srow + (int64_t)kc * 8);
  };
  auto sstore = [&](int buf) {
    // words 4*lseg .. 4*lseg+3 -> positions (g%2)*8 + g/2
    auto put = [&](uint8_t* base, int row, uint4 q) {
      uint8_t* p = base + row * ROWB;
      *reinterpret_cast<uint2*>(p + 8 * lseg) = make_uint2(q.x, q.z);
      *reinterpret_cast<uint2*>(p + 32 + 8 * lseg) = make_uint2(q.y, q.w);
    };
    put(sm.a[buf], lrow, ra0);
    put(sm.a[buf], lrow + 64, ra1);
    put(sm.b[buf], lrow, rb0);
    put(sm.b[buf], lrow + 64, rb1);
    if (tid < 128)
      *reinterpret_cast<uint2*>(sm.as[buf] + tid * 8) = rsc;
    else
      *reinterpret_cast<uint2*>(sm.bs[buf] + (tid - 128) * 8) = rsc;
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int half = lane >> 5, l32 = lane & 31;
  const int nk = K / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int buf = kc & 1;
    if (kc + 1 < nk) gload(kc + 1);
    uint32_t aw[2][8], bw[2][8];
    uint2 asc[2], bsc[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int arow = wm * 64 + i * 32 + l32;
      const uint4* pa = reinterpret_cast<const uint4*>(sm.a[buf] + arow * ROWB + half * 32);
      const uint4 q0 = pa[0], q1 = pa[1];
      aw[i][0] = q0.x; aw[i][1] = q0.y; aw[i][2] = q0.z; aw[i][3] = q0.w;
      aw[i][4] = q1.x; aw[i][5] = q1.y; aw[i][6] = q1.z; aw[i][7] = q1.w;
      asc[i] = *reinterpret_cast<const uint2*>(sm.as[buf] + arow * 8);
      const int brow = wn * 64 + i * 32 + l32;
      const uint4* pb = reinterpret_cast<const uint4*>(sm.b[buf] + brow * ROWB + half * 32);
      const uint4 p0 = pb[0], p1 = pb[1];
      bw[i][0] = p0.x; bw[i][1] = p0.y; bw[i][2] = p0.z; bw[i][3] = p0.w;
      bw[i][4] = p1.x; bw[i][5] = p1.y; bw[i][6] = p1.z; bw[i][7] = p1.w;
      bsc[i] = *reinterpret_cast<const uint2*>(sm.bs[buf] + brow * 8);
    }
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      half8_t af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t as_word = ks < 4 ? asc[i].x : asc[i].y;
        const uint32_t bs_word = ks < 4 ? bsc[i].x : bsc[i].y;
        af[i] = decode8(aw[i][ks], (as_word >> (8 * (ks & 3))) & 0xFFu);
        bf[i] = decode8(bw[i][ks], (bs_word >> (8 * (ks & 3))) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kc + 1 < nk) sstore(buf ^ 1);
    __syncthreads();
  }

  // Low-rank branch: bf16(u) (M x r) times wv^T (r x N) as extra K-steps of 16.
  for (int c0 = 0; c0 < r; c0 += 16) {
    bf16x8_t la[2], lb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t m = min(m0 + wm * 64 + i * 32 + l32, M - 1);
      const int64_t n = min(n0 + wn * 64 + i * 32 + l32, N - 1);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = c0 + half * 8 + e;
        la[i][e] = bf16_from_bits(c < r ? f32_to_bf16_rne(u[m * r + c]) : (uint16_t)0);
        lb[i][e] = bf16_from_bits(c < r ? wv[n * r + c] : (uint16_t)0);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[i], lb[j], acc[i][j], 0, 0, 0);
  }

  // Bias and store.  Accumulator element v of lane l is row
  // 8*(v/4) + 4*(l/32) + v%4 and column l%32 of the 32 x 32 tile.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = n0 + wn * 64 + j * 32 + l32;
    if (col >= N) continue;
    const float bcol = bias ? bias[col] : 0.0f;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
        if (row >= M) continue;
        const float val = acc[i][j][v] + bcol;
        if (y_bf16)
          reinterpret_cast<uint16_t*>(y)[(int64_t)row * N + col] = f32_to_bf16_rne(val);
        else
          reinterpret_cast<float*>(y)[(int64_t)row * N + col] = val;
      }
  }
}

int32_t launch_status(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(ASP_ERR_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return ASP_OK;
}

int32_t check_ptr(const void* p, const char* name, bool required) {
  if (!p) return required ? fail(ASP_ERR_ARG, "%s is NULL", name) : ASP_OK;
  if (!aligned16(p)) return fail(ASP_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return ASP_OK;
}

#define ASP_TRY(expr)                 \
  do {                                \
    if (int32_t st_ = (expr)) return st_; \
  } while (0)

constexpr int64_t kMaxK = 1 << 20;

int32_t check_mk(int64_t M, int64_t K) {
  ASP_TRY(check_k(K));
  if (K > kMaxK) return fail(ASP_ERR_SHAPE, "K=%lld above %lld", (long long)K, (long long)kMaxK);
  if (M < 0 || M > INT32_MAX) return fail(ASP_ERR_SHAPE, "M=%lld outside [0, 2^31)", (long long)M);
  return ASP_OK;
}

// Largest K for which the r > 0 prep keeps x_tilde of one row in 64 KiB of LDS.
constexpr int64_t kMaxKDeflate = (65536 / 4 - 256 - 64) / 128 * 128;

int32_t act_prep_impl(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                      const float* s, const float* v, uint8_t* x_codes, uint8_t* x_scales,
                      float* u, float* prequant, hipStream_t stream) {
  ASP_TRY(check_mk(M, K));
  ASP_TRY(check_rank(r));
  if (x_dtype != ASP_F32 && x_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "x_dtype=%d", x_dtype);
  if (r > 0 && K > kMaxKDeflate)
    return fail(ASP_ERR_UNSUPPORTED, "r > 0 needs K <= %lld in this build", (long long)kMaxKDeflate);
  if (M == 0) return ASP_OK;
  ASP_TRY(check_ptr(x, "x", true));
  ASP_TRY(check_ptr(s, "s", true));
  ASP_TRY(check_ptr(v, "v", r > 0));
  ASP_TRY(check_ptr(x_codes, "x_codes", true));
  ASP_TRY(check_ptr(x_scales, "x_scales", true));
  ASP_TRY(check_ptr(u, "u", r > 0));
  ASP_TRY(check_ptr(prequant, "prequant", false));
  const size_t lds = r > 0 ? (size_t)(K + 256 + 64) * sizeof(float) : 0;
  if (x_dtype == ASP_F32)
    hipLaunchKernelGGL(k_act_prep<float>, dim3((unsigned)M), dim3(256), lds, stream,
                       static_cast<const float*>(x), (int)K, (int)r, s, v, x_codes, x_scales, u,
                       prequant);
  else
    hipLaunchKernelGGL(k_act_prep<uint16_t>, dim3((unsigned)M), dim3(256), lds, stream,
                       static_cast<const uint16_t*>(x), (int)K, (int)r, s, v, x_codes, x_scales,
                       u, prequant);
  return launch_status("act_prep");
}

int32_t gemm_impl(const uint8_t* x_codes, const uint8_t* x_scales, const float* u, int64_t M,
                  int64_t N, int64_t K, int32_t r, const uint8_t* w_codes,
                  const uint8_t* w_scales, const uint16_t* wv, const float* bias, void* y,
                  int32_t y_dtype, hipStream_t stream) {
  ASP_TRY(check_mk(M, K));
  ASP_TRY(check_rank(r));
  if (N < 1 || N > INT32_MAX) return fail(ASP_ERR_SHAPE, "N=%lld outside [1, 2^31)", (long long)N);
  if (y_dtype != ASP_F32 && y_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "y_dtype=%d", y_dtype);
  if (M == 0) return ASP_OK;
  ASP_TRY(check_ptr(x_codes, "x_codes", true));
  ASP_TRY(check_ptr(x_scales, "x_scales", true));
  ASP_TRY(check_ptr(u, "u", r > 0));
  ASP_TRY(check_ptr(w_codes, "w_codes", true));
  ASP_TRY(check_ptr(w_scales, "w_scales", true));
  ASP_TRY(check_ptr(wv, "wv", r > 0));
  ASP_TRY(check_ptr(bias, "bias", false));
  ASP_TRY(check_ptr(y, "y", true));
  const dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
  if (grid.y > 65535) return fail(ASP_ERR_SHAPE, "M=%lld too large for one launch", (long long)M);
  hipLaunchKernelGGL(k_gemm, grid, dim3(256), 0, stream, x_codes, x_scales, u, (int)M, (int)N,
                     (int)K, (int)r, w_codes, w_scales, wv, bias, y, (int)(y_dtype == ASP_BF16));
  return launch_status("gemm");
}

}  // namespace

extern "C" {

int32_t asp_quantize_nvfp4(const float* in, int64_t rows, int64_t cols, uint8_t* codes,
                           uint8_t* scales, void* stream) {
  clear_error();
  if (rows < 0 || cols <= 0 || cols % 16)
    return fail(ASP_ERR_SHAPE, "rows=%lld cols=%lld: need rows >= 0, cols a positive multiple of 16",
                (long long)rows, (long long)cols);
  if (rows == 0) return ASP_OK;
  ASP_TRY(check_ptr(in, "in", true));
  ASP_TRY(check_ptr(codes, "codes", true));
  ASP_TRY(check_ptr(scales, "scales", true));
  const int64_t n_half = rows * cols / 8;
  const int64_t blocks = (n_half + 255) / 256;
  if (blocks > INT32_MAX) return fail(ASP_ERR_SHAPE, "input too large for one launch");
  hipLaunchKernelGGL(k_quantize, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, in,
                     n_half, reinterpret_cast<uint32_t*>(codes), scales);
  return launch_status("quantize");
}

int32_t asp_dequantize_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int64_t cols, float* out, void* stream) {
  clear_error();
  if (rows < 0 || cols <= 0 || cols % 16)
    return fail(ASP_ERR_SHAPE, "rows=%lld cols=%lld: need rows >= 0, cols a positive multiple of 16",
                (long long)rows, (long long)cols);
  if (rows == 0) return ASP_OK;
  ASP_TRY(check_ptr(codes, "codes", true));
  ASP_TRY(check_ptr(scales, "scales", true));
  ASP_TRY(check_ptr(out, "out", true));
  const int64_t n_half = rows * cols / 8;
  const int64_t blocks = (n_half + 255) / 256;
  if (blocks > INT32_MAX) return fail(ASP_ERR_SHAPE, "input too large for one launch");
  hipLaunchKernelGGL(k_dequantize, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<const uint32_t*>(codes), scales, n_half, out);
  return launch_status("dequantize");
}

int32_t asp_act_prep(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                     const float* s, const float* v, uint8_t* x_codes, uint8_t* x_scales,
                     float* u, float* prequant, void* stream) {
  clear_error();
  return act_prep_impl(x, x_dtype, M, K, r, s, v, x_codes, x_scales, u, prequant,
                       (hipStream_t)stream);
}

int32_t asp_gemm_lowrank(const uint8_t* x_codes, const uint8_t* x_scales, const float* u,
                         int64_t M, int64_t N, int64_t K, int32_t r, const uint8_t* w_codes,
                         const uint8_t* w_scales, const uint16_t* wv, const float* bias, void* y,
                         int32_t y_dtype, void* stream) {
  clear_error();
  return gemm_impl(x_codes, x_scales, u, M, N, K, r, w_codes, w_scales, wv, bias, y, y_dtype,
                   (hipStream_t)stream);
}

int32_t asp_forward(const void* x, int32_t x_dtype, int64_t M, int64_t N, int64_t K, int32_t r,
                    const float* s, const float* v, const uint8_t* w_codes,
                    const uint8_t* w_scales, const uint16_t* wv, const float* bias, void* y,
                    int32_t y_dtype, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  size_t need = 0;
  ASP_TRY(asp_workspace_bytes(M, K, r, &need));
  if (N < 1 || N > INT32_MAX) return fail(ASP_ERR_SHAPE, "N=%lld outside [1, 2^31)", (long long)N);
  if (M == 0) return ASP_OK;
  if (!workspace) return fail(ASP_ERR_ARG, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(ASP_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(ASP_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, need);
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  uint8_t* base = static_cast<uint8_t*>(workspace);
  uint8_t* xc = base;
  uint8_t* xs = xc + up((size_t)M * K / 2);
  float* uu = r > 0 ? reinterpret_cast<float*>(xs + up((size_t)M * K / 16)) : nullptr;
  // validate the GEMM side before enqueuing anything
  if (y_dtype != ASP_F32 && y_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "y_dtype=%d", y_dtype);
  ASP_TRY(check_ptr(w_codes, "w_codes", true));
  ASP_TRY(check_ptr(w_scales, "w_scales", true));
  ASP_TRY(check_ptr(wv, "wv", r > 0));
  ASP_TRY(check_ptr(bias, "bias", false));
  ASP_TRY(check_ptr(y, "y", true));
  if ((N + BN - 1) / BN > INT32_MAX || (M + BM - 1) / BM > 65535)
    return fail(ASP_ERR_SHAPE, "M=%lld too large for one launch", (long long)M);
  ASP_TRY(act_prep_impl(x, x_dtype, M, K, r, s, v, xc, xs, uu, nullptr, (hipStream_t)stream));
  return gemm_impl(xc, xs, uu, M, N, K, r, w_codes, w_scales, wv, bias, y, y_dtype,
                   (hipStream_t)stream);
}

}  // extern "C"
