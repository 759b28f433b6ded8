// Device side of the SVDQuant-style INT4 (group 64) W4A4 arm (model card
// "FastWAM UR3 3-task -- 4-bit quantisations", method table: INT4 with groups
// of 64 for weights and activations, contracted on INT8 tensor cores, which
// are exact for 4-bit codes; the rank-r branch in 16 bits):
//
//   u      = x V''                 (k_prep_u, V'' = diag(1/s) V_r: partial sums)
//   x_hat  = float32(x * (1/s));   INT4 codes and bfloat16 scales per group of 64
//   y      = sum_g sx[m,g] sw[n,g] (sum_{k in g} qx[m,k] qw[n,k])
//          + bfloat16(u) L1^T + b
//
// The group products run on v_mfma_i32_16x16x64_i8: one instruction is one
// group of one 16 x 16 tile, exact in int32, then scaled by the product of the
// two bfloat16 scales (exact in float32) into float32 accumulators.  A code c
// is fed to the MFMA as the byte 16 c (its nibble in the high half of a byte,
// so unpacking two nibbles per byte is one mask and one shift-and-mask); the
// factor 256 is folded into the scale product.  Even and odd elements of a
// group land in different bytes, in the same order for both operands, so the
// (exact, integer) group sum is unchanged.
#include "asp_device.h"

namespace asp {
namespace {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGroupK = 64;

inline int64_t pad128(int64_t v) { return (v + 127) / 128 * 128; }

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

// --------------------------------------------------------------- quantiser

// Lane t handles 16 consecutive elements of a row; the 4 lanes of a group of
// 64 share its absolute maximum.  x_hat = float32(x * rs); scale =
// bfloat16(amax / 7); code = clamp(rint(x_hat / scale), -8, 7) (IEEE float32
// division, ties to even), stored as two's-complement nibbles, element 2j in
// the low nibble of byte j.  Scales (bfloat16 values, held as float32 so the
// GEMM uses them as they are) go to xs[g * Mp + m].
template <typename XT>
__global__ void __launch_bounds__(256) k_svdq_quant(const XT* __restrict__ x,
                                                    const float* __restrict__ rs, int M, int K,
                                                    int Mp, uint8_t* __restrict__ xc,
                                                    float* __restrict__ xs) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int cpr = K / 16;  // 16-element chunks per row (a multiple of 4)
  if (t >= (int64_t)M * cpr) return;  // whole 4-lane groups leave together
  const int64_t m = t / cpr;
  const int c = (int)(t % cpr);
  float v[16];
  if constexpr (sizeof(XT) == 2) {
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(x + m * K + 16 * c);
    const u32x4_t p0 = src[0], p1 = src[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_to_f32(p0[e] & 0xFFFFu);
      v[2 * e + 1] = bf16_to_f32(p0[e] >> 16);
      v[8 + 2 * e] = bf16_to_f32(p1[e] & 0xFFFFu);
      v[8 + 2 * e + 1] = bf16_to_f32(p1[e] >> 16);
    }
  } else {
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(x + m * K + 16 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x4_t p = src[e];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[4 * e + j] = p[j];
    }
  }
  const f32x4_t* rsv = reinterpret_cast<const f32x4_t*>(rs + 16 * c);
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x4_t r4 = rsv[e];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[4 * e + j] = v[4 * e + j] * r4[j];
      amax = fmaxf(amax, fabsf(v[4 * e + j]));
    }
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const uint16_t sb = bf16_rne(amax / 7.0f);
  const float sc = bf16_to_f32(sb);
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    int q = sc > 0.0f ? (int)__builtin_rintf(v[e] / sc) : 0;
    q = q < -8 ? -8 : (q > 7 ? 7 : q);
    w[e >> 3] |= (uint32_t)(q & 15) << (4 * (e & 7));
  }
  *reinterpret_cast<uint2*>(xc + m * (K / 2) + 8 * c) = make_uint2(w[0], w[1]);
  if ((c & 3) == 0) xs[(int64_t)(c >> 2) * Mp + m] = sc;
}

// ---------------------------------------------------------------- the GEMM

struct SvdqGemmArgs {
  const uint8_t* xc;   // M x K/2 codes
  const float* xs;     // (K/64) x Mp scales (bfloat16 values as float32)
  const float* u;      // u_slices partial sums, [s][M][u_ld] float32, u_ld = r rounded up to 32,
                       // the columns past r zero (summed in slice order)
  const uint8_t* wc;   // N x K/2 codes
  const uint16_t* ws;  // (K/64) x Np bfloat16 scales
  const uint16_t* l1;  // N x RP bfloat16 (zero padded)
  const float* bias;   // N or null
  void* y;             // M x N
  int M, N, K, r, Mp, Np, u_slices, u_ld, y_bf16;
};

// two nibble-packed words (16 codes) -> 16 bytes 16*c for the i8 MFMA: the
// even elements of each word, then the odd ones
__device__ __forceinline__ i32x4_t unpack16(uint2 w) {
  const uint32_t m = 0xF0F0F0F0u;
  return i32x4_t{(int)((w.x << 4) & m), (int)(w.x & m), (int)((w.y << 4) & m), (int)(w.y & m)};
}

// Workgroup: a BM x BN tile of y (BM = BN = 32 TI; TI = 2 is launched), 4
// waves as 2 x 2, each wave TI x TI MFMA tiles of 16 x 16.  Per group of 64 the workgroup's code
// rows (32 bytes each) and scales are loaded into registers two groups ahead
// and written to one of two LDS buffers one group ahead, so each load has two
// groups of compute to land in; the compiler waits only on the registers a
// write uses.  MFMA lane layout (checked on gfx950): lane l supplies row l%16
// of A (column l%16 of B) with the 16 bytes of K-quarter l/16; output element
// v is row 4 (l/16) + v, column l%16.
template <int TI, int RPK>
__global__ void __launch_bounds__(256) k_svdq_gemm(SvdqGemmArgs a) {
  constexpr int BM = 32 * TI, BN = 32 * TI;
  constexpr int CX = BM * 2, CW = BN * 2;  // 16-byte pieces of codes per group
  static_assert(CX + CW <= 512, "two pieces of codes per thread at most");
  __shared__ __attribute__((aligned(16))) uint8_t sxc[2][BM * 32];
  __shared__ __attribute__((aligned(16))) uint8_t swc[2][BN * 32];
  __shared__ __attribute__((aligned(16))) float sxs[2][BM];
  __shared__ __attribute__((aligned(16))) uint16_t sws[2][BN];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1, q = lane >> 4, l16 = lane & 15;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  const int M = a.M, N = a.N, KB = a.K / 2, G = a.K / kGroupK;

  // the pieces this thread moves: code piece tid (and tid + 256 when there are
  // more than 256), and scale piece tid - 0 / tid - BM/8 for the first threads
  struct Regs {
    u32x4_t c0, c1, sc;
  };
  auto piece_src = [&](int P, int g) -> const uint8_t* {
    const int64_t mr = min(m0 + (P >> 1), M - 1);
    const int64_t nr = min(n0 + max((P - CX) >> 1, 0), N - 1);
    return P < CX ? a.xc + mr * KB + 32 * g + 16 * (P & 1)
                  : a.wc + nr * KB + 32 * g + 16 * ((P - CX) & 1);
  };
  auto piece_dst = [&](int P, int b) -> uint8_t* {
    return P < CX ? &sxc[b][16 * P] : &swc[b][16 * (P - CX)];
  };
  constexpr int SX = BM / 4, SW = BN / 8;  // 16-byte pieces of scales (float32 x, bf16 w)
  // every thread issues the same loads (no lane-dependent branch around a
  // load, so the compiler can count them and wait only for the ones a store
  // needs): scale piece min(tid, SX + SW - 1), its address selected per lane
  static_assert(CX + CW == 256 || CX + CW == 512, "one or two code pieces per thread");
  auto gload = [&](int g, Regs& r) {
    r.c0 = *reinterpret_cast<const u32x4_t*>(piece_src(tid, g));
    if constexpr (CX + CW == 512) r.c1 = *reinterpret_cast<const u32x4_t*>(piece_src(tid + 256, g));
    const int sp = min(tid, SX + SW - 1);
    const void* src = sp < SX ? static_cast<const void*>(a.xs + (int64_t)g * a.Mp + m0 + 4 * sp)
                              : static_cast<const void*>(a.ws + (int64_t)g * a.Np + n0 +
                                                         8 * max(sp - SX, 0));
    r.sc = *reinterpret_cast<const u32x4_t*>(src);
  };
  auto sstore = [&](int b, const Regs& r) {
    *reinterpret_cast<u32x4_t*>(piece_dst(tid, b)) = r.c0;
    if constexpr (CX + CW == 512) *reinterpret_cast<u32x4_t*>(piece_dst(tid + 256, b)) = r.c1;
    if (tid < SX)
      *reinterpret_cast<u32x4_t*>(&sxs[b][4 * tid]) = r.sc;
    else if (tid < SX + SW)
      *reinterpret_cast<u32x4_t*>(&sws[b][8 * (tid - SX)]) = r.sc;
  };
  auto barrier = [&]() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  f32x4_t out[TI][TI];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TI; ++j) out[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

  auto compute = [&](int b) {
    i32x4_t A[TI], B[TI];
    float sx[TI][4], sw[TI];
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int row = 16 * (TI * wm + i) + l16;
      A[i] = unpack16(*reinterpret_cast<const uint2*>(&sxc[b][row * 32 + 8 * q]));
      const f32x4_t s4 = *reinterpret_cast<const f32x4_t*>(&sxs[b][16 * (TI * wm + i) + 4 * q]);
#pragma unroll
      for (int v = 0; v < 4; ++v) sx[i][v] = s4[v];
    }
#pragma unroll
    for (int j = 0; j < TI; ++j) {
      const int row = 16 * (TI * wn + j) + l16;
      B[j] = unpack16(*reinterpret_cast<const uint2*>(&swc[b][row * 32 + 8 * q]));
      // the 2^-8 undoes the 16 x 16 of the byte encoding (exact)
      sw[j] = bf16_to_f32(sws[b][row]) * 0.00390625f;
    }
    const i32x4_t zero = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TI; ++j) {
        const i32x4_t acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[i], B[j], zero, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) out[i][j][v] = fmaf((float)acc[v], sx[i][v] * sw[j], out[i][j][v]);
      }
  };

  // group k is held in register set k % 2 and LDS buffer k % 2 (G is even).
  // Loads past the last group re-read group G - 1 (valid memory, never used),
  // so that no load sits behind a branch.
  Regs r0, r1;
  gload(0, r0);
  gload(1, r1);
  sstore(0, r0);
  gload(min(2, G - 1), r0);
  barrier();
  for (int g = 0; g < G; g += 2) {
    compute(0);
    sstore(1, r1);                   // group g + 1 (buffer 1 was last read at g - 1)
    gload(min(g + 3, G - 1), r1);
    barrier();
    compute(1);
    sstore(0, r0);                   // group g + 2 (unused after the last pair)
    gload(min(g + 4, G - 1), r0);
    barrier();
  }

  // rank-r branch: bfloat16(u) L1^T on v_mfma_f32_16x16x32_bf16 (lane l: row
  // l%16, k-slots 8 (l/16) .. +7 of both operands), then the bias.  u is
  // [slices][M][RP] float32 with the columns past r zero; the slices are added
  // in order, every load in flight together.
  if constexpr (RPK > 0) {
    constexpr int RP = 32 * RPK;
#pragma unroll
    for (int ks = 0; ks < RPK; ++ks) {
      bf16x8_t au[TI], bl[TI];
#pragma unroll
      for (int i = 0; i < TI; ++i) {
        const int64_t m = min(m0 + 16 * (TI * wm + i) + l16, M - 1);
        f32x4_t lo[8], hi[8];
#pragma unroll
        for (int sl = 0; sl < 8; ++sl) {
          const float* p = a.u + ((int64_t)min(sl, a.u_slices - 1) * M + m) * RP + 32 * ks + 8 * q;
          lo[sl] = *reinterpret_cast<const f32x4_t*>(p);
          hi[sl] = *reinterpret_cast<const f32x4_t*>(p + 4);
        }
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
          for (int sl = 0; sl < 8; ++sl) {
            s0 += sl < a.u_slices ? lo[sl][e] : 0.0f;
            s1 += sl < a.u_slices ? hi[sl][e] : 0.0f;
          }
          f[e] = s0;
          f[4 + e] = s1;
        }
        au[i] = bf16x8_rne(f);
      }
#pragma unroll
      for (int j = 0; j < TI; ++j) {
        const int64_t n = min(n0 + 16 * (TI * wn + j) + l16, N - 1);
        bl[j] = __builtin_bit_cast(bf16x8_t,
                                   *reinterpret_cast<const u32x4_t*>(a.l1 + n * RP + 32 * ks + 8 * q));
      }
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TI; ++j)
          out[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(au[i], bl[j], out[i][j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < TI; ++j) {
    const int n = n0 + 16 * (TI * wn + j) + l16;
    if (n >= N) continue;
    const float b = a.bias ? a.bias[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = m0 + 16 * (TI * wm + i) + 4 * q + v;
        if (m >= M) continue;
        const float val = out[i][j][v] + b;
        if (a.y_bf16)
          static_cast<uint16_t*>(a.y)[(int64_t)m * N + n] = bf16_rne(val);
        else
          static_cast<float*>(a.y)[(int64_t)m * N + n] = val;
      }
  }
}

// ----------------------------------------------------------------- host side

struct SvdqWs {
  size_t xc, xs, up, total;
};

SvdqWs svdq_ws(int64_t M, int64_t K, int32_t r) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  SvdqWs L;
  L.xc = 0;
  L.xs = up((size_t)M * K / 2);
  L.up = L.xs + up((size_t)pad128(M) * (K / kGroupK) * 4);
  L.total = L.up + up(act_prep_scratch_bytes(M, K, r));
  return L;
}

int32_t svdq_shape(int64_t M, int64_t N, int64_t K, int32_t r, int32_t y_dtype) {
  ASP_TRY(check_mk(M, K));
  ASP_TRY(check_rank(r));
  if (N < 1 || N > INT32_MAX || M * N > ((int64_t)1 << 40))
    return fail(ASP_ERR_SHAPE, "N=%lld", (long long)N);
  if (y_dtype != ASP_F32 && y_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "y_dtype=%d", y_dtype);
  return ASP_OK;
}

int32_t launch_quant(const void* x, int32_t x_dtype, int64_t M, int64_t K, const float* rs,
                     uint8_t* xc, float* xs, hipStream_t st) {
  const int64_t lanes = M * (K / 16);
  const unsigned blocks = (unsigned)((lanes + 255) / 256);
  const int Mp = (int)pad128(M);
  if (x_dtype == ASP_BF16)
    k_svdq_quant<uint16_t><<<blocks, 256, 0, st>>>(static_cast<const uint16_t*>(x), rs, (int)M,
                                                   (int)K, Mp, xc, xs);
  else
    k_svdq_quant<float><<<blocks, 256, 0, st>>>(static_cast<const float*>(x), rs, (int)M, (int)K,
                                                Mp, xc, xs);
  return launch_status("svdq quantise");
}

int32_t launch_gemm(const SvdqGemmArgs& a, hipStream_t st) {
  // 64 x 64 tiles (2 x 2 MFMA tiles per wave, 4 waves per SIMD): the
  // per-group scaling after every MFMA is a chain of dependent VALU steps,
  // hidden by other waves.  (A 128 x 128 tile, 4 x 4 per wave, needs 256
  // VGPRs -- 2 waves per SIMD -- and was slower at M = 4096, K = N = 3072.)
  const int rp = a.r == 0 ? 0 : (a.r + 31) / 32;
  const dim3 grid((unsigned)((a.N + 63) / 64), (unsigned)((a.M + 63) / 64));
  if (rp == 0) k_svdq_gemm<2, 0><<<grid, 256, 0, st>>>(a);
  else if (rp == 1) k_svdq_gemm<2, 1><<<grid, 256, 0, st>>>(a);
  else k_svdq_gemm<2, 2><<<grid, 256, 0, st>>>(a);
  return launch_status("svdq gemm");
}

}  // namespace
}  // namespace asp

using namespace asp;

extern "C" {

int32_t asp_svdq_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r, size_t* bytes) {
  clear_error();
  ASP_TRY(svdq_shape(M, N, K, r, ASP_F32));
  if (!bytes) return fail(ASP_ERR_ARG, "null output pointer");
  *bytes = svdq_ws(M, K, r).total;
  return ASP_OK;
}

int32_t asp_svdq_act_quant(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                           const uint8_t* prep_pack, uint8_t* x_codes, float* x_scales,
                           void* stream) {
  clear_error();
  ASP_TRY(check_mk(M, K));
  if (x_dtype != ASP_F32 && x_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "x_dtype=%d", x_dtype);
  if (M == 0) return ASP_OK;
  ASP_TRY(check_ptr(x, "x", true));
  ASP_TRY(check_ptr(prep_pack, "prep_pack", true));
  ASP_TRY(check_ptr(x_codes, "x_codes", true));
  ASP_TRY(check_ptr(x_scales, "x_scales", true));
  const PrepPackLayout P = prep_pack_layout(K, 0);
  return launch_quant(x, x_dtype, M, K, reinterpret_cast<const float*>(prep_pack + P.cvec), x_codes,
                      x_scales, (hipStream_t)stream);
}

int32_t asp_svdq_gemm(const uint8_t* x_codes, const float* x_scales, const float* u, int64_t M,
                      int64_t N, int64_t K, int32_t r, const uint8_t* w_codes,
                      const uint16_t* w_scales, const uint16_t* l1, const float* bias, void* y,
                      int32_t y_dtype, void* stream) {
  clear_error();
  ASP_TRY(svdq_shape(M, N, K, r, y_dtype));
  if (M == 0) return ASP_OK;
  ASP_TRY(check_ptr(x_codes, "x_codes", true));
  ASP_TRY(check_ptr(x_scales, "x_scales", true));
  ASP_TRY(check_ptr(u, "u", r > 0));
  ASP_TRY(check_ptr(w_codes, "w_codes", true));
  ASP_TRY(check_ptr(w_scales, "w_scales", true));
  ASP_TRY(check_ptr(l1, "l1", r > 0));
  ASP_TRY(check_ptr(bias, "bias", false));
  ASP_TRY(check_ptr(y, "y", true));
  SvdqGemmArgs a = {x_codes, x_scales, u, w_codes, w_scales, l1, bias, y,
                    (int)M, (int)N, (int)K, r, (int)pad128(M), (int)pad128(N), 1,
                    (r + 31) / 32 * 32, y_dtype == ASP_BF16};
  return launch_gemm(a, (hipStream_t)stream);
}

int32_t asp_svdq_forward(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                         const uint8_t* prep_pack, const uint8_t* w_codes,
                         const uint16_t* w_scales, const uint16_t* l1, const float* bias,
                         int64_t N, void* y, int32_t y_dtype, void* workspace,
                         size_t workspace_bytes, void* stream) {
  clear_error();
  ASP_TRY(svdq_shape(M, N, K, r, y_dtype));
  if (x_dtype != ASP_F32 && x_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "x_dtype=%d", x_dtype);
  if (M == 0) return ASP_OK;
  ASP_TRY(check_ptr(x, "x", true));
  ASP_TRY(check_ptr(prep_pack, "prep_pack", true));
  ASP_TRY(check_ptr(w_codes, "w_codes", true));
  ASP_TRY(check_ptr(w_scales, "w_scales", true));
  ASP_TRY(check_ptr(l1, "l1", r > 0));
  ASP_TRY(check_ptr(bias, "bias", false));
  ASP_TRY(check_ptr(y, "y", true));
  if (!workspace) return fail(ASP_ERR_ARG, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(ASP_ERR_ALIGN, "workspace must be 256-byte aligned");
  const SvdqWs L = svdq_ws(M, K, r);
  if (workspace_bytes < L.total)
    return fail(ASP_ERR_WORKSPACE, "workspace: %zu bytes, need %zu", workspace_bytes, L.total);
  uint8_t* base = static_cast<uint8_t*>(workspace);
  const hipStream_t st = (hipStream_t)stream;
  const PrepPackLayout P = prep_pack_layout(K, r);
  int slices = 0;
  float* upart = reinterpret_cast<float*>(base + L.up);
  if (r > 0) {
    const PrepCall pc = {x, prep_pack, nullptr, nullptr, nullptr, nullptr, upart,
                         workspace_bytes - L.up};
    ASP_TRY(act_prep_impl(1, 1, &pc, x_dtype, M, K, r, st));
    slices = (int)(act_prep_scratch_bytes(M, K, r) / ((size_t)M * P.rp32 * sizeof(float)));
  }
  ASP_TRY(launch_quant(x, x_dtype, M, K, reinterpret_cast<const float*>(prep_pack + P.cvec),
                       base + L.xc, reinterpret_cast<float*>(base + L.xs), st));
  SvdqGemmArgs a = {base + L.xc, reinterpret_cast<const float*>(base + L.xs), upart, w_codes,
                    w_scales, l1, bias, y, (int)M, (int)N, (int)K, r, (int)pad128(M),
                    (int)pad128(N), slices, P.rp32, y_dtype == ASP_BF16};
  return launch_gemm(a, st);
}

}  // extern "C"
