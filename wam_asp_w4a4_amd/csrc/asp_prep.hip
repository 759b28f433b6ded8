// Fused activation prep on gfx950: x/s, block Hadamard, u = x_tilde V,
// deflation x_tilde - u V^T, NVFP4 quantise + pack (model card "FastWAM UR3
// 3-task -- 4-bit quantisations", section "What ASP is, and what the deflated
// form means").
//
// Two kernels, because every element of a row's deflated value needs the
// row's full reduction u = x_tilde V first:
//
//  k_prep_u      u partial sums over K-slices.  u = x_tilde V = x (diag(1/s) H V)
//                = x V'', with V'' a per-layer constant, so this is a thin GEMM
//                on the raw input: MFMA 32x32x16 bf16, x exact in bf16 (an fp32
//                x is split into bf16 hi + lo), V'' split into bf16 hi + lo
//                (about 16 significant bits; the dropped lo*lo term is below
//                fp32 rounding of the sum).  Slices are summed in a fixed order
//                by the second kernel, so results are deterministic.
//  k_prep_quant  one wave per (32 rows, 128-column Hadamard block): load 8
//                consecutive columns per lane, scale by 1/(s sqrt 128), six
//                in-register butterfly stages, the seventh across lane halves
//                with v_permlane32_swap, which also leaves the values in the
//                32x32 MFMA accumulator layout; the deflation then runs as
//                MFMA (V bf16 hi/lo) x (-u bf16 hi/lo) accumulated onto
//                x_tilde; finally the NVFP4 quantiser and the code packing.
#include "asp_device.h"

namespace asp {
namespace {

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

// Butterfly across lane halves for the value pair (x, y) that differ in the
// column bit held in-register, while the lane-half bit h selects the column
// bit being transformed.  On return lane half 0 holds x's two outputs and lane
// half 1 holds y's: the in-register bit and the lane-half bit trade places.
__device__ __forceinline__ void half_swap_butterfly(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(y), false, false);
  const float a = bitsf(r[0]), b = bitsf(r[1]);
  x = a + b;
  y = a - b;
}

// Exchange so that lane half 0 gets (x of both halves) and half 1 gets (y of both).
__device__ __forceinline__ void half_swap(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = r[0];
  y = r[1];
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 q) { return __builtin_bit_cast(bf16x8_t, q); }

__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16_rne(v);
  lo = f32_to_bf16_rne(v - bits_f32((uint32_t)hi << 16));
}

// ---------------------------------------------------------------------------
// k_prep_u: workgroup = 4 waves x 32 rows; blockIdx.y selects a K-slice.
// A operand (rows of x): lane l supplies row l%32, K-elements 8*(l/32)..+7 of
// each 16-step; B operand (columns of V''): lane l supplies column l%32.
constexpr int kUChunk = 128;

template <typename XT, int CT>
__global__ void __launch_bounds__(256) k_prep_u(const XT* __restrict__ x, int M, int K, int r,
                                                const uint16_t* __restrict__ vth,
                                                const uint16_t* __restrict__ vtl,
                                                float* __restrict__ u_part, int kslice) {
  __shared__ uint4 sv[2][CT * 32][kUChunk / 8 + 1];  // V''^T chunk, hi and lo, padded rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int row0 = blockIdx.x * 128 + wave * 32;
  const int64_t mc = min(row0 + l32, M - 1);
  const int kb = blockIdx.y * kslice, ke = min(K, kb + kslice);

  // one accumulator per product term, so consecutive MFMAs are independent
  f32x16_t acc[CT], acc2[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = acc2[c][v] = 0.0f;

  for (int k0 = kb; k0 < ke; k0 += kUChunk) {
    // this lane's x fragments for the chunk (issued before the barrier)
    uint4 xa[8];
    uint4 xb[8];  // fp32 input: second half of the 8 values
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const XT* p = x + mc * K + k0 + 16 * ks + 8 * h;
      if constexpr (sizeof(XT) == 2) {
        xa[ks] = *reinterpret_cast<const uint4*>(p);
      } else {
        xa[ks] = reinterpret_cast<const uint4*>(p)[0];
        xb[ks] = reinterpret_cast<const uint4*>(p)[1];
      }
    }
    // stage V''^T for the chunk: CT*32 rows x 128 k, two pieces, 16 bytes per load
    for (int i = tid; i < 2 * CT * 32 * (kUChunk / 8); i += 256) {
      const int piece = i / (CT * 32 * (kUChunk / 8));
      const int rem = i % (CT * 32 * (kUChunk / 8));
      const int c = rem / (kUChunk / 8), seg = rem % (kUChunk / 8);
      const uint16_t* src = piece ? vtl : vth;
      sv[piece][c][seg] = *reinterpret_cast<const uint4*>(src + (int64_t)c * K + k0 + seg * 8);
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      bf16x8_t a_hi, a_lo;
      if constexpr (sizeof(XT) == 2) {
        a_hi = as_bf16x8(xa[ks]);
      } else {
        const float f[8] = {bitsf(xa[ks].x), bitsf(xa[ks].y), bitsf(xa[ks].z), bitsf(xa[ks].w),
                            bitsf(xb[ks].x), bitsf(xb[ks].y), bitsf(xb[ks].z), bitsf(xb[ks].w)};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          uint16_t hi, lo;
          split_bf16(f[e], hi, lo);
          a_hi[e] = bf16_from_bits(hi);
          a_lo[e] = bf16_from_bits(lo);
        }
      }
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const bf16x8_t b_hi = as_bf16x8(sv[0][c * 32 + l32][2 * ks + h]);
        const bf16x8_t b_lo = as_bf16x8(sv[1][c * 32 + l32][2 * ks + h]);
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi, b_hi, acc[c], 0, 0, 0);
        acc2[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi, b_lo, acc2[c], 0, 0, 0);
        if constexpr (sizeof(XT) == 4)
          acc2[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo, b_hi, acc2[c], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // accumulator element v of lane l: row 8*(v/4) + 4*(l/32) + v%4, column l%32
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const int col = c * 32 + l32;
    if (col >= r) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = row0 + 8 * (v >> 2) + 4 * h + (v & 3);
      if (row < M) u_part[((int64_t)blockIdx.y * M + row) * r + col] = acc[c][v] + acc2[c][v];
    }
  }
}

// ---------------------------------------------------------------------------
// k_prep_quant: workgroup = 4 waves sharing 32 rows; wave w of workgroup
// (i, j) handles 128-column blocks 4j + w, 4j + w + 4*gridDim.y, ...
template <typename XT, int KS>
__global__ void __launch_bounds__(256) k_prep_quant(const XT* __restrict__ x, int M, int K, int r,
                                                    const float* __restrict__ cvec,
                                                    const uint16_t* __restrict__ vh,
                                                    const uint16_t* __restrict__ vl,
                                                    const float* __restrict__ u_part, int S,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales,
                                                    float* __restrict__ u_out,
                                                    float* __restrict__ pre) {
  constexpr int RP = KS * 16;  // padded rank (row stride of vh / vl)
  __shared__ float us[32][RP > 0 ? RP + 1 : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int m0 = blockIdx.x * 32;
  const int m = m0 + l32;
  const int64_t mc = min(m, M - 1);
  const bool mok = m < M;
  const int nblk = K / 128;

  // -u for the 32 rows, as the bf16 hi/lo B operand of the deflation MFMA
  bf16x8_t nuh[KS > 0 ? KS : 1], nul[KS > 0 ? KS : 1];
  if constexpr (KS > 0) {
    for (int i = tid; i < 32 * RP; i += 256) {
      const int rr = i / RP, c = i % RP;
      float acc = 0.0f;
      if (c < r && m0 + rr < M)
        for (int s = 0; s < S; ++s) acc += u_part[((int64_t)s * M + m0 + rr) * r + c];
      us[rr][c] = acc;
      if (blockIdx.y == 0 && c < r && m0 + rr < M) u_out[(int64_t)(m0 + rr) * r + c] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint16_t hi, lo;
        split_bf16(-us[l32][16 * ks + 8 * h + e], hi, lo);
        nuh[ks][e] = bf16_from_bits(hi);
        nul[ks][e] = bf16_from_bits(lo);
      }
  }

  for (int b = blockIdx.y * 4 + wave; b < nblk; b += gridDim.y * 4) {
    const int col0 = b * 128;
    // w[g][e]: column col0 + 16g + 8h + e
    float w[8][8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      float cv[8];
      load8(x + mc * K + col0 + 16 * g + 8 * h, w[g]);
      load8(cvec + col0 + 16 * g + 8 * h, cv);
#pragma unroll
      for (int e = 0; e < 8; ++e) w[g][e] *= cv[e];
    }
    // Sylvester butterflies on column bits 0..2 (index e) and 4..6 (index g)
#pragma unroll
    for (int hs = 1; hs < 8; hs <<= 1)
#pragma unroll
      for (int g = 0; g < 8; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & hs) == 0) {
            const float a = w[g][e], c = w[g][e + hs];
            w[g][e] = a + c;
            w[g][e + hs] = a - c;
          }
#pragma unroll
    for (int gs = 1; gs < 8; gs <<= 1)
#pragma unroll
      for (int g = 0; g < 8; ++g)
        if ((g & gs) == 0)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float a = w[g][e], c = w[g + gs][e];
            w[g][e] = a + c;
            w[g + gs][e] = a - c;
          }
    // column bit 3 lives in the lane half: butterfly across halves on the
    // pairs (e, e+4).  Afterwards the lane half holds column bit 2 and the
    // pair slot holds column bit 3 -- the MFMA accumulator layout, where
    // element v = 4a + b of tile t is column 32t + 8a + 4h + b.
    f32x16_t acc[4];
#pragma unroll
    for (int g = 0; g < 8; ++g)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        float lo = w[g][bb], hi = w[g][bb + 4];
        half_swap_butterfly(lo, hi);
        const int a = 2 * (g & 1);
        acc[g >> 1][4 * a + bb] = lo;
        acc[g >> 1][4 * (a + 1) + bb] = hi;
      }
    if constexpr (KS > 0) {
      // x_d = x_tilde - u V^T, transposed: rows of the MFMA are the columns
      // of this block (A = V rows), its columns are the 32 rows (B = -u).
      // the four tiles' MFMAs are interleaved so that consecutive MFMAs are
      // independent (no back-to-back accumulator dependence)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8_t a_hi[4], a_lo[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int64_t vrow = (int64_t)(col0 + 32 * t + l32) * RP + 16 * ks + 8 * h;
          a_hi[t] = as_bf16x8(*reinterpret_cast<const uint4*>(vh + vrow));
          a_lo[t] = as_bf16x8(*reinterpret_cast<const uint4*>(vl + vrow));
        }
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[t], nuh[ks], acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_hi[t], nul[ks], acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a_lo[t], nuh[ks], acc[t], 0, 0, 0);
      }
    }
    // NVFP4: block g = columns col0 + 16g .. +15; this lane holds columns
    // 16g + 4h + bb (slot 0) and 16g + 8 + 4h + bb (slot 1), the other lane
    // half the rest.
    float amax[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int t = g >> 1, a = 2 * (g & 1);
      float mx = 0.0f;
#pragma unroll
      for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf(acc[t][4 * a + i]));
      amax[g] = mx;
    }
#pragma unroll
    for (int g = 0; g < 8; g += 2) {
      uint32_t p = fbits(amax[g]), q = fbits(amax[g + 1]);
      half_swap(p, q);  // half 0: block g of both halves; half 1: block g+1
      uint32_t both = fbits(fmaxf(bitsf(p), bitsf(q)));
      uint32_t both2 = both;
      half_swap(both, both2);  // everyone: (block g, block g+1)
      amax[g] = bitsf(both);
      amax[g + 1] = bitsf(both2);
    }
    uint8_t* crow = codes + mc * (K / 2);
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const int t = g >> 1, a = 2 * (g & 1);
      const uint32_t sc = block_scale_code(amax[g]);
      const float sd = e4m3_decode(sc);
      uint32_t g0 = 0, g1 = 0;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        g0 |= e2m1_code(acc[t][4 * a + bb], sd) << (4 * bb);
        g1 |= e2m1_code(acc[t][4 * (a + 1) + bb], sd) << (4 * bb);
      }
      half_swap(g0, g1);  // half 0: columns 16g+0..3 | 4..7, half 1: 8..11 | 12..15
      const uint32_t word = g0 | (g1 << 16);
      if (mok) {
        *reinterpret_cast<uint32_t*>(crow + (col0 + 16 * g + 8 * h) / 2) = word;
        if (h == 0) scales[mc * (K / 16) + (col0 + 16 * g) / 16] = (uint8_t)sc;
        if (pre) {
          float* prow = pre + mc * K + col0 + 16 * g + 4 * h;
          reinterpret_cast<float4*>(prow)[0] =
              make_float4(acc[t][4 * a], acc[t][4 * a + 1], acc[t][4 * a + 2], acc[t][4 * a + 3]);
          reinterpret_cast<float4*>(prow + 8)[0] =
              make_float4(acc[t][4 * a + 4], acc[t][4 * a + 5], acc[t][4 * a + 6], acc[t][4 * a + 7]);
        }
      }
    }
  }
}

// K-slices for the u partial sums: enough workgroups to cover the chip,
// each slice a whole number of 128-element chunks.
void u_slicing(int64_t M, int64_t K, int* S, int* kslice) {
  const int64_t row_tiles = (M + 127) / 128;
  const int64_t chunks = K / kUChunk;
  int64_t s = (256 + row_tiles - 1) / row_tiles;
  s = s < 1 ? 1 : (s > chunks ? chunks : s);
  const int64_t per = (chunks + s - 1) / s;
  *kslice = (int)(per * kUChunk);
  *S = (int)((chunks + per - 1) / per);
}

template <typename XT>
int32_t launch_prep(const XT* x, int64_t M, int64_t K, int32_t r, const uint8_t* pack,
                    uint8_t* x_codes, uint8_t* x_scales, float* u, float* prequant, float* u_part,
                    hipStream_t stream) {
  PrepPackLayout L = prep_pack_layout(K, r);
  const float* cvec = reinterpret_cast<const float*>(pack + L.cvec);
  const uint16_t* vth = reinterpret_cast<const uint16_t*>(pack + L.vt_hi);
  const uint16_t* vtl = reinterpret_cast<const uint16_t*>(pack + L.vt_lo);
  const uint16_t* vh = reinterpret_cast<const uint16_t*>(pack + L.v_hi);
  const uint16_t* vl = reinterpret_cast<const uint16_t*>(pack + L.v_lo);
  int S = 0, kslice = 0;
  if (r > 0) {
    u_slicing(M, K, &S, &kslice);
    const dim3 ga((unsigned)((M + 127) / 128), (unsigned)S);
    if (L.rp32 == 32)
      hipLaunchKernelGGL((k_prep_u<XT, 1>), ga, dim3(256), 0, stream, x, (int)M, (int)K, (int)r, vth, vtl, u_part, kslice);
    else
      hipLaunchKernelGGL((k_prep_u<XT, 2>), ga, dim3(256), 0, stream, x, (int)M, (int)K, (int)r, vth, vtl, u_part, kslice);
    ASP_TRY(launch_status("prep_u"));
  }
  const int64_t nblk = K / 128;
  const dim3 gb((unsigned)((M + 31) / 32), (unsigned)((nblk + 3) / 4));
#define ASP_PREP_QUANT(KS_)                                                                     \
  hipLaunchKernelGGL((k_prep_quant<XT, KS_>), gb, dim3(256), 0, stream, x, (int)M, (int)K, (int)r, \
                     cvec, vh, vl, u_part, S, x_codes, x_scales, u, prequant)
  switch (L.rp16 / 16) {
    case 0: ASP_PREP_QUANT(0); break;
    case 1: ASP_PREP_QUANT(1); break;
    case 2: ASP_PREP_QUANT(2); break;
    case 3: ASP_PREP_QUANT(3); break;
    default: ASP_PREP_QUANT(4); break;
  }
#undef ASP_PREP_QUANT
  return launch_status("prep_quant");
}

}  // namespace

size_t act_prep_scratch_bytes(int64_t M, int64_t K, int32_t r) {
  if (r == 0 || M == 0) return 0;
  int S, kslice;
  u_slicing(M, K, &S, &kslice);
  return (size_t)S * (size_t)M * (size_t)r * sizeof(float);
}

int32_t act_prep_impl(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                      const uint8_t* prep_pack, uint8_t* x_codes, uint8_t* x_scales, float* u,
                      float* prequant, void* scratch, size_t scratch_bytes, hipStream_t stream) {
  ASP_TRY(check_mk(M, K));
  ASP_TRY(check_rank(r));
  if (x_dtype != ASP_F32 && x_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "x_dtype=%d", x_dtype);
  if (M == 0) return ASP_OK;
  ASP_TRY(check_ptr(x, "x", true));
  ASP_TRY(check_ptr(prep_pack, "prep_pack", true));
  ASP_TRY(check_ptr(x_codes, "x_codes", true));
  ASP_TRY(check_ptr(x_scales, "x_scales", true));
  ASP_TRY(check_ptr(u, "u", r > 0));
  ASP_TRY(check_ptr(prequant, "prequant", false));
  const size_t need = act_prep_scratch_bytes(M, K, r);
  if (need) {
    ASP_TRY(check_ptr(scratch, "workspace", true));
    if (scratch_bytes < need)
      return fail(ASP_ERR_WORKSPACE, "workspace %zu bytes, need %zu", scratch_bytes, need);
  }
  float* u_part = static_cast<float*>(scratch);
  if (x_dtype == ASP_F32)
    return launch_prep(static_cast<const float*>(x), M, K, r, prep_pack, x_codes, x_scales, u,
                       prequant, u_part, stream);
  return launch_prep(static_cast<const uint16_t*>(x), M, K, r, prep_pack, x_codes, x_scales, u,
                     prequant, u_part, stream);
}

}  // namespace asp

using namespace asp;

extern "C" {

int32_t asp_act_prep_workspace_bytes(int64_t M, int64_t K, int32_t r, size_t* bytes) {
  clear_error();
  ASP_TRY(check_mk(M, K));
  ASP_TRY(check_rank(r));
  if (!bytes) return fail(ASP_ERR_ARG, "null output pointer");
  *bytes = act_prep_scratch_bytes(M, K, r);
  return ASP_OK;
}

int32_t asp_act_prep(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                     const uint8_t* prep_pack, uint8_t* x_codes, uint8_t* x_scales, float* u,
                     float* prequant, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  return act_prep_impl(x, x_dtype, M, K, r, prep_pack, x_codes, x_scales, u, prequant, workspace,
                       workspace_bytes, (hipStream_t)stream);
}

}  // extern "C"
