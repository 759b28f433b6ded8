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

// Exchange across lane rows (16 lanes): even rows get (x of both rows), odd rows (y of both).
__device__ __forceinline__ void half_swap16(uint32_t& x, uint32_t& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(x, y, false, false);
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
// k_prep_quant: a wave works on units of 16 rows x one 128-column Hadamard
// block.  Lane l holds row l%16; its lane quarter q = l/16 selects columns.
//
//  load layout:  the lane holds columns 64*b + 16*q + j (b = 0..1, j = 0..15):
//                two runs of 16 consecutive columns, so loads are 32 bytes.
//  transform:    column bits 0..3 (j) and 6 (b) are butterflied in-register;
//                bit 4 (lane bit q0) and bit 5 (lane bit q1) across lane rows
//                with v_permlane16_swap / v_permlane32_swap on value pairs
//                that differ in column bit 2, resp. 3.  Each swap-butterfly
//                trades the lane bit with that register bit, which leaves the
//                lane quarter holding column bits 2..3: tile t = 16 columns,
//                the lane's 4 consecutive columns 16t + 4q + i -- exactly the
//                output layout of a 16x16 MFMA with the block's columns as
//                its rows and the 16 rows of x as its columns.
//  deflation:    acc_t += V[cols of tile t] (-u)^T via v_mfma_f32_16x16x32_bf16
//                with bf16 hi/lo splits (hi*hi + hi*lo + lo*hi).
//  quantise:     tile t is one NVFP4 block; its maximum across the four lane
//                quarters comes from two cross-lane maxima, and pairs of
//                tiles' 16-bit code groups are merged into 32-bit words by one
//                v_permlane16_swap.
//
// Workgroup = 4 waves on the same 16 rows; wave w of workgroup (i, j) takes
// blocks 4j + w, 4j + w + 4*gridDim.y, ...

__device__ __forceinline__ void swap16_butterfly(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(y), false, false);
  const float a = bitsf(r[0]), b = bitsf(r[1]);
  x = a + b;
  y = a - b;
}

__device__ __forceinline__ void load16(const float* p, float* v) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float4 a = reinterpret_cast<const float4*>(p)[k];
    v[4 * k] = a.x; v[4 * k + 1] = a.y; v[4 * k + 2] = a.z; v[4 * k + 3] = a.w;
  }
}

__device__ __forceinline__ void load16(const uint16_t* p, float* v) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[k];
    const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[8 * k + 2 * e] = bits_f32(w[e] << 16);
      v[8 * k + 2 * e + 1] = bits_f32(w[e] & 0xFFFF0000u);
    }
  }
}

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
  constexpr int RP = KS * 32;  // padded rank (row stride of vh / vl)
  __shared__ float us[16][RP > 0 ? RP + 1 : 1];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int m0 = blockIdx.x * 16;
  const int m = m0 + l16;
  const int64_t mc = min(m, M - 1);
  const bool mok = m < M;
  const int nblk = K / 128;

  // -u for the 16 rows, as the bf16 hi/lo B operand of the deflation MFMA:
  // lane supplies row l%16, K-elements 8q .. 8q+7 of each 32-step
  bf16x8_t nuh[KS > 0 ? KS : 1], nul[KS > 0 ? KS : 1];
  if constexpr (KS > 0) {
    for (int i = tid; i < 16 * RP; i += 256) {
      const int rr = i / RP, c = i % RP;
      float acc = 0.0f;
      if (c < r && m0 + rr < M)
        for (int s = 0; s < S; ++s) acc += u_part[((int64_t)s * M + m0 + rr) * r + c];
      us[rr][c] = acc;
      if (blockIdx.y == 0 && c < r && m0 + rr < M) u_out[(int64_t)(m0 + rr) * r + c] = acc;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint16_t hi, lo;
        split_bf16(-us[l16][32 * kk + 8 * q + e], hi, lo);
        nuh[kk][e] = bf16_from_bits(hi);
        nul[kk][e] = bf16_from_bits(lo);
      }
  }

  for (int b = blockIdx.y * 4 + wave; b < nblk; b += gridDim.y * 4) {
    const int col0 = b * 128;
    // w[bb][j]: column col0 + 64*bb + 16*q + j
    float w[2][16];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const int c = col0 + 64 * bb + 16 * q;
      float cv[16];
      load16(x + mc * K + c, w[bb]);
      load16(cvec + c, cv);
#pragma unroll
      for (int j = 0; j < 16; ++j) w[bb][j] *= cv[j];
    }
    // Sylvester butterflies on column bits 0..3 (j) and 6 (bb)
#pragma unroll
    for (int hs = 1; hs < 16; hs <<= 1)
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
          if ((j & hs) == 0) {
            const float a = w[bb][j], c = w[bb][j + hs];
            w[bb][j] = a + c;
            w[bb][j + hs] = a - c;
          }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float a = w[0][j], c = w[1][j];
      w[0][j] = a + c;
      w[1][j] = a - c;
    }
    // column bit 4 (lane bit q0) against column bit 2 (j bit 2), then column
    // bit 5 (lane bit q1) against column bit 3 (j bit 3)
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if ((j & 4) == 0) swap16_butterfly(w[bb][j], w[bb][j + 4]);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if ((j & 8) == 0) half_swap_butterfly(w[bb][j], w[bb][j + 8]);
    // now w[bb][j] is column 16*t + 4*q + (j & 3) with tile t = (j >> 2) + 4*bb
    f32x4_t acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[t][i] = w[t >> 2][4 * (t & 3) + i];
    if constexpr (KS > 0) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        bf16x8_t a_hi[8], a_lo[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t vrow = (int64_t)(col0 + 16 * t + l16) * RP + 32 * kk + 8 * q;
          a_hi[t] = as_bf16x8(*reinterpret_cast<const uint4*>(vh + vrow));
          a_lo[t] = as_bf16x8(*reinterpret_cast<const uint4*>(vl + vrow));
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi[t], nuh[kk], acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi[t], nul[kk], acc[t], 0, 0, 0);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo[t], nuh[kk], acc[t], 0, 0, 0);
      }
    }
    // NVFP4 per tile: maximum over the tile's 16 columns = 4 lane quarters
    uint32_t sc[8];
    float sd[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      float mx = fmaxf(fmaxf(fabsf(acc[t][0]), fabsf(acc[t][1])),
                       fmaxf(fabsf(acc[t][2]), fabsf(acc[t][3])));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      sc[t] = block_scale_code(mx);
      sd[t] = e4m3_decode(sc[t]);
    }
    uint8_t* crow = codes + mc * (K / 2) + col0 / 2;
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
      uint32_t g0 = 0, g1 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        g0 |= e2m1_code(acc[t][i], sd[t]) << (4 * i);
        g1 |= e2m1_code(acc[t + 1][i], sd[t + 1]) << (4 * i);
      }
      // even lane rows: tile t, columns 8*q1 .. +7; odd rows: tile t+1
      half_swap16(g0, g1);
      if (mok) {
        const int tt = t + (q & 1);
        *reinterpret_cast<uint32_t*>(crow + 8 * tt + 4 * (q >> 1)) = g0 | (g1 << 16);
      }
    }
    if (mok) {
      // lane quarter q stores the scales of tiles 2q and 2q+1
      const uint32_t pair = (q == 0 ? sc[0] | sc[1] << 8
                           : q == 1 ? sc[2] | sc[3] << 8
                           : q == 2 ? sc[4] | sc[5] << 8 : sc[6] | sc[7] << 8);
      *reinterpret_cast<uint16_t*>(scales + mc * (K / 16) + col0 / 16 + 2 * q) = (uint16_t)pair;
      if (pre) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
          *reinterpret_cast<float4*>(pre + mc * K + col0 + 16 * t + 4 * q) =
              make_float4(acc[t][0], acc[t][1], acc[t][2], acc[t][3]);
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
  const dim3 gb((unsigned)((M + 15) / 16), (unsigned)((nblk + 3) / 4));
#define ASP_PREP_QUANT(KS_)                                                                     \
  hipLaunchKernelGGL((k_prep_quant<XT, KS_>), gb, dim3(256), 0, stream, x, (int)M, (int)K, (int)r, \
                     cvec, vh, vl, u_part, S, x_codes, x_scales, u, prequant)
  switch (L.rp32 / 32) {
    case 0: ASP_PREP_QUANT(0); break;
    case 1: ASP_PREP_QUANT(1); break;
    default: ASP_PREP_QUANT(2); break;
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
