// Fused activation prep on gfx950: x/s, block Hadamard, u = x_tilde V,
// deflation x_tilde - u V^T, NVFP4 quantise + pack (model card "FastWAM UR3
// 3-task -- 4-bit quantisations", section "What ASP is, and what the deflated
// form means").  One kernel, k_prep; a workgroup owns 16 rows of x.
//
// Every element of a row's deflated value needs the row's full reduction
// u = x_tilde V first, so for r > 0 the workgroup covers the whole of K for
// its rows and works in two phases:
//
//  phase 1  u.  u = x_tilde V = x (diag(1/s) H V) = x V'', with V'' a per-layer
//           constant, so each wave contracts the raw rows of its Hadamard
//           blocks against V'' on MFMA 16x16x32 bf16 (x is exact in bf16; an
//           fp32 x is split into bf16 high + low; V'' is split into bf16 high +
//           low, about 16 significant bits, the dropped low*low term lying
//           below float32 rounding of the sum).  The waves' partial sums meet
//           in LDS and are added in a fixed order: results are deterministic.
//  phase 2  per (16 rows, 128-column block): scale by 1/(s sqrt 128), the
//           Sylvester butterflies in registers and across lane rows, the
//           deflation on MFMA, the NVFP4 quantiser and the packed stores.
//           The raw x fragments of phase 1 stay in registers when they fit.
//
// With r == 0 there is no phase 1; a workgroup then takes a strip of blocks
// and the grid also spans K.
#include "asp_device.h"

namespace asp {
namespace {

__device__ __forceinline__ uint32_t fbits(float f) { return __builtin_bit_cast(uint32_t, f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __builtin_bit_cast(float, u); }

// v_permlane32_swap / v_permlane16_swap on a value pair (x, y): lanes of the
// lower half (resp. even 16-lane row) end with (x of own lanes, x of partner
// lanes), lanes of the upper half (odd row) with (y of partner, y of own).
// Applied to pairs that differ in one register index bit, it trades that bit
// with the lane bit.
__device__ __forceinline__ void swap32(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane32_swap(fbits(x), fbits(y), false, false);
  x = bitsf(r[0]);
  y = bitsf(r[1]);
}

__device__ __forceinline__ void swap16(float& x, float& y) {
  const auto r = __builtin_amdgcn_permlane16_swap(fbits(x), fbits(y), false, false);
  x = bitsf(r[0]);
  y = bitsf(r[1]);
}

// The same exchange followed by the butterfly (a + b, a - b) of the pair that
// now sits in one lane: one Sylvester stage across lanes.
__device__ __forceinline__ void swap32_butterfly(float& x, float& y) {
  swap32(x, y);
  const float a = x, b = y;
  x = a + b;
  y = a - b;
}

__device__ __forceinline__ void swap16_butterfly(float& x, float& y) {
  swap16(x, y);
  const float a = x, b = y;
  x = a + b;
  y = a - b;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 q) { return __builtin_bit_cast(bf16x8_t, q); }

__device__ __forceinline__ void split_bf16(float v, uint16_t& hi, uint16_t& lo) {
  hi = f32_to_bf16_rne(v);
  lo = f32_to_bf16_rne(v - bits_f32((uint32_t)hi << 16));
}

// Raw x of one (16 rows, 128 columns) unit as this lane loads it: columns
// 64*(g >> 1) + 16*q + 8*(g & 1) + e (fragment g = 0..3, e = 0..7) of row l16,
// q being the lane quarter.
template <typename XT>
struct XFrag;

template <>
struct XFrag<uint16_t> {
  uint4 f[4];  // 8 bf16 per fragment
  __device__ __forceinline__ void load(const uint16_t* row, int col0, int q) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      f[g] = *reinterpret_cast<const uint4*>(row + col0 + 64 * (g >> 1) + 16 * q + 8 * (g & 1));
  }
  __device__ __forceinline__ void get(int g, float* v) const {
    const uint32_t w[4] = {f[g].x, f[g].y, f[g].z, f[g].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bits_f32(w[e] << 16);
      v[2 * e + 1] = bits_f32(w[e] & 0xFFFF0000u);
    }
  }
};

template <>
struct XFrag<float> {
  float4 f[8];  // 8 floats per fragment
  __device__ __forceinline__ void load(const float* row, int col0, int q) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4* p =
          reinterpret_cast<const float4*>(row + col0 + 64 * (g >> 1) + 16 * q + 8 * (g & 1));
      f[2 * g] = p[0];
      f[2 * g + 1] = p[1];
    }
  }
  __device__ __forceinline__ void get(int g, float* v) const {
    const float4 a = f[2 * g], b = f[2 * g + 1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// ---------------------------------------------------------------------------
// k_prep.  Lane l of a wave: row l16 = l % 16 of the workgroup's 16 rows, lane
// quarter q = l / 16.
//
// Phase 1 (KS > 0): per block, 4 k-steps of v_mfma_f32_16x16x32_bf16 per 16
// columns of u: A = raw x (row l16; fragment g supplies k-slots 8q..8q+7 --
// any fixed pairing of k-slots with columns works as long as B uses the same),
// B = rows of V''^T (u column l16, the same 8 columns).  Output: u row 4q + i,
// column l16.
//
// Phase 2, per block:
//  transform:  the lane's 32 values are columns 64*bb + 16*q + j (bb = 0..1,
//              j = 0..15).  Column bits 0..3 (j) and 6 (bb) are butterflied in
//              registers; bit 4 (lane bit q0) against register bit j2 with
//              v_permlane16_swap, bit 5 (lane bit q1) against j3 with
//              v_permlane32_swap.  Each swap-butterfly trades the lane bit with
//              the register bit, leaving tile t = (j >> 2) + 4*bb, columns
//              16t + 4q + (j & 3): the output layout of a 16x16 MFMA with the
//              block's columns as its rows and the 16 rows of x as its columns.
//  deflation:  acc_t += V[cols of tile t] (-u)^T, v_mfma_f32_16x16x32_bf16 with
//              bf16 hi/lo splits (hi*hi + hi*lo + lo*hi).
//  transpose:  two more swap stages (tile bit 2 with lane bit q1, tile bit 1
//              with q0) give each lane the whole of tiles 2q and 2q+1, i.e. two
//              complete NVFP4 blocks: column c of tile 2q+b sits in
//              acc[b + 2*(c >> 2)][c & 3].
//  quantise:   per block in one lane: amax, E4M3 scale, codes; one 16-byte
//              code store and one 2-byte scale store per lane.
//
// Blocks of a wave: KS > 0, NB > 0: wave + i*nw for i < NB, raw x held in
// registers between the phases; KS > 0, NB == 0: wave, wave + nw, ... with x
// loaded again in phase 2; KS == 0: (blockIdx.y*NB + i)*nw + wave.
template <typename XT, int KS, int NB>
__global__ void __launch_bounds__(512) k_prep(const XT* __restrict__ x, int M, int K, int r,
                                              const float* __restrict__ cvec,
                                              const uint16_t* __restrict__ vth,
                                              const uint16_t* __restrict__ vtl,
                                              const uint16_t* __restrict__ vh,
                                              const uint16_t* __restrict__ vl,
                                              uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ scales,
                                              float* __restrict__ u_out,
                                              float* __restrict__ pre) {
  constexpr int RP = KS * 32;  // padded rank: row stride of V, rows of V''^T
  constexpr int CT = KS * 2;   // 16-column tiles of u
  constexpr int NH = NB > 0 ? NB : 1;
  constexpr bool fp32_x = sizeof(XT) == 4;
  __shared__ float up[KS > 0 ? 8 : 1][16][RP + 1];  // each wave's partial u
  __shared__ float us[16][RP + 1];                  // u of the 16 rows
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int m0 = blockIdx.x * 16;
  const int m = m0 + l16;
  const int64_t mc = min(m, M - 1);
  const bool mok = m < M;
  const int nblk = K >> 7;
  const XT* xrow = x + mc * K;

  XFrag<XT> xr[NH];
  auto block_of = [&](int i) {
    return KS > 0 ? wave + i * nw : ((int)blockIdx.y * NH + i) * nw + wave;
  };

  // Operands of phase 2 for one block: the V rows of its 8 tiles (hi, lo) for
  // the deflation and its 128 values of 1/(s sqrt 128), all issued together
  struct P2 {
    uint4 vh[KS > 0 ? KS : 1][8], vl[KS > 0 ? KS : 1][8];
    float4 cv[2][4];
  };
  auto load_p2 = [&](P2& o, int b) {
    const int col0 = b * 128;
    if constexpr (KS > 0) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int64_t vrow = (int64_t)(col0 + 16 * t + l16) * RP + 32 * kk + 8 * q;
          o.vh[kk][t] = *reinterpret_cast<const uint4*>(vh + vrow);
          o.vl[kk][t] = *reinterpret_cast<const uint4*>(vl + vrow);
        }
    }
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        o.cv[bb][k] = reinterpret_cast<const float4*>(cvec + col0 + 64 * bb + 16 * q)[k];
  };

  // With one block per wave (and bf16 x, for registers) its phase-2 operands
  // are issued during phase 1, right after phase 1's own loads, so their
  // memory latency overlaps phase 1 instead of following it.
  constexpr bool kHoist = NB == 1 && !fp32_x;
  P2 p2first;
  if constexpr (kHoist && KS == 0) {
    if (block_of(0) < nblk) load_p2(p2first, block_of(0));
  }

  // -u for the 16 rows as the bf16 hi/lo B operand of the deflation MFMA:
  // lane supplies row l16, k-elements 8q .. 8q+7 of each 32-step
  bf16x8_t nuh[KS > 0 ? KS : 1], nul[KS > 0 ? KS : 1];

  if constexpr (KS > 0) {
    f32x4_t ah[CT], al[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) ah[c][i] = al[c][i] = 0.0f;

    // B fragments (rows of V''^T, hi and lo) of one block: all issued at once,
    // so a block costs one memory round trip rather than one per MFMA
    struct VFrag {
      uint4 h[4][CT], l[4][CT];
    };
    auto load_v = [&](VFrag& vf, int col0) {
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          const int64_t off = (int64_t)(c * 16 + l16) * K + col0 + 64 * (g >> 1) + 16 * q + 8 * (g & 1);
          vf.h[g][c] = *reinterpret_cast<const uint4*>(vth + off);
          vf.l[g][c] = *reinterpret_cast<const uint4*>(vtl + off);
        }
    };
    auto contract = [&](const XFrag<XT>& xf, const VFrag& vf) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x8_t a_hi, a_lo;
        if constexpr (!fp32_x) {
          a_hi = as_bf16x8(xf.f[g]);
        } else {
          float f[8];
          xf.get(g, f);
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
          const bf16x8_t b_hi = as_bf16x8(vf.h[g][c]);
          const bf16x8_t b_lo = as_bf16x8(vf.l[g][c]);
          ah[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, b_hi, ah[c], 0, 0, 0);
          al[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, b_lo, al[c], 0, 0, 0);
          if constexpr (fp32_x)
            al[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, b_hi, al[c], 0, 0, 0);
        }
      }
    };

    if constexpr (NB > 0) {
      // x of every block, then the V'' fragments double-buffered: block i+1's
      // loads are in flight while block i's MFMAs run
      VFrag vf[2];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int b = block_of(i);
        if (b < nblk) xr[i].load(xrow, b * 128, q);
      }
      if (block_of(0) < nblk) load_v(vf[0], block_of(0) * 128);
      if constexpr (kHoist) {  // after phase 1's own loads, so they are served first
        if (block_of(0) < nblk) load_p2(p2first, block_of(0));
      }
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int b = block_of(i);
        if (i + 1 < NB && block_of(i + 1) < nblk) load_v(vf[(i + 1) & 1], block_of(i + 1) * 128);
        if (b < nblk) contract(xr[i], vf[i & 1]);
      }
    } else {
      VFrag vf;
      for (int b = wave; b < nblk; b += nw) {
        xr[0].load(xrow, b * 128, q);
        load_v(vf, b * 128);
        contract(xr[0], vf);
      }
    }
    // partial u (rows 4q + i, column 16c + l16) to LDS, then the fixed-order sum
#pragma unroll
    for (int c = 0; c < CT; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) up[wave][4 * q + i][16 * c + l16] = ah[c][i] + al[c][i];
    __syncthreads();
    for (int i = tid; i < 16 * RP; i += blockDim.x) {
      const int rr = i / RP, c = i % RP;
      float s = 0.0f;
      for (int w = 0; w < nw; ++w) s += up[w][rr][c];
      us[rr][c] = s;
      if (c < r && m0 + rr < M) u_out[(int64_t)(m0 + rr) * r + c] = s;
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

  auto phase2 = [&](const XFrag<XT>& xf, const P2& p2, int b) {
    const int col0 = b * 128;
    // w[bb][j]: column col0 + 64*bb + 16*q + j times 1/(s sqrt 128); the
    // scaling is folded into the first butterfly stage (pairs j, j+1)
    float w[2][16];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      float cv[16], xv[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 t = p2.cv[bb][k];
        cv[4 * k] = t.x; cv[4 * k + 1] = t.y; cv[4 * k + 2] = t.z; cv[4 * k + 3] = t.w;
      }
      xf.get(2 * bb, xv);
      xf.get(2 * bb + 1, xv + 8);
#pragma unroll
      for (int j = 0; j < 16; j += 2) {
        const float t = xv[j + 1] * cv[j + 1];
        w[bb][j] = __builtin_fmaf(xv[j], cv[j], t);
        w[bb][j + 1] = __builtin_fmaf(xv[j], cv[j], -t);
      }
    }
    // Sylvester butterflies on column bits 1..3 (j) and 6 (bb)
#pragma unroll
    for (int hs = 2; hs < 16; hs <<= 1)
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
        if ((j & 8) == 0) swap32_butterfly(w[bb][j], w[bb][j + 8]);
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
          a_hi[t] = as_bf16x8(p2.vh[kk][t]);
          a_lo[t] = as_bf16x8(p2.vl[kk][t]);
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
    // lane quarters against tile bits: afterwards the lane holds tiles 2q and
    // 2q+1 whole
    float a[8][4];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) a[t][i] = acc[t][i];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) swap32(a[t][i], a[t + 4][i]);
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if ((j & 2) == 0)
#pragma unroll
        for (int i = 0; i < 4; ++i) swap16(a[j][i], a[j + 2][i]);
    uint32_t sc[2];
    uint2 cw[2];
#pragma unroll
    for (int bt = 0; bt < 2; ++bt) {
      float v[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) v[c] = a[bt + 2 * (c >> 2)][c & 3];
      cw[bt] = quantize_block(v, sc[bt]);
      if (pre && mok) {
        float4* pp = reinterpret_cast<float4*>(pre + mc * K + col0 + 32 * q + 16 * bt);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          pp[k] = make_float4(v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]);
      }
    }
    if (mok) {
      *reinterpret_cast<uint4*>(codes + mc * (K / 2) + col0 / 2 + 16 * q) =
          make_uint4(cw[0].x, cw[0].y, cw[1].x, cw[1].y);
      *reinterpret_cast<uint16_t*>(scales + mc * (K / 16) + col0 / 16 + 2 * q) =
          (uint16_t)(sc[0] | (sc[1] << 8));
    }
  };

  if constexpr (NB > 0) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int b = block_of(i);
      if (b < nblk) {
        if constexpr (KS == 0) xr[i].load(xrow, b * 128, q);
        if constexpr (kHoist) {
          phase2(xr[i], p2first, b);
        } else {
          P2 p2;
          load_p2(p2, b);
          phase2(xr[i], p2, b);
        }
      }
    }
  } else {
    for (int b = wave; b < nblk; b += nw) {
      xr[0].load(xrow, b * 128, q);
      P2 p2;
      load_p2(p2, b);
      phase2(xr[0], p2, b);
    }
  }
}

// Most blocks per wave whose raw x stays in registers between the phases
// without spilling (checked on the compiled kernels): more for bf16 x and
// rank <= 32, fewer for fp32 x (twice the bytes) and rank 64 (twice the V
// fragments).
template <typename XT, int KS>
constexpr int max_nb() {
  return KS >= 2 ? 1 : (sizeof(XT) == 4 ? 2 : 4);
}

// Launch shape.  r > 0: one workgroup per 16 rows, nw <= 8 waves sharing the
// row's blocks, nb per wave held in registers (nb = 0: x reloaded in phase 2,
// when more than max_nb per wave would be needed).  r == 0: workgroups of up
// to 4 waves, one block per wave, the grid spanning the blocks too.
struct PrepShape {
  int nw, nb;
  dim3 grid;
};

PrepShape prep_shape(int64_t M, int64_t K, int32_t r, int maxnb) {
  const int nblk = (int)(K / 128);
  const unsigned row_groups = (unsigned)((M + 15) / 16);
  PrepShape s;
  if (r == 0) {
    s.nw = nblk < 4 ? nblk : 4;
    s.nb = 1;
    s.grid = dim3(row_groups, (unsigned)((nblk + s.nw - 1) / s.nw));
    return s;
  }
  const int nb = (nblk + 7) / 8;
  s.nb = nb <= maxnb ? nb : 0;
  s.nw = s.nb > 0 ? (nblk + nb - 1) / nb : 8;
  s.grid = dim3(row_groups, 1);
  return s;
}

template <typename XT, int KS>
void launch_ks(hipStream_t st, const XT* x, int M, int K, int r, const float* cvec,
               const uint16_t* vth, const uint16_t* vtl, const uint16_t* vh, const uint16_t* vl,
               uint8_t* xc, uint8_t* xs, float* u, float* pre) {
  constexpr int MAXNB = max_nb<XT, KS>();
  const PrepShape s = prep_shape(M, K, r, MAXNB);
  const dim3 blk(64 * s.nw);
#define ASP_PREP(NB_)                                                                           \
  hipLaunchKernelGGL((k_prep<XT, KS, NB_>), s.grid, blk, 0, st, x, M, K, r, cvec, vth, vtl, vh, \
                     vl, xc, xs, u, pre)
  if constexpr (KS == 0) {
    ASP_PREP(1);
  } else {
    switch (s.nb) {
      case 0: ASP_PREP(0); break;
      case 1: ASP_PREP(1); break;
      case 2: if constexpr (MAXNB >= 2) ASP_PREP(2); break;
      case 3: if constexpr (MAXNB >= 3) ASP_PREP(3); break;
      default: if constexpr (MAXNB >= 4) ASP_PREP(4); break;
    }
  }
#undef ASP_PREP
}

template <typename XT>
int32_t launch_prep(const XT* x, int64_t M, int64_t K, int32_t r, const uint8_t* pack,
                    uint8_t* x_codes, uint8_t* x_scales, float* u, float* prequant,
                    hipStream_t stream) {
  const PrepPackLayout L = prep_pack_layout(K, r);
  const float* cvec = reinterpret_cast<const float*>(pack + L.cvec);
  const uint16_t* vth = reinterpret_cast<const uint16_t*>(pack + L.vt_hi);
  const uint16_t* vtl = reinterpret_cast<const uint16_t*>(pack + L.vt_lo);
  const uint16_t* vh = reinterpret_cast<const uint16_t*>(pack + L.v_hi);
  const uint16_t* vl = reinterpret_cast<const uint16_t*>(pack + L.v_lo);
  const int Mi = (int)M, Ki = (int)K;
  switch (L.rp32 / 32) {
    case 0:
      launch_ks<XT, 0>(stream, x, Mi, Ki, r, cvec, vth, vtl, vh, vl, x_codes, x_scales, u, prequant);
      break;
    case 1:
      launch_ks<XT, 1>(stream, x, Mi, Ki, r, cvec, vth, vtl, vh, vl, x_codes, x_scales, u, prequant);
      break;
    default:
      launch_ks<XT, 2>(stream, x, Mi, Ki, r, cvec, vth, vtl, vh, vl, x_codes, x_scales, u, prequant);
      break;
  }
  return launch_status("prep");
}

}  // namespace

int32_t act_prep_impl(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                      const uint8_t* prep_pack, uint8_t* x_codes, uint8_t* x_scales, float* u,
                      float* prequant, hipStream_t stream) {
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
  if (x_dtype == ASP_F32)
    return launch_prep(static_cast<const float*>(x), M, K, r, prep_pack, x_codes, x_scales, u,
                       prequant, stream);
  return launch_prep(static_cast<const uint16_t*>(x), M, K, r, prep_pack, x_codes, x_scales, u,
                     prequant, stream);
}

}  // namespace asp

using namespace asp;

extern "C" {

int32_t asp_act_prep(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                     const uint8_t* prep_pack, uint8_t* x_codes, uint8_t* x_scales, float* u,
                     float* prequant, void* stream) {
  clear_error();
  return act_prep_impl(x, x_dtype, M, K, r, prep_pack, x_codes, x_scales, u, prequant,
                       (hipStream_t)stream);
}

}  // extern "C"
