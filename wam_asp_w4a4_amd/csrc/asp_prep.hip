// Activation prep on gfx950: x/s, block Hadamard, u = x_tilde V, deflation
// x_tilde - u V^T, NVFP4 quantise + pack (model card "FastWAM UR3 3-task --
// 4-bit quantisations", section "What ASP is, and what the deflated form
// means").
//
// Every deflated element needs its row's full reduction u = x_tilde V, and
// both reductions of the layer -- u over K, the deflation over the rank -- read
// a K x r basis (V'' = diag(1/s) H V for u, V for the deflation, each as bf16
// high + low parts).  Each basis is far larger per row tile than the rows of x
// themselves, so it is staged once per workgroup in LDS and shared by 64 rows:
//
//  k_prep_u  u = x_tilde V = x V'' (V'' a per-layer constant), a thin GEMM on
//            the raw input: workgroup = 64 rows x one of S slices of K, the
//            slice's V'' staged in LDS by direct global-to-LDS copies issued
//            all at once, MFMA 16x16x32 bf16 with x exact in bf16 (an fp32 x
//            split exactly into three bf16 terms) and V'' as three bf16
//            terms (hi, mid, lo; about 26 significant bits).  Every cross
//            term of combined order <= 2 is formed (the dropped ones lie
//            below 2^-26 of the product), so u is a float32-accurate
//            product.  Writes S partial sums of u.
//  k_prep_q  workgroup = 64 rows x one 128-column Hadamard block.  Each wave
//            loads its 16 rows of x, the block's 1/(s sqrt 128), its share of
//            the block's V rows and the S partial sums of u for its rows, all
//            at once into registers; it transforms x while the rest arrives,
//            puts V in LDS for the workgroup, adds the partial sums in a fixed
//            order (so results are deterministic), then deflates on MFMA
//            (V and -u each as three bf16 terms, the six cross terms of
//            order <= 2 summed from zero and added to x_tilde once, a
//            float32-accurate x_tilde - u V^T), quantises and stores.  For
//            r == 0 it runs alone, without u and V.
//
// S depends on K only, so a row's results do not depend on the batch it is in.
#include "asp_device.h"

#include <algorithm>

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

// The same exchanges on float64 values (each half separately), followed by
// the butterfly (a + b, a - b) of the pair that now sits in one lane: one
// Sylvester stage across lanes.
__device__ __forceinline__ void swap32_butterfly(double& x, double& y) {
  const u32x2_t xs = __builtin_bit_cast(u32x2_t, x), ys = __builtin_bit_cast(u32x2_t, y);
  const auto lo = __builtin_amdgcn_permlane32_swap(xs[0], ys[0], false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(xs[1], ys[1], false, false);
  const double a = __builtin_bit_cast(double, u32x2_t{lo[0], hi[0]});
  const double b = __builtin_bit_cast(double, u32x2_t{lo[1], hi[1]});
  x = a + b;
  y = a - b;
}

__device__ __forceinline__ void swap16_butterfly(double& x, double& y) {
  const u32x2_t xs = __builtin_bit_cast(u32x2_t, x), ys = __builtin_bit_cast(u32x2_t, y);
  const auto lo = __builtin_amdgcn_permlane16_swap(xs[0], ys[0], false, false);
  const auto hi = __builtin_amdgcn_permlane16_swap(xs[1], ys[1], false, false);
  const double a = __builtin_bit_cast(double, u32x2_t{lo[0], hi[0]});
  const double b = __builtin_bit_cast(double, u32x2_t{lo[1], hi[1]});
  x = a + b;
  y = a - b;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 q) { return __builtin_bit_cast(bf16x8_t, q); }
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t q) { return __builtin_bit_cast(bf16x8_t, q); }

// A float32 value as three bf16 terms: each the RNE bf16 rounding of what the
// earlier terms leave.  Both differences are exact in float32, and the third
// term is exact too, so v == t[0] + t[1] + t[2] for every normal float32 v.
__device__ __forceinline__ void split_bf16x3(float v, uint16_t (&t)[kSplit]) {
  t[0] = bf16_rne(v);
  const float r1 = v - bits_f32((uint32_t)t[0] << 16);
  t[1] = bf16_rne(r1);
  t[2] = bf16_rne(r1 - bits_f32((uint32_t)t[1] << 16));
}

// Raw x of one (16 rows, 128 columns) unit as this lane loads it: columns
// 64*(g >> 1) + 16*q + 8*(g & 1) + e (fragment g = 0..3, e = 0..7) of row l16,
// q being the lane quarter.
template <typename XT>
struct XFrag;

template <>
struct XFrag<uint16_t> {
  u32x4_t f[4];  // 8 bf16 per fragment
  __device__ __forceinline__ void load(const uint16_t* row, int col0, int q) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
      f[g] = *reinterpret_cast<const u32x4_t*>(row + col0 + 64 * (g >> 1) + 16 * q + 8 * (g & 1));
  }
  // from a wave's staged tile (XStage layout): row l16, fragment pieces
  __device__ __forceinline__ void load_lds(const u32x4_t* t, int q, int l16);
  __device__ __forceinline__ void get(int g, float* v) const {
    const uint32_t w[4] = {f[g][0], f[g][1], f[g][2], f[g][3]};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bits_f32(w[e] << 16);
      v[2 * e + 1] = bits_f32(w[e] & 0xFFFF0000u);
    }
  }
};

template <>
struct XFrag<float> {
  f32x4_t f[8];  // 8 floats per fragment
  __device__ __forceinline__ void load(const float* row, int col0, int q) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4_t* p =
          reinterpret_cast<const f32x4_t*>(row + col0 + 64 * (g >> 1) + 16 * q + 8 * (g & 1));
      f[2 * g] = p[0];
      f[2 * g + 1] = p[1];
    }
  }
  __device__ __forceinline__ void load_lds(const u32x4_t* t, int q, int l16);
  __device__ __forceinline__ void get(int g, float* v) const {
    const f32x4_t a = f[2 * g], b = f[2 * g + 1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = a[e];
      v[4 + e] = b[e];
    }
  }
};

// A wave's 16 rows x 128 columns of x staged in LDS by direct 16-byte copies
// (lds_copy16): copy j moves RPC whole rows (4 rows of 256 bytes for bf16, 2
// of 512 for fp32), so one instruction reads few, fully used cache lines.
// Slot l of copy j holds piece (l % PPR) ^ (R & 15) of tile row R = RPC*j +
// l / PPR; a fragment read (16 lanes: one piece of 16 different rows) then
// falls in 16 distinct bank groups.
template <typename XT>
struct XStage {
  static constexpr int PPR = 128 * (int)sizeof(XT) / 16;  // 16-byte pieces per row
  static constexpr int RPC = 64 / PPR;                     // rows per copy
  static constexpr int COPIES = 16 / RPC;
  static constexpr int PIECES = 16 * PPR;                  // per wave
  __device__ static __forceinline__ int slot(int row, int piece) {
    return (row / RPC) * 64 + (row % RPC) * PPR + (piece ^ (row & 15));
  }
  // rows m0 .. m0+15 (clamped to M - 1), columns col0 .. col0+127
  __device__ static __forceinline__ void issue(const XT* x, int64_t m0, int M, int64_t K, int col0,
                                               u32x4_t* t, int lane) {
    const int R0 = lane / PPR, p = lane % PPR;
#pragma unroll
    for (int j = 0; j < COPIES; ++j) {
      const int R = RPC * j + R0;
      const int64_t row = min(m0 + R, (int64_t)M - 1);
      lds_copy16(x + row * K + col0 + (p ^ (R & 15)) * (16 / (int)sizeof(XT)), t + 64 * j);
    }
  }
};

__device__ __forceinline__ void XFrag<uint16_t>::load_lds(const u32x4_t* t, int q, int l16) {
#pragma unroll
  for (int g = 0; g < 4; ++g) f[g] = t[XStage<uint16_t>::slot(l16, 8 * (g >> 1) + 2 * q + (g & 1))];
}

__device__ __forceinline__ void XFrag<float>::load_lds(const u32x4_t* t, int q, int l16) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int p = 16 * (g >> 1) + 4 * q + 2 * (g & 1);
    f[2 * g] = __builtin_bit_cast(f32x4_t, t[XStage<float>::slot(l16, p)]);
    f[2 * g + 1] = __builtin_bit_cast(f32x4_t, t[XStage<float>::slot(l16, p + 1)]);
  }
}

// ---------------------------------------------------------------------------
// k_prep_u.  Workgroup = 4 waves x 16 rows, one slice of K (blocks b0..b1).
// Lane l of wave w: row m0 + 16w + l%16, lane quarter q = l/16.  Per block,
// 4 k-steps of v_mfma_f32_16x16x32_bf16 per 16 columns of u: A = raw x
// (fragment g supplies k-slots 8q..8q+7 -- any fixed pairing of k-slots with
// columns works as long as B uses the same), B = rows of V''^T from LDS (u
// column l%16, the same 8 columns).  Output lane layout: u row 4q + i, column
// l%16.
//
// LDS per round: up to CHUNKS chunks (128-column blocks) of V''^T (three terms;
// RP rows of 128 bf16 = 16 pieces of 16 bytes) and of every wave's x rows
// (XStage), all staged at once with lds_copy16.  Piece p of V''^T row `row`
// sits in slot p ^ (row & 15), so the 16 lanes of a quarter, which read the
// same piece of 16 different rows, hit 16 different bank groups.
constexpr int kPrepRows = 64;  // rows of x per k_prep_q workgroup (4 waves x 16)
// Slices of K for the partial sums of u: up to 8 when u has at most 32
// columns, up to 4 when it has 64 (the quantise stage holds every slice's
// partial sums in registers at once).  Every 128-column workgroup of the
// quantise stage reads all of its rows' partial sums, so more slices cost
// there what they save in the u stage; 8 pay off only for long rows.
constexpr int max_slices(int ks) { return ks <= 1 ? 8 : 4; }

template <typename XT, int KS>
struct UStage {
  static constexpr int RP = 32 * KS;
  static constexpr int CHUNK_PIECES = kSplit * RP * 16;       // 3 terms, 16 pieces per row
  static constexpr int X_PIECES = 4 * XStage<XT>::PIECES;     // the 4 waves' x
  static constexpr int CHUNKS = 8192 / (CHUNK_PIECES + X_PIECES);  // up to 128 KB per round
  static_assert(CHUNKS >= 1, "one chunk must fit");
};

template <typename XT, int KS>
__device__ __forceinline__ void prep_u_body(const XT* __restrict__ x, int M, int K, int r,
                                            const uint16_t* __restrict__ vt, int64_t tstride,
                                            float* __restrict__ u_part, int bps) {
  using St = UStage<XT, KS>;
  constexpr int RP = St::RP, CT = KS * 2, NC = St::CHUNKS;
  constexpr bool fp32_x = sizeof(XT) == 4;
  extern __shared__ u32x4_t sv[];  // min(NC, bps) chunks of V''^T, then of x; sized at launch
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int m0 = blockIdx.x * kPrepRows + 16 * wave;
  const int64_t mc = min(m0 + l16, M - 1);
  const int nblk = K >> 7;
  const int b0 = blockIdx.y * bps, b1 = min(nblk, b0 + bps);

  f32x4_t ah[CT], al[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) ah[c][i] = al[c][i] = 0.0f;

  const int ncmax = min(NC, bps);
  for (int rb = b0; rb < b1; rb += ncmax) {
    const int nc = min(ncmax, b1 - rb);
    // stage chunks rb .. rb+nc-1: slot P = (chunk*3 + term)*RP*16 + row*16 + slot
    const int pieces = nc * St::CHUNK_PIECES;
    for (int base = 64 * wave; base < pieces; base += 256) {
      const int P = base + lane;
      const int c = P / St::CHUNK_PIECES, rem = P % St::CHUNK_PIECES;
      const int term = rem / (RP * 16), row = (rem / 16) % RP, slot = rem % 16;
      const uint16_t* src = vt + term * tstride + (int64_t)row * K + (rb + c) * 128 +
                            8 * (slot ^ (row & 15));
      lds_copy16(src, &sv[base]);
    }
    u32x4_t* sx = sv + ncmax * St::CHUNK_PIECES;  // chunk c, wave w: sx + (4c + w) * PIECES
    for (int c = 0; c < nc; ++c)
      XStage<XT>::issue(x, m0, M, K, (rb + c) * 128, sx + (4 * c + wave) * XStage<XT>::PIECES, lane);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
    __syncthreads();                // and everyone else's
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      if (c >= nc) break;
      const u32x4_t* ch = sv + c * St::CHUNK_PIECES;
      XFrag<XT> xc;
      xc.load_lds(sx + (4 * c + wave) * XStage<XT>::PIECES, q, l16);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int piece = 8 * (g >> 1) + 2 * q + (g & 1);
        // x as bf16 terms: one (exact) for bf16 x, three for float32 x
        bf16x8_t xa[fp32_x ? kSplit : 1];
        if constexpr (!fp32_x) {
          xa[0] = as_bf16x8(xc.f[g]);
        } else {
          float f[8];
          xc.get(g, f);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint16_t t[kSplit];
            split_bf16x3(f[e], t);
#pragma unroll
            for (int i = 0; i < kSplit; ++i) xa[i][e] = bf16_from_bits(t[i]);
          }
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int row = 16 * ct + l16;
          const int slot = row * 16 + (piece ^ (row & 15));
          bf16x8_t b[kSplit];
#pragma unroll
          for (int i = 0; i < kSplit; ++i) b[i] = as_bf16x8(ch[i * RP * 16 + slot]);
          // hi * hi alone; the smaller cross terms (order 1 and 2) together
          ah[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[0], b[0], ah[ct], 0, 0, 0);
          al[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[0], b[1], al[ct], 0, 0, 0);
          al[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[0], b[2], al[ct], 0, 0, 0);
          if constexpr (fp32_x) {
            al[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[1], b[0], al[ct], 0, 0, 0);
            al[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[1], b[1], al[ct], 0, 0, 0);
            al[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[2], b[0], al[ct], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();  // LDS is refilled by the next round
  }
  // partial u: rows 4q + i of the wave's 16, column 16c + l16
#pragma unroll
  for (int c = 0; c < CT; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + 4 * q + i;
      if (row < M) u_part[((int64_t)blockIdx.y * M + row) * RP + 16 * c + l16] = ah[c][i] + al[c][i];
    }
}

// ---------------------------------------------------------------------------
// k_prep_q.  Workgroup = 4 waves x 16 rows and one 128-column block.  Lane l
// of wave w: row m0 + 16w + l%16, lane quarter q = l/16.
//  staging:    the block's V rows (three bf16 terms; 128 rows of RP bf16 =
//              PPR pieces of 16 bytes each) through registers, piece p of row `row` in slot
//              p ^ ((row / (16/PPR)) % PPR) -- the 16 lanes of a quarter read
//              one piece of 16 consecutive rows and hit 16 different bank
//              groups; 1/(s sqrt 128) (float64) of the block by ordinary loads.
//  u:          the S partial sums for the wave's rows added in slice order.
//  transform:  in float64; the lane's 32 values are columns 64*bb + 16*q + j (bb = 0..1,
//              j = 0..15).  Column bits 0..3 (j) and 6 (bb) are butterflied in
//              registers; bit 4 (lane bit q0) against register bit j2 with
//              v_permlane16_swap, bit 5 (lane bit q1) against j3 with
//              v_permlane32_swap.  Each swap-butterfly trades the lane bit with
//              the register bit, leaving tile t = (j >> 2) + 4*bb, columns
//              16t + 4q + (j & 3): the output layout of a 16x16 MFMA with the
//              block's columns as its rows and the 16 rows of x as its columns.
//  deflation:  d_t = V[cols of tile t] (-u)^T on v_mfma_f32_16x16x32_bf16,
//              V and -u as three bf16 terms each (the six cross terms of
//              order <= 2, from zero, smallest first); x_d = float32(x_tilde
//              (float64) + d_t), one rounding.
//  transpose:  two more swap stages (tile bit 2 with lane bit q1, tile bit 1
//              with q0) give each lane the whole of tiles 2q and 2q+1, i.e. two
//              complete NVFP4 blocks: column c of tile 2q+b sits in
//              acc[b + 2*(c >> 2)][c & 3].
//  quantise:   per block in one lane: amax, E4M3 scale, codes; one 16-byte
//              code store and one 2-byte scale store per lane.
// One wave's loads for one 16-row x 128-column unit: its rows of x and the
// partial sums of u for those rows.  SMAX, the launch's power of two >= S,
// fixes the count (straight-line code, so the compiler waits for each load
// by count); slices past S re-read the last one and are not added.
template <typename XT, int KS, int SMAX>
struct QUnit {
  static constexpr int MS = KS > 0 ? SMAX : 1, KK = KS > 0 ? KS : 1;
  static_assert(KS == 0 || (SMAX >= 1 && SMAX <= max_slices(KS)), "slice bound");
  XFrag<XT> x;
  f32x4_t pa[MS][KK][2];

  // the partial sums of u for row mc (already clamped to M - 1) of this lane
  __device__ __forceinline__ void issue_u(int M, const float* __restrict__ u_part, int S,
                                          int64_t mc, int q) {
    if constexpr (KS > 0) {
      constexpr int RP = KS * 32;
#pragma unroll
      for (int s = 0; s < MS; ++s)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const f32x4_t* p = reinterpret_cast<const f32x4_t*>(
              u_part + ((int64_t)min(s, S - 1) * M + mc) * RP + 32 * kk + 8 * q);
          pa[s][kk][0] = p[0];
          pa[s][kk][1] = p[1];
        }
    }
  }
};

// 1/(s sqrt 128) (float64) of the lane's 32 columns 64*bb + 16*q + j of the block
__device__ __forceinline__ void load_col_scales(const double* __restrict__ cvec, int col0, int q,
                                                f64x2_t (&cq)[2][8]) {
#pragma unroll
  for (int bb = 0; bb < 2; ++bb)
#pragma unroll
    for (int k = 0; k < 8; ++k)
      cq[bb][k] = reinterpret_cast<const f64x2_t*>(cvec + col0 + 64 * bb + 16 * q)[k];
}

// The block's V rows (three bf16 terms) through registers, 16 bytes per
// thread and copy; written to LDS by store.  (A pending direct global-to-LDS
// copy would make the compiler wait for every load before the first use of
// any.)
template <int KS>
struct VRows {
  static constexpr int RP = KS * 32;
  static constexpr int PPR = KS > 0 ? RP / 8 : 1;          // 16-byte pieces per V row
  static constexpr int TERM = 128 * PPR;                    // pieces per term plane
  static constexpr int PIECES = KS > 0 ? kSplit * TERM : 1;
  static constexpr int RDIV = 16 / PPR;                     // rows sharing a swizzle key
  static constexpr int COPIES = KS > 0 ? PIECES / 256 : 1;
  static_assert(KS == 0 || PIECES % 256 == 0, "whole copies per thread");
  u32x4_t reg[COPIES];
  // piece p of row `row` of term plane t sits in slot t * TERM + row * PPR +
  // (p ^ ((row / RDIV) % PPR)): the 16 lanes of a quarter read one piece of
  // 16 consecutive rows and hit 16 different bank groups
  __device__ __forceinline__ void issue(const uint16_t* __restrict__ v, int64_t tstride, int bq,
                                        int tid) {
    if constexpr (KS > 0) {
#pragma unroll
      for (int j = 0; j < COPIES; ++j) {
        const int P = tid + 256 * j;
        const int t = P / TERM, row = (P / PPR) % 128, slot = P % PPR;
        const int piece = slot ^ ((row / RDIV) % PPR);
        reg[j] = *reinterpret_cast<const u32x4_t*>(v + t * tstride + (int64_t)(bq * 128 + row) * RP +
                                                   8 * piece);
      }
    }
  }
  __device__ __forceinline__ void store(u32x4_t* sv, int tid) const {
    if constexpr (KS > 0) {
#pragma unroll
      for (int j = 0; j < COPIES; ++j) sv[tid + 256 * j] = reg[j];
    }
  }
};

// Smoothing and the Sylvester transform of one unit, in float64 (x and
// 1/(s sqrt 128) exact, every stage rounded to 53 bits, so the result is
// x_tilde to far below a float32 ulp; it is rounded to float32 once, when the
// deflation is added): w[bb][j] is afterwards column 16*t + 4*q + (j & 3) of
// the block, tile t = (j >> 2) + 4*bb.
template <typename XT>
__device__ __forceinline__ void q_transform(const XFrag<XT>& xr, const f64x2_t (&cq)[2][8],
                                            double (&w)[2][16]) {
  // column 64*bb + 16*q + j of the block times 1/(s sqrt 128); the scaling
  // is folded into the first butterfly stage (pairs j, j+1)
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    float xv[16];
    xr.get(2 * bb, xv);
    xr.get(2 * bb + 1, xv + 8);
#pragma unroll
    for (int j = 0; j < 16; j += 2) {
      const double c0 = cq[bb][j >> 1][0], c1 = cq[bb][j >> 1][1];
      const double t = (double)xv[j + 1] * c1;
      w[bb][j] = __builtin_fma((double)xv[j], c0, t);
      w[bb][j + 1] = __builtin_fma((double)xv[j], c0, -t);
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
          const double a = w[bb][j], c = w[bb][j + hs];
          w[bb][j] = a + c;
          w[bb][j + hs] = a - c;
        }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const double a = w[0][j], c = w[1][j];
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
}

// The rest of one unit, after the transform and with the block's V in LDS:
// u from its partial sums (slice order), the deflation on MFMA, the
// transpose to whole NVFP4 blocks per lane, quantisation and the stores.
// Row m of this lane (mc = min(m, M - 1)), block bq at column col0.
template <typename XT, int KS, int SMAX>
__device__ __forceinline__ void q_finish(const double (&w)[2][16], const QUnit<XT, KS, SMAX>& U, int S,
                                         const u32x4_t* sv, int M, int K, int r, int bq, int m,
                                         int64_t mc, int q, int l16,
                                         uint8_t* __restrict__ codes,
                                         uint8_t* __restrict__ scales,
                                         float* __restrict__ u_out, float* __restrict__ pre) {
  using VR = VRows<KS>;
  constexpr int MS = QUnit<XT, KS, SMAX>::MS;
  const bool mok = m < M;
  const int col0 = bq * 128;
  // -u for the 16 rows as the B operand of the deflation MFMA, three bf16
  // terms: lane supplies row l16, k-elements 8q .. 8q+7 of each 32-step
  bf16x8_t nu[kSplit][KS > 0 ? KS : 1];
  if constexpr (KS > 0) {
    float us[KS][8];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) us[kk][e] = 0.0f;
#pragma unroll
    for (int s = 0; s < MS; ++s)
      if (s < S)
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            us[kk][e] += U.pa[s][kk][0][e];
            us[kk][4 + e] += U.pa[s][kk][1][e];
          }
    if (bq == 0 && mok) {
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (32 * kk + 8 * q + e < r) u_out[(int64_t)m * r + 32 * kk + 8 * q + e] = us[kk][e];
    }
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint16_t t[kSplit];
        split_bf16x3(-us[kk][e], t);
#pragma unroll
        for (int i = 0; i < kSplit; ++i) nu[i][kk][e] = bf16_from_bits(t[i]);
      }
  }
  f32x4_t acc[8];
  if constexpr (KS == 0) {
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] = (float)w[t >> 2][4 * (t & 3) + e];
  } else {
    // -u V^T from zero: the six cross terms (V term i, u term j) with i + j
    // <= 2, smallest first; x_tilde + that, rounded to float32 once
    f32x4_t d[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) d[t][e] = 0.0f;
#pragma unroll
    for (int i = kSplit - 1; i >= 0; --i)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        bf16x8_t a[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int row = 16 * t + l16, piece = 4 * kk + q;
          a[t] = as_bf16x8(sv[i * VR::TERM + row * VR::PPR + (piece ^ ((row / VR::RDIV) % VR::PPR))]);
        }
#pragma unroll
        for (int j = kSplit - 1 - i; j >= 0; --j)
#pragma unroll
          for (int t = 0; t < 8; ++t)
            d[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[t], nu[j][kk], d[t], 0, 0, 0);
      }
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] = (float)(w[t >> 2][4 * (t & 3) + e] + (double)d[t][e]);
  }
  // lane quarters against tile bits: afterwards the lane holds tiles 2q and
  // 2q+1 whole
  float a[8][4];
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) a[t][e] = acc[t][e];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) swap32(a[t][e], a[t + 4][e]);
#pragma unroll
  for (int j = 0; j < 8; ++j)
    if ((j & 2) == 0)
#pragma unroll
      for (int e = 0; e < 4; ++e) swap16(a[j][e], a[j + 2][e]);
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
}

// k_prep_q, one unit per wave (workgroup = 64 rows x block blockIdx.y).
// Every load is issued first: x, the column scales, V, the partial sums;
// the transform runs while V and u are in flight, and the workgroup meets at
// one barrier once V is in LDS.
template <typename XT, int KS, int SMAX>
__device__ __forceinline__ void prep_q_body(const XT* __restrict__ x, int M, int K, int r,
                                            const double* __restrict__ cvec,
                                            const uint16_t* __restrict__ vv, int64_t tstride,
                                            const float* __restrict__ u_part, int S,
                                            uint8_t* __restrict__ codes,
                                            uint8_t* __restrict__ scales,
                                            float* __restrict__ u_out,
                                            float* __restrict__ pre) {
  __shared__ u32x4_t sv[VRows<KS>::PIECES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int q = lane >> 4, l16 = lane & 15;
  const int m = blockIdx.x * kPrepRows + 16 * wave + l16;
  const int64_t mc = min(m, M - 1);
  const int bq = blockIdx.y;

  QUnit<XT, KS, SMAX> U;
  f64x2_t cq[2][8];
  VRows<KS> V;
  U.x.load(x + mc * K, bq * 128, q);
  load_col_scales(cvec, bq * 128, q, cq);
  V.issue(vv, tstride, bq, tid);
  U.issue_u(M, u_part, S, mc, q);
  __builtin_amdgcn_sched_barrier(0);  // every load is issued before the transform
  double w[2][16];
  q_transform(U.x, cq, w);
  V.store(sv, tid);
  __syncthreads();  // V is in LDS for every wave
  q_finish(w, U, S, sv, M, K, r, bq, m, mc, q, l16, codes, scales, u_out, pre);
}

// Per-layer pointers of a (grouped) launch; layer = blockIdx.z.
template <typename XT>
struct PrepLayerArgs {
  const XT* x;
  const double* cvec;
  const uint16_t* vt;  // V'' terms (u stage), term t at vt + t * tstride
  const uint16_t* v;   // V terms (deflation), term t at v + t * tstride
  int64_t tstride;     // elements between consecutive term planes
  float* u_part;
  uint8_t* xc;
  uint8_t* xs;
  float* u;
  float* pre;
};

template <typename XT>
struct PrepArgs {
  PrepLayerArgs<XT> l[kMaxGroup];
};

template <typename XT, int KS>
__global__ void __launch_bounds__(256) k_prep_u(const PrepArgs<XT> a, int M, int K, int r,
                                                int bps) {
  const PrepLayerArgs<XT>& L = a.l[blockIdx.z];
  prep_u_body<XT, KS>(L.x, M, K, r, L.vt, L.tstride, L.u_part, bps);
}

template <typename XT, int KS, int SMAX>
__global__ void __launch_bounds__(256) k_prep_q(const PrepArgs<XT> a, int M, int K, int r,
                                                int S) {
  const PrepLayerArgs<XT>& L = a.l[blockIdx.z];
  prep_q_body<XT, KS, SMAX>(L.x, M, K, r, L.cvec, L.v, L.tstride, L.u_part, S, L.xc, L.xs, L.u,
                            L.pre);
}


constexpr int kStageU = 1, kStageQ = 2;  // the two launches of the prep

// Slices of K for the partial sums of u (a function of K and the padded rank
// only, so a row's u does not depend on the batch): up to max_slices, each a
// whole number of blocks.
void u_slicing(int64_t K, int ks, int* S, int* bps) {
  const int nblk = (int)(K / 128);
  const int s = std::min(nblk, nblk >= 32 ? max_slices(ks) : 4);
  *bps = (nblk + s - 1) / s;
  *S = (nblk + *bps - 1) / *bps;
}

template <typename XT, int KS, int SMAX>
void launch_q(hipStream_t st, int n, const PrepArgs<XT>& a, int M, int K, int r, int S) {
  const int nblk = K / 128;
  const int tiles64 = (M + kPrepRows - 1) / kPrepRows;
  hipLaunchKernelGGL((k_prep_q<XT, KS, SMAX>), dim3((unsigned)tiles64, (unsigned)nblk, (unsigned)n),
                     dim3(256), 0, st, a, M, K, r, S);
}

template <typename XT, int KS>
void launch_ks(hipStream_t st, int stages, int n, const PrepArgs<XT>& a, int M, int K, int r) {
  const int nblk = K / 128;
  const int tiles64 = (M + kPrepRows - 1) / kPrepRows;
  int S = 0, bps = 0;
  if constexpr (KS > 0) {
    u_slicing(K, KS, &S, &bps);
    if (stages & kStageU) {
      // the chunks of a slice (up to a round's worth) in dynamic LDS; above the
      // default 64 KB this must be allowed per kernel (a host attribute of the
      // current device, not a stream operation)
      using St = UStage<XT, KS>;
      const size_t lds = (size_t)std::min(St::CHUNKS, bps) * (St::CHUNK_PIECES + St::X_PIECES) * 16;
      (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&k_prep_u<XT, KS>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      hipLaunchKernelGGL((k_prep_u<XT, KS>), dim3((unsigned)tiles64, (unsigned)S, (unsigned)n),
                         dim3(256), lds, st, a, M, K, r, bps);
    }
  }
  if (stages & kStageQ) {
    if constexpr (KS == 0) {
      launch_q<XT, 0, 1>(st, n, a, M, K, r, S);
    } else if (S <= 1) {
      launch_q<XT, KS, 1>(st, n, a, M, K, r, S);
    } else if (S <= 2) {
      launch_q<XT, KS, 2>(st, n, a, M, K, r, S);
    } else if (KS > 1 || S <= 4) {
      launch_q<XT, KS, 4>(st, n, a, M, K, r, S);
    } else {
      launch_q<XT, KS, (KS > 1 ? 4 : 8)>(st, n, a, M, K, r, S);
    }
  }
}

template <typename XT>
int32_t launch_prep(int stages, int n, const PrepCall* calls, int64_t M, int64_t K, int32_t r,
                    hipStream_t stream) {
  const PrepPackLayout P = prep_pack_layout(K, r);
  PrepArgs<XT> a = {};
  for (int i = 0; i < n; ++i) {
    const uint8_t* pack = calls[i].prep_pack;
    PrepLayerArgs<XT>& L = a.l[i];
    L.x = static_cast<const XT*>(calls[i].x);
    L.cvec = reinterpret_cast<const double*>(pack + P.cvec64);
    L.vt = reinterpret_cast<const uint16_t*>(pack + P.vt[0]);
    L.v = reinterpret_cast<const uint16_t*>(pack + P.v[0]);
    L.tstride = (int64_t)(P.plane_bytes / 2);
    L.u_part = static_cast<float*>(calls[i].scratch);
    L.xc = calls[i].x_codes;
    L.xs = calls[i].x_scales;
    L.u = calls[i].u;
    L.pre = calls[i].prequant;
  }
  const int Mi = (int)M, Ki = (int)K;
  switch (P.rp32 / 32) {
    case 0: launch_ks<XT, 0>(stream, stages, n, a, Mi, Ki, r); break;
    case 1: launch_ks<XT, 1>(stream, stages, n, a, Mi, Ki, r); break;
    default: launch_ks<XT, 2>(stream, stages, n, a, Mi, Ki, r); break;
  }
  return launch_status("prep");
}

}  // namespace

size_t act_prep_scratch_bytes(int64_t M, int64_t K, int32_t r) {
  if (r == 0 || M == 0) return 0;
  int S, bps;
  const int rp32 = prep_pack_layout(K, r).rp32;
  u_slicing(K, rp32 / 32, &S, &bps);
  return (size_t)S * (size_t)M * (size_t)rp32 * sizeof(float);
}

int32_t act_prep_impl(int stages, int n, const PrepCall* calls, int32_t x_dtype, int64_t M,
                      int64_t K, int32_t r, hipStream_t stream) {
  ASP_TRY(check_mk(M, K));
  ASP_TRY(check_rank(r));
  if (x_dtype != ASP_F32 && x_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "x_dtype=%d", x_dtype);
  if (n < 1 || n > kMaxGroup) return fail(ASP_ERR_ARG, "group of %d layers outside [1, %d]", n, kMaxGroup);
  if (M == 0) return ASP_OK;
  const size_t need = act_prep_scratch_bytes(M, K, r);
  for (int i = 0; i < n; ++i) {
    const PrepCall& c = calls[i];
    ASP_TRY(check_ptr(c.x, "x", true));
    ASP_TRY(check_ptr(c.prep_pack, "prep_pack", true));
    if (stages & kStageQ) {
      ASP_TRY(check_ptr(c.x_codes, "x_codes", true));
      ASP_TRY(check_ptr(c.x_scales, "x_scales", true));
      ASP_TRY(check_ptr(c.u, "u", r > 0));
      ASP_TRY(check_ptr(c.prequant, "prequant", false));
    }
    if (need) {
      ASP_TRY(check_ptr(c.scratch, "workspace", true));
      if (c.scratch_bytes < need)
        return fail(ASP_ERR_WORKSPACE, "workspace %zu bytes, need %zu", c.scratch_bytes, need);
    }
  }
  if (x_dtype == ASP_F32) return launch_prep<float>(stages, n, calls, M, K, r, stream);
  return launch_prep<uint16_t>(stages, n, calls, M, K, r, stream);
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
  const PrepCall c = {x, prep_pack, x_codes, x_scales, u, prequant, workspace, workspace_bytes};
  return act_prep_impl(kStageU | kStageQ, 1, &c, x_dtype, M, K, r, (hipStream_t)stream);
}

int32_t asp_act_prep_u(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                       const uint8_t* prep_pack, void* workspace, size_t workspace_bytes,
                       void* stream) {
  clear_error();
  const PrepCall c = {x, prep_pack, nullptr, nullptr, nullptr, nullptr, workspace, workspace_bytes};
  return act_prep_impl(kStageU, 1, &c, x_dtype, M, K, r, (hipStream_t)stream);
}

int32_t asp_act_prep_q(const void* x, int32_t x_dtype, int64_t M, int64_t K, int32_t r,
                       const uint8_t* prep_pack, uint8_t* x_codes, uint8_t* x_scales, float* u,
                       float* prequant, void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  const PrepCall c = {x, prep_pack, x_codes, x_scales, u, prequant, workspace, workspace_bytes};
  return act_prep_impl(kStageQ, 1, &c, x_dtype, M, K, r, (hipStream_t)stream);
}

}  // extern "C"
