// 4-bit GEMM with fused low-rank + bias epilogue on gfx950 (CDNA4):
//
//   y = DQ(x_codes, x_scales) DQ(w_codes, w_scales)^T + bf16(u) wv^T + bias
//
// the NVFP4GEMM term and the bf16 low-rank branch of the deflated contract
// (model card "FastWAM UR3 3-task -- 4-bit quantisations", section "What ASP
// is, and what the deflated form means"; the branch "stays in bf16 by
// design").
//
// gfx950's block-scaled FP4 MFMA takes one power-of-two (E8M0) scale per 32
// K-elements; NVFP4 has one E4M3 scale (4 significant bits) per 16.  Both
// operands are therefore decoded to exact fp16 (E2M1 value x E4M3 scale has at
// most 6 significant bits and lies in [2^-10, 2688]) and contracted on
// v_mfma_f32_32x32x16_f16: one MFMA K-step is exactly one NVFP4 block, and only
// fp32 accumulation order differs from exact arithmetic.  The low-rank branch
// adds ceil(r/16) bf16 MFMA K-steps into the same accumulators; bias and the
// output cast follow.
//
// Decoding 8 elements costs 8 VALU instructions (four 2-code conversions, four
// packed fp16 scale multiplies), so the kernels differ mainly in how often a
// fragment is decoded:
//  k_gemm_wb   (large layers, K % 256 == 0) decodes the weight tile once per
//              workgroup into LDS as fp16 and each activation fragment once,
//              in the registers of the one wave that uses it;
//  k_gemm      (other large and mid-size layers) stages codes and scales in
//              double-buffered LDS (256 K-elements a stage) and decodes both
//              operands in every wave's registers;
//  k_gemm_sk   (small M) splits K over the waves of a workgroup, each wave
//              staging its own K range of both operands.
// Two waves share each SIMD so that one wave's decode overlaps the other's
// MFMAs.
#include "asp_device.h"

#include <algorithm>

namespace asp {
namespace {

constexpr int BK = 256;                 // K elements per stage (16 NVFP4 blocks / K-steps)
constexpr int KSTEPS = BK / 16;
constexpr int CROW = BK / 2;            // code bytes per row per stage
constexpr int ROWB = CROW + 8;          // padded LDS code row (136 B = 34 dwords)
constexpr int SROWB = KSTEPS * 2 + 4;   // padded LDS scale row: 16 fp16 + 4 (36 B = 9 dwords)

template <int WM, int WN, int TM, int TN>
struct Cfg {
  static constexpr int NW = WM * WN;
  static constexpr int NT = NW * 64;
  static constexpr int BM = WM * TM * 32;
  static constexpr int BN = WN * TN * 32;
  static constexpr int ROWS = BM + BN;                    // tile rows staged per stage
  static constexpr int SEGS = CROW / 16;                  // 16-byte code loads per row
  static constexpr int CODE_LOADS = ROWS * SEGS;
  static constexpr int CL_PER_T = (CODE_LOADS + NT - 1) / NT;
  static constexpr int SC_PER_T = (ROWS + NT - 1) / NT;   // one row's 16 scale bytes each
  static constexpr int CODES = ROWS * ROWB;
  static constexpr int STAGE = CODES + ROWS * SROWB;
  static constexpr int LDS = 2 * STAGE;
};

// Map a linear workgroup id to a tile.  Consecutive workgroups go to
// different XCDs (round-robin dispatch), so ids are first regrouped so that
// each XCD's share is a contiguous run, then the run is rastered in groups of
// GROUP_M tile rows so that neighbouring workgroups on one XCD share A rows
// and B columns in its L2.
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
  constexpr int GROUP_M = 4;
  const int total = tiles_m * tiles_n;
  if ((total & 7) == 0) {
    const int per = total >> 3;
    bid = (bid & 7) * per + (bid >> 3);
  }
  const int group = bid / (GROUP_M * tiles_n);
  const int first = group * GROUP_M;
  const int gsize = min(GROUP_M, tiles_m - first);
  const int in = bid - group * GROUP_M * tiles_n;
  tm = first + in % gsize;
  tn = in / gsize;
}

// E4M3 scale bytes 0,1 (hi = false) or 2,3 (hi = true) of w as two fp16
// values: v_cvt_scalef32_pk_f16_fp8 with scale 1 decodes OCP E4M3FN, and every
// finite E4M3 value (subnormals included) is an fp16 normal, so it is exact.
template <bool HI>
__device__ __forceinline__ uint32_t scale_pair_f16(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI));
}

// Low-rank branch straight from memory: bf16(u) (M x r) times wv^T (r x N)
// in K-steps of 16 into the wave's accumulators, for its tile rows rb + 32 i +
// l32 and columns cb + 32 j + l32.  Addresses are clamped (always valid) and
// columns past r are zeroed after the load, so no lane-dependent branch sits
// around a load; when r % 8 == 0 a lane's 8 columns are one 16-byte-aligned
// piece (u and wv are) lying wholly inside or wholly past the row.
template <int TM, int TN>
__device__ __forceinline__ void lowrank_from_memory(f32x16_t (&acc)[TM][TN],
                                                    const float* __restrict__ u,
                                                    const uint16_t* __restrict__ wv, int M, int N,
                                                    int r, int rb, int cb0, int half, int l32) {
  for (int c0 = 0; c0 < r; c0 += 16) {
    bf16x8_t la[TM], lb[TN];
    const int cb = c0 + half * 8;                      // this lane's 8 columns
    const bool in = cb < r;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float f[8];
      const int64_t m = min(rb + i * 32 + l32, M - 1);
      if ((r & 7) == 0) {
        const float* pu = u + m * r + (in ? cb : 0);
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(pu);
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(pu + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[e] = in ? a[e] : 0.0f;
          f[4 + e] = in ? b[e] : 0.0f;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = u[m * r + min(cb + e, r - 1)];
          f[e] = cb + e < r ? v : 0.0f;
        }
      }
      la[i] = bf16x8_rne(f);
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = min(cb0 + j * 32 + l32, N - 1);
      if ((r & 7) == 0) {
        u32x4_t q = *reinterpret_cast<const u32x4_t*>(wv + n * r + (in ? cb : 0));
        if (!in) q = u32x4_t{0, 0, 0, 0};
        lb[j] = __builtin_bit_cast(bf16x8_t, q);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t v = wv[n * r + min(cb + e, r - 1)];
          lb[j][e] = bf16_from_bits(cb + e < r ? v : (uint16_t)0);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[i], lb[j], acc[i][j], 0, 0, 0);
  }
}

// Bytes of LDS a bf16 output tile takes in store_tile: rows padded by 8
// elements (16 bytes), so the two lane halves of a store, 4 rows apart, fall
// in different banks.
constexpr int out_tile_bytes(int BM, int BN) { return BM * (BN + 8) * 2; }

// Bias and store of a workgroup's BM x BN tile (origin m0, n0); the wave holds
// rows wr0 + 32 i and columns wc0 + 32 j of it.  Accumulator element v of lane
// l is row 8*(v/4) + 4*(l/32) + v%4 and column l%32 of its 32 x 32 tile.  A
// bf16 output goes through LDS (smem, free once every wave is past its K loop:
// the barrier below; out_tile_bytes of it) so that each thread writes 16
// consecutive bytes of a row.
template <int TM, int TN, int BM, int BN, int NT>
__device__ __forceinline__ void store_tile(const f32x16_t (&acc)[TM][TN],
                                           const float* __restrict__ bias, void* __restrict__ y,
                                           int y_bf16, int M, int N, int m0, int n0, int wr0,
                                           int wc0, int half, int l32, int tid, uint8_t* smem) {
  float bj[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + wc0 + j * 32 + l32;
    bj[j] = (bias && col < N) ? bias[col] : 0.0f;
  }
  if (y_bf16) {
    __syncthreads();
    uint16_t* ot = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = wr0 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          const int col = wc0 + j * 32 + l32;
          ot[row * (BN + 8) + col] = bf16_rne(acc[i][j][v] + bj[j]);
        }
    __syncthreads();
    uint16_t* yo = reinterpret_cast<uint16_t*>(y);
    constexpr int CHUNKS = BM * BN / 8;
    for (int c = tid; c < CHUNKS; c += NT) {
      const int row = c / (BN / 8), col = (c % (BN / 8)) * 8;
      const int gm = m0 + row, gn = n0 + col;
      if (gm >= M) continue;
      const int64_t off = (int64_t)gm * N + gn;
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(ot + row * (BN + 8) + col);
      if (gn + 8 <= N && (off & 7) == 0) {
        *reinterpret_cast<u32x4_t*>(yo + off) = val;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (gn + e < N) yo[off + e] = (uint16_t)(val[e >> 1] >> (16 * (e & 1)));
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wc0 + j * 32 + l32;
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + wr0 + i * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          if (row < M) reinterpret_cast<float*>(y)[(int64_t)row * N + col] = acc[i][j][v] + bj[j];
        }
    }
  }
}

template <int WM, int WN, int TM, int TN>
__device__ __forceinline__ void gemm_body(const uint8_t* __restrict__ xc,
                                          const uint8_t* __restrict__ xs,
                                          const float* __restrict__ u, int M, int N, int K, int r,
                                          const uint8_t* __restrict__ wc,
                                          const uint8_t* __restrict__ ws,
                                          const uint16_t* __restrict__ wv,
                                          const float* __restrict__ bias, void* __restrict__ y,
                                          int y_bf16, int tiles_m, int tiles_n) {
  using C = Cfg<WM, WN, TM, TN>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[C::LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int half = lane >> 5, l32 = lane & 31;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * C::BM, n0 = tn * C::BN;
  const int64_t KB = K / 2, KS = K / 16;

  // staging assignments: code load i -> tile row i / SEGS, 16-byte segment i % SEGS
  const uint8_t* csrc[C::CL_PER_T];
  int cdst[C::CL_PER_T];
  bool cok[C::CL_PER_T];
#pragma unroll
  for (int j = 0; j < C::CL_PER_T; ++j) {
    const int i = tid + j * C::NT;
    cok[j] = i < C::CODE_LOADS;
    const int ii = cok[j] ? i : 0;
    const int row = ii / C::SEGS, seg = ii % C::SEGS;
    cdst[j] = row * ROWB + seg * 16;
    const int64_t g = row < C::BM ? min(m0 + row, M - 1) : min(n0 + row - C::BM, N - 1);
    csrc[j] = (row < C::BM ? xc : wc) + g * KB + seg * 16;
  }
  const uint8_t* ssrc[C::SC_PER_T];
  int sdst[C::SC_PER_T];
  bool sok[C::SC_PER_T];
#pragma unroll
  for (int j = 0; j < C::SC_PER_T; ++j) {
    const int row = tid + j * C::NT;
    sok[j] = row < C::ROWS;
    const int rr = sok[j] ? row : 0;
    sdst[j] = C::CODES + rr * SROWB;
    const int64_t g = rr < C::BM ? min(m0 + rr, M - 1) : min(n0 + rr - C::BM, N - 1);
    ssrc[j] = (rr < C::BM ? xs : ws) + g * KS;
  }

  uint4 rc[C::CL_PER_T];
  uint4 rs[C::SC_PER_T];
  // A last stage over only 128 K-elements (K % 256 == 128) loads the valid
  // half and zero-fills the rest: zero codes with zero scales add nothing.
  auto gload = [&](int kc) {
#pragma unroll
    for (int j = 0; j < C::CL_PER_T; ++j) {
      const int seg = (cdst[j] % ROWB) / 16;
      const bool in_k = (int64_t)kc * CROW + seg * 16 < KB;
      rc[j] = (cok[j] && in_k) ? *reinterpret_cast<const uint4*>(csrc[j] + (int64_t)kc * CROW)
                               : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < C::SC_PER_T; ++j) {
      if (!sok[j]) continue;
      const uint8_t* p = ssrc[j] + (int64_t)kc * KSTEPS;
      if ((int64_t)kc * KSTEPS + KSTEPS <= KS) {
        rs[j] = *reinterpret_cast<const uint4*>(p);
      } else {
        const uint2 h = *reinterpret_cast<const uint2*>(p);
        rs[j] = make_uint4(h.x, h.y, 0, 0);
      }
    }
  };
  auto sstore = [&](int buf) {
    uint8_t* base = smem + buf * C::STAGE;
#pragma unroll
    for (int j = 0; j < C::CL_PER_T; ++j)
      if (cok[j]) {
        *reinterpret_cast<uint2*>(base + cdst[j]) = make_uint2(rc[j].x, rc[j].y);
        *reinterpret_cast<uint2*>(base + cdst[j] + 8) = make_uint2(rc[j].z, rc[j].w);
      }
#pragma unroll
    for (int j = 0; j < C::SC_PER_T; ++j)
      if (sok[j]) {
        // 16 E4M3 scales -> 16 exact fp16, converted once per stage
        uint32_t* d = reinterpret_cast<uint32_t*>(base + sdst[j]);
        const uint32_t q[4] = {rs[j].x, rs[j].y, rs[j].z, rs[j].w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          d[2 * p] = scale_pair_f16<false>(q[p]);
          d[2 * p + 1] = scale_pair_f16<true>(q[p]);
        }
      }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // per-lane LDS offsets of this wave's fragment rows (code word of K-step ks
  // at + 4 * (2 ks + half); fp16 scale of K-steps 2p, 2p+1 at + 4 p)
  int aoff[TM], boff[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) aoff[i] = ((wm * TM + i) * 32 + l32);
#pragma unroll
  for (int j = 0; j < TN; ++j) boff[j] = (C::BM + (wn * TN + j) * 32 + l32);

  // Low-rank operands through LDS when r <= 32 and r % 8 == 0: during the
  // last stage the other staging buffer is free, and direct 16-byte copies
  // (no registers) fill it with the tile's rows of u (BM x 32 fp32, 128 B a
  // row) and W~V (BN x 32 bf16, 64 B a row).  Piece p of a u row sits in slot
  // p ^ (row & 7), of a W~V row in slot p ^ (row & 3), so the fragment reads
  // below spread over the banks; pieces past r copy piece 0 (never read).
  static_assert(C::BM * 128 + C::BN * 64 <= C::STAGE, "low-rank rows must fit a staging buffer");
  // (Measured: this pays off for the 64 x 64 tiles; in the 256 x 192 tiles it
  // costs more in the K loop's registers than it hides.)
  constexpr bool kLrStage = TM * TN == 1;
  const bool lr_lds = kLrStage && r > 0 && r <= 32 && (r & 7) == 0;
  auto lr_issue = [&](uint8_t* buf) {
    // an opaque zero keeps the address arithmetic inside the last stage
    // instead of live across the whole K loop
    int zo = 0;
    asm volatile("" : "+s"(zo));
    const int w = (tid >> 6) + zo;
#pragma unroll
    for (int j = 0; j < (C::BM * 8 + C::NT - 1) / C::NT; ++j) {
      const int P0 = (j * C::NW + w) * 64;
      if (P0 >= C::BM * 8) break;
      const int P = P0 + lane, row = P >> 3, slot = P & 7, pc = slot ^ (row & 7);
      const int64_t m = min(m0 + row, M - 1);
      lds_copy16(u + m * r + (4 * pc < r ? 4 * pc : 0), buf + 16 * P0);
    }
#pragma unroll
    for (int j = 0; j < (C::BN * 4 + C::NT - 1) / C::NT; ++j) {
      const int P0 = (j * C::NW + w) * 64;
      if (P0 >= C::BN * 4) break;
      const int P = P0 + lane, row = P >> 2, slot = P & 3, pc = slot ^ (row & 3);
      const int64_t n = min(n0 + row, N - 1);
      lds_copy16(wv + n * r + (8 * pc < r ? 8 * pc : 0), buf + C::BM * 128 + 16 * P0);
    }
  };

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  if (nk > 1) gload(1);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const uint8_t* base = smem + (kc & 1) * C::STAGE;
    if constexpr (kLrStage)
      if (lr_lds && kc == nk - 1) lr_issue(smem + ((kc + 1) & 1) * C::STAGE);
    uint32_t aw[TM], bw[TN], asw[TM], bsw[TN];
    auto read_words = [&](int ks, uint32_t (&a)[TM], uint32_t (&b)[TN]) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        a[i] = *reinterpret_cast<const uint32_t*>(base + aoff[i] * ROWB + 4 * (2 * ks + half));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        b[j] = *reinterpret_cast<const uint32_t*>(base + boff[j] * ROWB + 4 * (2 * ks + half));
    };
    auto read_scales = [&](int p) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
        asw[i] = *reinterpret_cast<const uint32_t*>(base + C::CODES + aoff[i] * SROWB + 4 * p);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bsw[j] = *reinterpret_cast<const uint32_t*>(base + C::CODES + boff[j] * SROWB + 4 * p);
    };
    read_words(0, aw, bw);
    read_scales(0);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      uint32_t an[TM], bn[TN];
      if (ks + 1 < KSTEPS) read_words(ks + 1, an, bn);  // one K-step ahead
      half8_t af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const half2_t s2 = __builtin_bit_cast(half2_t, asw[i]);
        af[i] = decode8(aw[i], (ks & 1) ? s2[1] : s2[0]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const half2_t s2 = __builtin_bit_cast(half2_t, bsw[j]);
        bf[j] = decode8(bw[j], (ks & 1) ? s2[1] : s2[0]);
      }
      if ((ks & 1) && ks + 1 < KSTEPS) read_scales((ks + 1) >> 1);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
      if (ks + 1 < KSTEPS) {
#pragma unroll
        for (int i = 0; i < TM; ++i) aw[i] = an[i];
#pragma unroll
        for (int j = 0; j < TN; ++j) bw[j] = bn[j];
      }
    }
    // The other buffer held stage kc-1, which every wave finished reading
    // before the barrier that ended the previous iteration, so it can be
    // refilled now; one barrier per stage publishes it.
    if (kc + 1 < nk) {
      sstore((kc + 1) & 1);
      if (kc + 2 < nk) gload(kc + 2);
      __syncthreads();
    }
  }

  // low-rank branch: bf16(u) (M x r) times wv^T (r x N), K-steps of 16.  The
  // operand rows come from the staging buffer filled during the last stage
  // (lr_lds), else straight from memory.
  const int wr0 = wm * TM * 32, wc0 = wn * TN * 32;
  if (lr_lds) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies have landed
    __syncthreads();                                   // and every other wave's
    const uint8_t* lrb = smem + (nk & 1) * C::STAGE;
    for (int c0 = 0; c0 < r; c0 += 16) {
      bf16x8_t la[TM], lb[TN];
      const int cb = c0 + half * 8;                    // this lane's 8 columns
      const bool in = cb < r;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wr0 + i * 32 + l32, p0 = cb >> 2;
        const f32x4_t a = *reinterpret_cast<const f32x4_t*>(lrb + row * 128 + 16 * ((p0 ^ (row & 7)) & 7));
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(lrb + row * 128 + 16 * (((p0 + 1) ^ (row & 7)) & 7));
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[e] = in ? a[e] : 0.0f;
          f[4 + e] = in ? b[e] : 0.0f;
        }
        la[i] = bf16x8_rne(f);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int row = wc0 + j * 32 + l32;
        u32x4_t q = *reinterpret_cast<const u32x4_t*>(lrb + C::BM * 128 + row * 64 + 16 * (((cb >> 3) ^ (row & 3)) & 3));
        if (!in) q = u32x4_t{0, 0, 0, 0};
        lb[j] = __builtin_bit_cast(bf16x8_t, q);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[i], lb[j], acc[i][j], 0, 0, 0);
    }
  } else {
    lowrank_from_memory<TM, TN>(acc, u, wv, M, N, r, m0 + wr0, n0 + wc0, half, l32);
  }
  static_assert(out_tile_bytes(C::BM, C::BN) <= C::LDS, "a bf16 output tile must fit the staging LDS");
  store_tile<TM, TN, C::BM, C::BN, C::NT>(acc, bias, y, y_bf16, M, N, m0, n0, wr0, wc0, half, l32,
                                          tid, smem);
}

// Per-layer pointers of a (grouped) launch; layer = blockIdx.y.  A layer
// with fewer tiles than the grid's x extent leaves the rest idle.
struct GemmLayerArgs {
  const uint8_t* xc;
  const uint8_t* xs;
  const float* u;
  const uint8_t* wc;
  const uint8_t* ws;
  const uint16_t* wv;
  const float* bias;
  void* y;
  int N;
  int tiles_n;
};

struct GemmArgs {
  GemmLayerArgs l[kMaxGroup];
};

template <int WM, int WN, int TM, int TN>
__global__ void __launch_bounds__(WM * WN * 64)
    k_gemm(const GemmArgs a, int M, int K, int r, int y_bf16, int tiles_m) {
  const GemmLayerArgs& L = a.l[blockIdx.y];
  if ((int)blockIdx.x >= tiles_m * L.tiles_n) return;
  gemm_body<WM, WN, TM, TN>(L.xc, L.xs, L.u, M, L.N, K, r, L.wc, L.ws, L.wv, L.bias, L.y, y_bf16,
                            tiles_m, L.tiles_n);
}

// The grid's x extent: the largest layer's tile count; every layer's count
// must fit an int.
inline int32_t group_args(int n, const GemmCall* calls, int64_t M, int BM, int BN, GemmArgs& a,
                          int64_t& tiles_m, int64_t& max_tiles) {
  tiles_m = (M + BM - 1) / BM;
  max_tiles = 0;
  a = GemmArgs{};
  for (int i = 0; i < n; ++i) {
    const int64_t tn = (calls[i].N + BN - 1) / BN;
    if (tiles_m * tn > INT32_MAX)
      return fail(ASP_ERR_SHAPE, "M=%lld N=%lld too large for one launch", (long long)M,
                  (long long)calls[i].N);
    max_tiles = std::max(max_tiles, tiles_m * tn);
    a.l[i] = {calls[i].x_codes, calls[i].x_scales, calls[i].u, calls[i].w_codes,
              calls[i].w_scales, calls[i].wv, calls[i].bias, calls[i].y, (int)calls[i].N, (int)tn};
  }
  return ASP_OK;
}

template <int WM, int WN, int TM, int TN>
int32_t launch_gemm(int n, const GemmCall* calls, int64_t M, int64_t K, int32_t r, int32_t y_dtype,
                    hipStream_t stream) {
  using C = Cfg<WM, WN, TM, TN>;
  GemmArgs a;
  int64_t tiles_m, max_tiles;
  ASP_TRY(group_args(n, calls, M, C::BM, C::BN, a, tiles_m, max_tiles));
  hipLaunchKernelGGL((k_gemm<WM, WN, TM, TN>), dim3((unsigned)max_tiles, (unsigned)n), dim3(C::NT),
                     0, stream, a, (int)M, (int)K, (int)r, (int)(y_dtype == ASP_BF16),
                     (int)tiles_m);
  return launch_status("gemm");
}

// ---------------------------------------------------------------------------
// k_gemm_wb: the path for large layers with K % 256 == 0.  Eight waves stacked
// in M (512 x 96 workgroup tile, 64 x 96 per wave).  The weight tile is
// decoded once per workgroup into LDS as exact fp16 (in K order, rows padded
// to 528 bytes so the 16-byte fragment reads of 16 consecutive rows hit
// distinct banks) and shared by all eight waves; each wave streams its own
// activation rows from memory straight into registers and decodes them there,
// so no activation fragment is decoded twice and none passes through LDS.
// Stages of 256 K-elements, double-buffered, one barrier each.
//
// K-slot mapping: per group of 64 K-elements (32 code bytes a row), lane half
// h holds bytes 16h .. 16h+15 (elements 32h .. 32h+31: blocks 2h and 2h+1 of
// the group) and K-step t of the group uses its word t (elements 32h + 8t ..
// +7); the weight fragment of that K-step is the 16 bytes of fp16 at element
// 64g + 32h + 8t of its row.  Products thus pair equal K indices, and a lane's
// 8 values of a K-step share one block scale.
namespace wb {
constexpr int NW = 8, NT = NW * 64, TM = 2, TN = 3;
constexpr int BM = NW * TM * 32, BN = TN * 32;         // 512 x 96
constexpr int BK = 256, KST = BK / 16, GPS = BK / 64;  // 16 K-steps, 4 groups of 64 a stage
constexpr int BROWB = BK * 2 + 16;                     // padded fp16 weight row (528 B)
constexpr int STAGE = BN * BROWB;
constexpr int LDS = 2 * STAGE > out_tile_bytes(BM, BN) ? 2 * STAGE : out_tile_bytes(BM, BN);
constexpr int B_PAIRS = BN * (BK / 16) / NT;           // (row, block) pairs a thread decodes
static_assert(BN * (BK / 16) % NT == 0, "weight staging split");
}  // namespace wb

__device__ __forceinline__ void gemm_wb_body(const uint8_t* __restrict__ xc,
                                             const uint8_t* __restrict__ xs,
                                             const float* __restrict__ u, int M, int N, int K,
                                             int r, const uint8_t* __restrict__ wc,
                                             const uint8_t* __restrict__ ws,
                                             const uint16_t* __restrict__ wv,
                                             const float* __restrict__ bias,
                                             void* __restrict__ y, int y_bf16, int tiles_m,
                                             int tiles_n) {
  using wb::NT, wb::TM, wb::TN, wb::BM, wb::BN, wb::BK, wb::KST, wb::GPS, wb::BROWB, wb::STAGE,
      wb::LDS, wb::B_PAIRS;
  __shared__ __attribute__((aligned(16))) uint8_t smem[LDS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t KB = K / 2, KS = K / 16;

  // this wave's activation rows (clamped to M - 1; their results are not stored)
  const uint8_t* arow[TM];
  const uint8_t* asrow[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = min(m0 + wave * TM * 32 + i * 32 + l32, M - 1);
    arow[i] = xc + m * KB + 16 * half;
    asrow[i] = xs + m * KS;
  }
  // weight staging: pair p = tid + j * NT is block p % 16 of tile row p / 16,
  // so 16 consecutive threads read one row's 128 code bytes of the stage
  const uint8_t* bsrc[B_PAIRS];
  const uint8_t* bssrc[B_PAIRS];
  int bdst[B_PAIRS];
#pragma unroll
  for (int j = 0; j < B_PAIRS; ++j) {
    const int p = tid + j * NT, row = p >> 4, blk = p & 15;
    const int64_t n = min(n0 + row, N - 1);
    bsrc[j] = wc + n * KB + blk * 8;
    bssrc[j] = ws + n * KS + blk;
    bdst[j] = row * BROWB + blk * 32;
  }
  uint2 rb[B_PAIRS];
  uint32_t rbs[B_PAIRS];
  auto bload = [&](int kc) {
#pragma unroll
    for (int j = 0; j < B_PAIRS; ++j) {
      rb[j] = *reinterpret_cast<const uint2*>(bsrc[j] + (int64_t)kc * (BK / 2));
      rbs[j] = bssrc[j][(int64_t)kc * KST];
    }
  };
  auto bstore = [&](int buf) {
    uint8_t* base = smem + buf * STAGE;
#pragma unroll
    for (int j = 0; j < B_PAIRS; ++j) {
      const _Float16 sc = __builtin_bit_cast(half2_t, scale_pair_f16<false>(rbs[j]))[0];
      *reinterpret_cast<half8_t*>(base + bdst[j]) = decode8(rb[j].x, sc);
      *reinterpret_cast<half8_t*>(base + bdst[j] + 16) = decode8(rb[j].y, sc);
    }
  };
  // a stage's activation codes (per group and fragment) and scales (per fragment)
  u32x4_t ac[GPS][TM];
  u32x4_t as[TM];
  auto aload_group = [&](int kc, int g) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      ac[g][i] = *reinterpret_cast<const u32x4_t*>(arow[i] + (int64_t)kc * (BK / 2) + 32 * g);
  };
  auto aload_scales = [&](int kc) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
      as[i] = *reinterpret_cast<const u32x4_t*>(asrow[i] + (int64_t)kc * KST);
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  int boff[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) boff[j] = (j * 32 + l32) * BROWB + 64 * half;

  const int nk = K / BK;
  bload(0);
#pragma unroll
  for (int g = 0; g < GPS; ++g) aload_group(0, g);
  aload_scales(0);
  bstore(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const uint8_t* base = smem + (kc & 1) * STAGE;
    const bool more = kc + 1 < nk;
    if (more) bload(kc + 1);
    u32x4_t asc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i) asc[i] = as[i];
    if (more) aload_scales(kc + 1);
    half8_t bf[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) bf[j] = *reinterpret_cast<const half8_t*>(base + boff[j]);
#pragma unroll
    for (int g = 0; g < GPS; ++g) {
      // this lane's two block scales of the group, as fp16
      half2_t sp[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        sp[i] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(asc[i][g] >> (16 * half), 1.0f, false);
      const u32x4_t (&cur)[TM] = ac[g];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int ks = 4 * g + t;
        half8_t bn[TN];
        if (ks + 1 < KST)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            bn[j] = *reinterpret_cast<const half8_t*>(base + boff[j] + 128 * ((ks + 1) >> 2) +
                                                      16 * ((ks + 1) & 3));
        half8_t af[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) af[i] = decode8(cur[i][t], sp[i][t >> 1]);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
        if (ks + 1 < KST)
#pragma unroll
          for (int j = 0; j < TN; ++j) bf[j] = bn[j];
      }
      // the group's registers, refilled for the next stage once its four
      // K-steps are issued (no copy of the codes is kept meanwhile)
      if (more) aload_group(kc + 1, g);
      // the other buffer held stage kc - 1, which every wave finished reading
      // before the barrier that ended the previous stage
      if (g == 2 && more) bstore((kc + 1) & 1);
    }
    if (more) __syncthreads();
  }

  const int wr0 = wave * TM * 32;
  lowrank_from_memory<TM, TN>(acc, u, wv, M, N, r, m0 + wr0, n0, half, l32);
  store_tile<TM, TN, BM, BN, NT>(acc, bias, y, y_bf16, M, N, m0, n0, wr0, 0, half, l32, tid, smem);
}

__global__ void __launch_bounds__(wb::NT)
    k_gemm_wb(const GemmArgs a, int M, int K, int r, int y_bf16, int tiles_m) {
  const GemmLayerArgs& L = a.l[blockIdx.y];
  if ((int)blockIdx.x >= tiles_m * L.tiles_n) return;
  gemm_wb_body(L.xc, L.xs, L.u, M, L.N, K, r, L.wc, L.ws, L.wv, L.bias, L.y, y_bf16, tiles_m,
               L.tiles_n);
}

int32_t launch_gemm_wb(int n, const GemmCall* calls, int64_t M, int64_t K, int32_t r,
                       int32_t y_dtype, hipStream_t stream) {
  GemmArgs a;
  int64_t tiles_m, max_tiles;
  ASP_TRY(group_args(n, calls, M, wb::BM, wb::BN, a, tiles_m, max_tiles));
  hipLaunchKernelGGL(k_gemm_wb, dim3((unsigned)max_tiles, (unsigned)n), dim3(wb::NT), 0, stream, a,
                     (int)M, (int)K, (int)r, (int)(y_dtype == ASP_BF16), (int)tiles_m);
  return launch_status("gemm_wb");
}

// ---------------------------------------------------------------------------
// k_gemm_sk: the path for few output tiles (small M).  A workgroup owns a
// (32*FM) x (32*FN) tile of y; its W waves split K into W equal ranges, and
// each wave computes the whole tile over its range, streaming its operand rows
// straight from memory into registers (16-byte loads, two chunks in flight, no
// LDS staging and no barrier in the K loop).  The W partial tiles then meet in
// LDS and are added in a fixed order (deterministic), and each thread stores
// a run of consecutive columns with one vector store.
//
// K-slot mapping.  Per group of 64 K elements (32 code bytes), lane half h
// loads the 16 bytes holding elements 32h .. 32h+31 of the group (two NVFP4
// blocks); K-step t = 0..3 of the group feeds its k-slots 8h .. 8h+7 with
// elements 32h + 8t .. 32h + 8t + 7, which lie in block 2h + (t >> 1).  A and B
// use the same mapping, so every product pairs equal K indices, and a lane's 8
// values of a K-step share one block scale.
template <int FM, int FN, int W>
__device__ __forceinline__ void gemm_sk_body(const uint8_t* __restrict__ xc,
                                             const uint8_t* __restrict__ xs,
                                             const float* __restrict__ u, int M, int N, int K,
                                             int r, const uint8_t* __restrict__ wc,
                                             const uint8_t* __restrict__ ws,
                                             const uint16_t* __restrict__ wv,
                                             const float* __restrict__ bias,
                                             void* __restrict__ y, int y_bf16, int tiles_n) {
  constexpr int BM = 32 * FM, BN = 32 * FN, NF = FM + FN;
  constexpr int CH = 4;                      // groups of 64 K per chunk
  constexpr int EPT = BM * BN / (W * 64);    // output elements per thread
  // Each wave stages a chunk of its operand rows (32 rows x 128 bytes per
  // fragment) in a private LDS slot; after the K loop the same memory holds
  // the partial tiles.
  constexpr int STAGE = NF * 4 * 64;         // 16-byte pieces per wave
  static_assert(W * BM * (BN + 4) * 4 <= W * STAGE * 16, "partials must fit the staging LDS");
  __shared__ u32x4_t stage[W][STAGE];
  auto part = reinterpret_cast<float(*)[BM][BN + 4]>(&stage[0][0]);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t KB = K / 2, KS = K / 16;
  const int ng = K / 64 / W;                 // groups of this wave
  const int gbeg = wave * ng, gend = gbeg + ng;

  const uint8_t* srow[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int64_t row = f < FM ? min(m0 + 32 * f + l32, M - 1) : min(n0 + 32 * (f - FM) + l32, N - 1);
    srow[f] = (f < FM ? xs : ws) + row * KS;
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // The low-rank operands and the bias are loaded before the main loop so
  // their latency hides behind it.  Low-rank K-step c (16 of the r columns)
  // belongs to wave c % W; lane half h supplies columns 16c + 8h .. 16c + 8h + 7.
  // Loads read clamped, always valid addresses; columns past r (and bias
  // entries past N) are zeroed only where the values are used, so nothing
  // waits for these loads before the main loop.  When r % 8 == 0 the 8
  // columns are 16-byte aligned (u and wv are) and lie wholly inside or
  // wholly past the row.
  constexpr int LRW = (4 + W - 1) / W;       // r <= 64: at most 4 steps, spread over W waves
  f32x4_t lu[LRW][FM][2];
  u32x4_t lw[LRW][FN];
  const bool vec = (r & 7) == 0;
#pragma unroll
  for (int k = 0; k < LRW; ++k) {
    const int cb = 16 * (wave + k * W) + 8 * half;
    if (cb - 8 * half >= r) continue;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const float* pu = u + min(m0 + 32 * i + l32, M - 1) * (int64_t)r;
      if (vec) {
        const float* p = pu + (cb < r ? cb : 0);
        lu[k][i][0] = *reinterpret_cast<const f32x4_t*>(p);
        lu[k][i][1] = *reinterpret_cast<const f32x4_t*>(p + 4);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) lu[k][i][e >> 2][e & 3] = pu[min(cb + e, r - 1)];
      }
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const uint16_t* pw = wv + min(n0 + 32 * j + l32, N - 1) * (int64_t)r;
      if (vec) {
        lw[k][j] = *reinterpret_cast<const u32x4_t*>(pw + (cb < r ? cb : 0));
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          lw[k][j][e] = pw[min(cb + 2 * e, r - 1)] | ((uint32_t)pw[min(cb + 2 * e + 1, r - 1)] << 16);
      }
    }
  }
  const int e0 = tid * EPT, orow = e0 / BN, ocol = e0 % BN;
  const int gm = m0 + orow, gn = n0 + ocol;
  float bv[EPT];
  if (bias) {
    if (gn + EPT <= N && ((gn | N) & 3) == 0 && EPT % 4 == 0) {
#pragma unroll
      for (int e = 0; e < EPT; e += 4) {
        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(bias + gn + e);
#pragma unroll
        for (int t = 0; t < 4; ++t) bv[e + t] = b[t];
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) bv[e] = bias[min(gn + e, N - 1)];
    }
  }

  // Codes: global -> LDS by direct 16-byte copies.  Copy j of fragment f
  // moves tile rows 8j .. 8j+7 x the chunk's 128 bytes (8 pieces of 16 bytes,
  // 8 whole rows per instruction); slot s of the copy receives piece
  // (s % 8) ^ (row % 8) of row 8j + s / 8, so that the MFMA-layout reads below
  // (lane: row l32, piece 2c + half) fall in distinct banks.  Pieces past the
  // wave's K range copy valid bytes of the range that nobody reads.
  const uint8_t* srcrow[NF][4];
  const int crr = lane >> 3;
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int trow = 8 * j + crr;
      const int64_t row = f < FM ? min(m0 + 32 * f + trow, M - 1) : min(n0 + 32 * (f - FM) + trow, N - 1);
      srcrow[f][j] = (f < FM ? xc : wc) + row * KB;
    }
  const int cp = (lane & 7) ^ (crr & 7);     // the piece this lane copies (rows 8j + crr)
  auto issue = [&](int g0) {
    const int g = g0 + (cp >> 1) < gend ? g0 + (cp >> 1) : g0;
#pragma unroll
    for (int f = 0; f < NF; ++f)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        lds_copy16(srcrow[f][j] + 32 * (int64_t)g + 16 * (cp & 1), &stage[wave][(f * 4 + j) * 64]);
  };
  static_assert(CH == 4, "a chunk's scales are one 16-byte load");
  auto load_scales = [&](uint32_t (&sw)[CH][NF], int g0) {
    // the chunk's 4 groups' scales (16 consecutive bytes of the row) in one
    // load when they are whole and 16-byte aligned
    if ((KS & 15) == 0 && (g0 & 3) == 0 && g0 + CH <= gend) {
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const u32x4_t q = *reinterpret_cast<const u32x4_t*>(srow[f] + 4 * (int64_t)g0);
#pragma unroll
        for (int c = 0; c < CH; ++c) sw[c][f] = q[c];
      }
    } else {
#pragma unroll
      for (int c = 0; c < CH; ++c)
        if (g0 + c < gend)
#pragma unroll
          for (int f = 0; f < NF; ++f)
            sw[c][f] = *reinterpret_cast<const uint32_t*>(srow[f] + 4 * (int64_t)(g0 + c));
    }
  };
  auto fetch = [&](u32x4_t (&cw)[CH][NF]) {
    const int key = l32 & 7;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int f = 0; f < NF; ++f)
        cw[c][f] = stage[wave][(f * 4 + (l32 >> 3)) * 64 + key * 8 + ((2 * c + half) ^ key)];
  };
  auto compute = [&](const u32x4_t (&cw)[CH][NF], const uint32_t (&sw)[CH][NF], int g0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (g0 + c >= gend) break;
      half2_t sp[NF];  // this lane's two block scales of the group, as fp16
#pragma unroll
      for (int f = 0; f < NF; ++f)
        sp[f] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw[c][f] >> (16 * half), 1.0f, false);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        half8_t fr[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) fr[f] = decode8(cw[c][f][t], sp[f][t >> 1]);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[i], fr[FM + j], acc[i][j], 0, 0, 0);
      }
    }
  };
  uint32_t sw[CH][NF];
  issue(gbeg);
  load_scales(sw, gbeg);
  for (int g0 = gbeg; g0 < gend; g0 += CH) {
    // the copies into this wave's slot have landed (and nothing else of the
    // wave is in flight); the memory clobber keeps the LDS reads below
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    u32x4_t cw[CH][NF];
    fetch(cw);
    const bool more = g0 + CH < gend;
    uint32_t swn[CH][NF];
    if (more) {
      // the reads of the slot are complete before it is refilled
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue(g0 + CH);
      load_scales(swn, g0 + CH);
    }
    compute(cw, sw, g0);
    if (more)
#pragma unroll
      for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int f = 0; f < NF; ++f) sw[c][f] = swn[c][f];
  }
  __syncthreads();  // every wave is done with the staging slots: they become the partials

  // low-rank branch bf16(u) wv^T: this wave's steps, into its partial
#pragma unroll
  for (int k = 0; k < LRW; ++k) {
    const int cb = 16 * (wave + k * W) + 8 * half;
    if (cb - 8 * half >= r) continue;
    bf16x8_t la[FM], lb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float f[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = cb + e < r ? lu[k][i][e >> 2][e & 3] : 0.0f;
      la[i] = bf16x8_rne(f);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        lb[j][e] = bf16_from_bits(cb + e < r ? (uint16_t)(lw[k][j][e >> 1] >> (16 * (e & 1))) : (uint16_t)0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[i], lb[j], acc[i][j], 0, 0, 0);
  }

  // partial tiles to LDS (accumulator element v of lane l: row 8*(v/4) +
  // 4*(l/32) + v%4, column l%32), then the fixed-order sum, bias and store
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        part[wave][32 * i + 8 * (v >> 2) + 4 * half + (v & 3)][32 * j + l32] = acc[i][j][v];
  __syncthreads();
  if (gm >= M) return;
  float out[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) s += part[w][orow][ocol + e];
    out[e] = s + ((bias && gn + e < N) ? bv[e] : 0.0f);
  }
  const int64_t base = (int64_t)gm * N + gn;
  if (y_bf16) {
    uint16_t* yo = reinterpret_cast<uint16_t*>(y) + base;
    if (gn + EPT <= N && (base & 3) == 0 && EPT % 4 == 0) {
#pragma unroll
      for (int e = 0; e < EPT; e += 4) {
        uint2 pk;
        pk.x = bf16x2_rne(out[e], out[e + 1]);
        pk.y = bf16x2_rne(out[e + 2], out[e + 3]);
        *reinterpret_cast<uint2*>(yo + e) = pk;
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (gn + e < N) yo[e] = bf16_rne(out[e]);
    }
  } else {
    float* yo = reinterpret_cast<float*>(y) + base;
    if (gn + EPT <= N && (base & 3) == 0 && EPT % 4 == 0) {
#pragma unroll
      for (int e = 0; e < EPT; e += 4)
        *reinterpret_cast<float4*>(yo + e) = make_float4(out[e], out[e + 1], out[e + 2], out[e + 3]);
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (gn + e < N) yo[e] = out[e];
    }
  }
}

// Waves per workgroup for k_gemm_sk: K split into W ranges of at least 256
// elements (at most 8 ranges), each a whole number of 64-element groups.
int sk_waves(int64_t K) {
  const int64_t groups = K / 64;
  for (int w : {8, 4, 2})
    if (K / w >= 256 && groups % w == 0) return w;
  return 1;
}

template <int FM, int FN, int W>
__global__ void __launch_bounds__(W * 64)
    k_gemm_sk(const GemmArgs a, int M, int K, int r, int y_bf16, int tiles_m) {
  const GemmLayerArgs& L = a.l[blockIdx.y];
  if ((int)blockIdx.x >= tiles_m * L.tiles_n) return;
  gemm_sk_body<FM, FN, W>(L.xc, L.xs, L.u, M, L.N, K, r, L.wc, L.ws, L.wv, L.bias, L.y, y_bf16,
                          L.tiles_n);
}

template <int FM, int FN, int W>
int32_t launch_gemm_sk(int n, const GemmCall* calls, int64_t M, int64_t K, int32_t r,
                       int32_t y_dtype, hipStream_t stream) {
  GemmArgs a;
  int64_t tiles_m, max_tiles;
  ASP_TRY(group_args(n, calls, M, 32 * FM, 32 * FN, a, tiles_m, max_tiles));
  hipLaunchKernelGGL((k_gemm_sk<FM, FN, W>), dim3((unsigned)max_tiles, (unsigned)n), dim3(W * 64),
                     0, stream, a, (int)M, (int)K, (int)r, (int)(y_dtype == ASP_BF16),
                     (int)tiles_m);
  return launch_status("gemm_sk");
}

}  // namespace

int32_t gemm_check(int64_t M, int64_t N, int64_t K, int32_t r, int32_t y_dtype) {
  ASP_TRY(check_mk(M, K));
  ASP_TRY(check_rank(r));
  if (N < 1 || N > INT32_MAX) return fail(ASP_ERR_SHAPE, "N=%lld outside [1, 2^31)", (long long)N);
  if (y_dtype != ASP_F32 && y_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "y_dtype=%d", y_dtype);
  return ASP_OK;
}

enum GemmVariant { kGemm512x96, kGemm256x192, kGemm64x64, kGemmSplitK8, kGemmSplitK4,
                   kGemmSplitK2, kGemmSplitK1 };

// Tile choice.  Large layers with K % 256 == 0 and at least 256 tiles of 512
// x 96 (one per CU for a 4096 x 3072 output): k_gemm_wb, whose weight tile is
// decoded once per workgroup and whose activation fragments are decoded once,
// by the one wave that uses them (two decodes per six MFMAs a K-step, plus the
// workgroup's share of the weight decode).  Other large layers: 256 x 192
// workgroup tiles of 8 waves with 64 x 96 per-wave tiles (five fragment
// decodes feed six MFMAs per K-step); in both, two waves per SIMD overlap one
// wave's decode with the other's MFMAs.  Mid-size layers (M > 256) with at
// least 256 tiles of 64 x 64: those tiles, 4 waves each (at M = 256 the
// split-K form is faster: 8.2 against 9.4 us at N = 4096, K = 1024).  Fewer
// tiles (small M): 32 x 32 tiles with K split over the workgroup's waves
// (k_gemm_sk), so that more waves share the work and each one's chain of
// dependent K-steps is shorter.
GemmVariant gemm_variant(int64_t M, int64_t N, int64_t K) {
  if (K % wb::BK == 0 && ((M + wb::BM - 1) / wb::BM) * ((N + wb::BN - 1) / wb::BN) >= 256)
    return kGemm512x96;
  if (((M + 255) / 256) * ((N + 191) / 192) >= 128) return kGemm256x192;
  if (M > 256 && ((M + 63) / 64) * ((N + 63) / 64) >= 256) return kGemm64x64;
  switch (sk_waves(K)) {
    case 8: return kGemmSplitK8;
    case 4: return kGemmSplitK4;
    case 2: return kGemmSplitK2;
    default: return kGemmSplitK1;
  }
}

const char* gemm_variant_name(GemmVariant v) {
  switch (v) {
    case kGemm512x96: return "k_gemm_wb";
    case kGemm256x192: return "k_gemm<4, 2, 2, 3>";
    case kGemm64x64: return "k_gemm<2, 2, 1, 1>";
    case kGemmSplitK8: return "k_gemm_sk<1, 1, 8>";
    case kGemmSplitK4: return "k_gemm_sk<1, 1, 4>";
    case kGemmSplitK2: return "k_gemm_sk<1, 1, 2>";
    default: return "k_gemm_sk<1, 1, 1>";
  }
}

int32_t gemm_impl(int n, const GemmCall* calls, int64_t M, int64_t K, int32_t r, int32_t y_dtype,
                  hipStream_t stream) {
  if (n < 1 || n > kMaxGroup) return fail(ASP_ERR_ARG, "group of %d layers outside [1, %d]", n, kMaxGroup);
  int64_t n_total = 0;
  for (int i = 0; i < n; ++i) {
    ASP_TRY(gemm_check(M, calls[i].N, K, r, y_dtype));
    n_total += calls[i].N;
  }
  if (M == 0) return ASP_OK;
  for (int i = 0; i < n; ++i) {
    const GemmCall& c = calls[i];
    ASP_TRY(check_ptr(c.x_codes, "x_codes", true));
    ASP_TRY(check_ptr(c.x_scales, "x_scales", true));
    ASP_TRY(check_ptr(c.u, "u", r > 0));
    ASP_TRY(check_ptr(c.w_codes, "w_codes", true));
    ASP_TRY(check_ptr(c.w_scales, "w_scales", true));
    ASP_TRY(check_ptr(c.wv, "wv", r > 0));
    ASP_TRY(check_ptr(c.bias, "bias", false));
    ASP_TRY(check_ptr(c.y, "y", true));
  }
  // one kernel for the whole group, chosen for its total output width
  switch (gemm_variant(M, n_total, K)) {
    case kGemm512x96: return launch_gemm_wb(n, calls, M, K, r, y_dtype, stream);
    case kGemm256x192: return launch_gemm<4, 2, 2, 3>(n, calls, M, K, r, y_dtype, stream);
    case kGemm64x64: return launch_gemm<2, 2, 1, 1>(n, calls, M, K, r, y_dtype, stream);
    case kGemmSplitK8: return launch_gemm_sk<1, 1, 8>(n, calls, M, K, r, y_dtype, stream);
    case kGemmSplitK4: return launch_gemm_sk<1, 1, 4>(n, calls, M, K, r, y_dtype, stream);
    case kGemmSplitK2: return launch_gemm_sk<1, 1, 2>(n, calls, M, K, r, y_dtype, stream);
    default: return launch_gemm_sk<1, 1, 1>(n, calls, M, K, r, y_dtype, stream);
  }
}

}  // namespace asp

using namespace asp;

extern "C" {

int32_t asp_gemm_lowrank(const uint8_t* x_codes, const uint8_t* x_scales, const float* u,
                         int64_t M, int64_t N, int64_t K, int32_t r, const uint8_t* w_codes,
                         const uint8_t* w_scales, const uint16_t* wv, const float* bias, void* y,
                         int32_t y_dtype, void* stream) {
  clear_error();
  const GemmCall c = {x_codes, x_scales, u, w_codes, w_scales, wv, bias, y, N};
  return gemm_impl(1, &c, M, K, r, y_dtype, (hipStream_t)stream);
}

const char* asp_gemm_kernel_name(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N <= 0 || K <= 0 || K % 128 != 0) return "";
  return gemm_variant_name(gemm_variant(M, N, K));
}

}  // extern "C"
