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
// operands are therefore decoded in registers to exact fp16 (E2M1 value x
// E4M3 scale has at most 6 significant bits and lies in [2^-10, 2688]) and
// contracted on v_mfma_f32_32x32x16_f16: one MFMA K-step is exactly one NVFP4
// block, and only fp32 accumulation order differs from exact arithmetic.  The
// low-rank branch adds ceil(r/16) bf16 MFMA K-steps into the same
// accumulators; bias and the output cast follow.
//
// Decoding a lane's 8 elements of a fragment costs 8 VALU instructions (four
// 2-code conversions, four packed fp16 scale multiplies); two waves share each
// SIMD so that one wave's decode overlaps the other's MFMAs.  Codes and scales are staged through double-buffered LDS in stages of
// 256 K-elements (16 MFMA K-steps per workgroup barrier).  Tile rows are padded
// so that the 32 rows a fragment reads hit distinct banks, and each lane reads
// the one 32-bit code word it needs per K-step one step ahead of its use, so
// the LDS latency hides behind the current K-step's decode and MFMAs.  Scale
// bytes are converted to fp16 once, when a stage is written to LDS.
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

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  if (nk > 1) gload(1);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const uint8_t* base = smem + (kc & 1) * C::STAGE;
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
  // operand rows are fetched with vector loads when r is a multiple of 8.
  for (int c0 = 0; c0 < r; c0 += 16) {
    bf16x8_t la[TM], lb[TN];
    const int cb = c0 + half * 8;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = min(m0 + (wm * TM + i) * 32 + l32, M - 1);
      float f[8];
      if ((r & 7) == 0) {
        const float4 p = *reinterpret_cast<const float4*>(u + m * r + cb);
        const float4 q = *reinterpret_cast<const float4*>(u + m * r + cb + 4);
        f[0] = p.x; f[1] = p.y; f[2] = p.z; f[3] = p.w; f[4] = q.x; f[5] = q.y; f[6] = q.z; f[7] = q.w;
        if (cb >= r) for (int e = 0; e < 8; ++e) f[e] = 0.0f;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = cb + e < r ? u[m * r + cb + e] : 0.0f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) la[i][e] = bf16_from_bits(f32_to_bf16_rne(f[e]));
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t n = min(n0 + (wn * TN + j) * 32 + l32, N - 1);
      if ((r & 7) == 0) {
        uint4 q = cb < r ? *reinterpret_cast<const uint4*>(wv + n * r + cb) : make_uint4(0, 0, 0, 0);
        lb[j] = __builtin_bit_cast(bf16x8_t, q);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) lb[j][e] = bf16_from_bits(cb + e < r ? wv[n * r + cb + e] : (uint16_t)0);
      }
    }
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[i], lb[j], acc[i][j], 0, 0, 0);
  }

  // bias and store; accumulator element v of lane l is row 8*(v/4) + 4*(l/32)
  // + v%4 and column l%32 of its 32 x 32 tile
  float bj[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int col = n0 + (wn * TN + j) * 32 + l32;
    bj[j] = (bias && col < N) ? bias[col] : 0.0f;
  }
  if (y_bf16) {
    // through LDS (the staging buffers are free once every wave is past the
    // K loop), so that each thread writes 16 consecutive bytes of a row
    static_assert(C::BM * C::BN * 2 <= C::LDS, "output tile must fit the staging LDS");
    __syncthreads();
    uint16_t* ot = reinterpret_cast<uint16_t*>(smem);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = (wm * TM + i) * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          const int col = (wn * TN + j) * 32 + l32;
          ot[row * C::BN + col] = f32_to_bf16_rne(acc[i][j][v] + bj[j]);
        }
    __syncthreads();
    uint16_t* yo = reinterpret_cast<uint16_t*>(y);
    constexpr int CHUNKS = C::BM * C::BN / 8;
    for (int c = tid; c < CHUNKS; c += C::NT) {
      const int row = c / (C::BN / 8), col = (c % (C::BN / 8)) * 8;
      const int gm = m0 + row, gn = n0 + col;
      if (gm >= M) continue;
      const int64_t off = (int64_t)gm * N + gn;
      const u32x4_t val = *reinterpret_cast<const u32x4_t*>(ot + row * C::BN + col);
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
      const int col = n0 + (wn * TN + j) * 32 + l32;
      if (col >= N) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = m0 + (wm * TM + i) * 32 + 8 * (v >> 2) + 4 * half + (v & 3);
          if (row < M) reinterpret_cast<float*>(y)[(int64_t)row * N + col] = acc[i][j][v] + bj[j];
        }
    }
  }
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
  constexpr int CH = 4;                      // groups of 64 K per register chunk
  constexpr int EPT = BM * BN / (W * 64);    // output elements per thread
  __shared__ float part[W][BM][BN + 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * BM, n0 = tn * BN;
  const int64_t KB = K / 2, KS = K / 16;
  const int ng = K / 64 / W;                 // groups of this wave
  const int gbeg = wave * ng, gend = gbeg + ng;

  const uint8_t* crow[NF];
  const uint8_t* srow[NF];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int64_t row = f < FM ? min(m0 + 32 * f + l32, M - 1) : min(n0 + 32 * (f - FM) + l32, N - 1);
    crow[f] = (f < FM ? xc : wc) + row * KB + 16 * half;
    srow[f] = (f < FM ? xs : ws) + row * KS;
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  uint4 cw[2][CH][NF];
  uint32_t sw[2][CH][NF];
  auto load = [&](int buf, int g0) {
#pragma unroll
    for (int c = 0; c < CH; ++c)
      if (g0 + c < gend)
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          cw[buf][c][f] = *reinterpret_cast<const uint4*>(crow[f] + 32 * (int64_t)(g0 + c));
          sw[buf][c][f] = *reinterpret_cast<const uint32_t*>(srow[f] + 4 * (int64_t)(g0 + c));
        }
  };
  auto compute = [&](int buf, int g0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      if (g0 + c >= gend) break;
      half2_t sp[NF];  // this lane's two block scales of the group, as fp16
#pragma unroll
      for (int f = 0; f < NF; ++f)
        sp[f] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw[buf][c][f] >> (16 * half), 1.0f, false);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        half8_t fr[NF];
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const uint4 q = cw[buf][c][f];
          const uint32_t wd = t == 0 ? q.x : t == 1 ? q.y : t == 2 ? q.z : q.w;
          fr[f] = decode8(wd, sp[f][t >> 1]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fr[i], fr[FM + j], acc[i][j], 0, 0, 0);
      }
    }
  };
  load(0, gbeg);
  for (int g0 = gbeg; g0 < gend; g0 += 2 * CH) {
    if (g0 + CH < gend) load(1, g0 + CH);
    compute(0, g0);
    if (g0 + CH >= gend) break;
    if (g0 + 2 * CH < gend) load(0, g0 + 2 * CH);
    compute(1, g0 + CH);
  }

  // low-rank branch bf16(u) wv^T, in the first wave's partial
  if (wave == 0) {
    for (int c0 = 0; c0 < r; c0 += 16) {
      const int cb = c0 + half * 8;
      bf16x8_t la[FM], lb[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int64_t m = min(m0 + 32 * i + l32, M - 1);
#pragma unroll
        for (int e = 0; e < 8; ++e)
          la[i][e] = bf16_from_bits(f32_to_bf16_rne(cb + e < r ? u[m * r + cb + e] : 0.0f));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int64_t n = min(n0 + 32 * j + l32, N - 1);
#pragma unroll
        for (int e = 0; e < 8; ++e) lb[j][e] = bf16_from_bits(cb + e < r ? wv[n * r + cb + e] : (uint16_t)0);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(la[i], lb[j], acc[i][j], 0, 0, 0);
    }
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
  const int e0 = tid * EPT, row = e0 / BN, col = e0 % BN;
  const int gm = m0 + row, gn = n0 + col;
  if (gm >= M) return;
  float out[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    float s = 0.0f;
#pragma unroll
    for (int w = 0; w < W; ++w) s += part[w][row][col + e];
    out[e] = s + ((bias && gn + e < N) ? bias[gn + e] : 0.0f);
  }
  const int64_t base = (int64_t)gm * N + gn;
  if (y_bf16) {
    uint16_t* yo = reinterpret_cast<uint16_t*>(y) + base;
    if (gn + EPT <= N && (base & 7) == 0 && EPT % 8 == 0) {
#pragma unroll
      for (int e = 0; e < EPT; e += 8) {
        uint4 pk;
        pk.x = f32_to_bf16_rne(out[e]) | ((uint32_t)f32_to_bf16_rne(out[e + 1]) << 16);
        pk.y = f32_to_bf16_rne(out[e + 2]) | ((uint32_t)f32_to_bf16_rne(out[e + 3]) << 16);
        pk.z = f32_to_bf16_rne(out[e + 4]) | ((uint32_t)f32_to_bf16_rne(out[e + 5]) << 16);
        pk.w = f32_to_bf16_rne(out[e + 6]) | ((uint32_t)f32_to_bf16_rne(out[e + 7]) << 16);
        *reinterpret_cast<uint4*>(yo + e) = pk;
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (gn + e < N) yo[e] = f32_to_bf16_rne(out[e]);
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

enum GemmVariant { kGemm256x192, kGemm64x64, kGemmSplitK8, kGemmSplitK4, kGemmSplitK2,
                   kGemmSplitK1 };

// Tile choice.  Large layers: 256 x 192 workgroup tiles (256 tiles, one per
// CU, for a 4096 x 3072 output) of 8 waves with 64 x 96 per-wave tiles: five
// fragment decodes feed six MFMAs per K-step, and two waves per SIMD overlap
// one wave's decode with the other's MFMAs.  Mid-size layers with at least
// 256 tiles of 64 x 64: those tiles, 4 waves each.  Fewer tiles (small M):
// 32 x 32 tiles with K split over the workgroup's waves (k_gemm_sk), so that
// more waves share the work and each one's chain of dependent K-steps is
// shorter.
GemmVariant gemm_variant(int64_t M, int64_t N, int64_t K) {
  if (((M + 255) / 256) * ((N + 191) / 192) >= 128) return kGemm256x192;
  if (((M + 63) / 64) * ((N + 63) / 64) >= 256) return kGemm64x64;
  switch (sk_waves(K)) {
    case 8: return kGemmSplitK8;
    case 4: return kGemmSplitK4;
    case 2: return kGemmSplitK2;
    default: return kGemmSplitK1;
  }
}

const char* gemm_variant_name(GemmVariant v) {
  switch (v) {
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
