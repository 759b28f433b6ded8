// Top-r eigenspace of a symmetric positive semi-definite metric G (K x K):
// the protected basis V of a layer.  Model card "FastWAM UR3 3-task -- 4-bit
// quantisations", section "What ASP is, and what the deflated form means": V
// spans the top eigenspace of the layer's action metric G = E[J^T J]; Q-WAM,
// Figure 3(b): that metric's leading eigenvalues fall quickly, so a block of
// p = r + oversampling vectors converges in a few subspace iterations.
//
// Method (all arithmetic in float64; G is read as float32):
//   mu   = 2^-16 ||G||_F (1 when G = 0): a shift that keeps G + mu I positive
//          definite, so every iterate has full rank even when G does not;
//   V    = orthonormal basis of the caller's random start V0 (K x p);
//   iters times:  Y = (G + mu I) V,  V = Y R^-1  with R^T R = Y^T Y
//          (Cholesky QR; Y's condition number is at most ~ ||G|| / mu);
//   V    = V R^-1 once more (Cholesky QR2: orthonormal to rounding);
//   Rayleigh-Ritz: Y = G V, T = (V^T Y + Y^T V) / 2 (p x p), T = Z diag(theta) Z^T
//          by cyclic Jacobi rotations (Golub & Van Loan, "Matrix Computations",
//          the symmetric Schur decomposition of a 2 x 2 block and the parallel
//          round-robin ordering), sorted largest first;
//   output the r leading Ritz pairs: V Z[:, :r] (each column's largest-magnitude
//          entry made positive), theta[:r] and ||G v - theta v||.
//
// Kernels: G V on float64 MFMA (v_mfma_f64_16x16x4f64), K split into slices
// whose partial products are summed in a fixed order; Gram sums per 64-row
// block, reduced in a fixed order; Cholesky, triangular inverse and Jacobi in
// one workgroup each (p <= 64).  Every reduction has a fixed order, so results
// are bitwise reproducible run to run.
#include "asp_device.h"

#include <cmath>

namespace asp {
namespace {

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// 1/sqrt(d) and 1/x for positive normal d and nonzero normal x: the hardware
// estimate (v_rsq_f64, v_rcp_f64) refined by two Newton-Raphson steps
// (y <- y + y (1 - d y^2) / 2 and y <- y + y (1 - x y)), each of which roughly
// doubles the number of correct bits, to within a few ulps.
__device__ __forceinline__ double rsqrt_nr(double d) {
  double y = __builtin_amdgcn_rsq(d);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double r = fma(-(d * y), y, 1.0);
    y = fma(0.5 * y, r, y);
  }
  return y;
}
__device__ __forceinline__ double rcp_nr(double x) {
  double y = __builtin_amdgcn_rcp(x);
#pragma unroll
  for (int it = 0; it < 2; ++it) y = fma(y, fma(-x, y, 1.0), y);
  return y;
}

constexpr int kEigMaxP = 64;
constexpr int64_t kEigMaxK = 65536;
constexpr int kRows = 64;   // rows per block of the row-blocked kernels
constexpr int kBK = 32;     // K-chunk of the G V kernel

// --------------------------------------------------------------- G V (MFMA)

// yp[s] = G[:, slice s] V[slice s, :] for one 64-row tile of G per workgroup.
// Wave w owns rows 16w..16w+15 and all p columns (p/16 accumulator tiles).
// MFMA operands: lane (lr = lane % 16, lg = lane / 16) supplies A[lr][lg] and
// B[lg][lr]; a lane's float4 of G covers k = 4 lg + j (j = 0..3) of a 16-k
// group, so MFMA step j contracts over k = 4 lg + j for lg = 0..3, and the B
// operand is V's row at that same k.  Accumulator element v of a lane is
// output row lg + 4 v, column lr (the float64 16x16x4 MFMA interleaves its
// output rows across lane groups; checked on gfx950 with lane-coded inputs).
// V chunks (32 rows x p) are staged in LDS by
// direct global-to-LDS copies, double buffered; G goes straight to registers.
template <int P>
__global__ void __launch_bounds__(256) k_eig_gv(const float* __restrict__ g,
                                                const double* __restrict__ v,
                                                double* __restrict__ yp, int K, int slice) {
  constexpr int NT = P / 16;
  __shared__ __attribute__((aligned(16))) double vs[2][kBK * P];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;
  const int row0 = blockIdx.x * kRows + wave * 16;
  const int k_lo = blockIdx.y * slice, nch = slice / kBK;
  const float* grow = g + (int64_t)(row0 + lr) * K + k_lo + 4 * lg;
  const double* vsl = v + (int64_t)k_lo * P;

  auto stage = [&](int c, int buf) {
    // kBK x P doubles, contiguous in V; 16 bytes per lane per copy
#pragma unroll
    for (int i = 0; i < P / 16; ++i)
      lds_copy16(vsl + (int64_t)c * kBK * P + (i * 256 + tid) * 2, &vs[buf][(i * 256 + wave * 64) * 2]);
  };
  auto gload = [&](int c, f32x4_t (&out)[2]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      out[h] = *reinterpret_cast<const f32x4_t*>(grow + c * kBK + 16 * h);
  };

  f64x4_t acc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) acc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  f32x4_t gnext[2];
  stage(0, 0);
  gload(0, gnext);
  for (int c = 0; c < nch; ++c) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const f32x4_t gcur[2] = {gnext[0], gnext[1]};
    if (c + 1 < nch) {
      stage(c + 1, (c + 1) & 1);
      gload(c + 1, gnext);
    }
    const double* vb = vs[c & 1];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const double a = (double)gcur[h][j];
        const int kr = 16 * h + 4 * lg + j;
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, vb[kr * P + t * 16 + lr], acc[t], 0, 0, 0);
      }
  }
  double* out = yp + ((int64_t)blockIdx.y * K + row0) * P;
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int e = 0; e < 4; ++e) out[(int64_t)(lg + 4 * e) * P + t * 16 + lr] = acc[t][e];
}

// ------------------------------------------------------- row-blocked passes

// Rows of the per-block LDS tiles are padded to P + 2 doubles (16-byte aligned
// rows, consecutive rows on different banks).
template <int P>
using Tile = double[kRows][P + 2];

// Partial Gram sums of one 64-row block: part[a][b] = sum_rows L[row][a] R[row][b],
// rows in ascending order (L = R gives an exactly symmetric result).  Thread t
// owns a 4 x 4 block of entries, so each pair of 4-wide row reads feeds 16 FMAs.
template <int P>
__device__ __forceinline__ void block_gram(const double (*L)[P + 2], const double (*R)[P + 2],
                                           double* __restrict__ part) {
  constexpr int NB = P / 4;
  const int t = threadIdx.x;
  if (t >= NB * NB) return;
  const int a0 = (t / NB) * 4, b0 = (t % NB) * 4;
  double acc[4][4] = {};
#pragma unroll 4
  for (int i = 0; i < kRows; ++i) {
    double la[4], rb[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      la[x] = L[i][a0 + x];
      rb[x] = R[i][b0 + x];
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) acc[x][y] = fma(la[x], rb[y], acc[x][y]);
  }
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) part[(a0 + x) * P + b0 + y] = acc[x][y];
}

enum GramMode { kCast = 0, kShift = 1, kCross = 2 };

// Forms one 64-row block of Y and its Gram partial:
//   kCast : Y = float64(v0)                      part = Y^T Y
//   kShift: Y = sum_s yp[s] + mu V               part = Y^T Y
//   kCross: Y = sum_s yp[s]                      part = V^T Y
// slices are added in ascending order; each thread keeps its P/4 elements'
// loads of one slice in flight together.
template <int P, int MODE>
__global__ void __launch_bounds__(256) k_eig_gram(const float* __restrict__ v0,
                                                  const double* __restrict__ yp, int nslices,
                                                  const double* __restrict__ v,
                                                  const double* __restrict__ scal, int K,
                                                  double* __restrict__ y, double* __restrict__ cp) {
  constexpr int EPT = kRows * P / 256;
  __shared__ __attribute__((aligned(16))) Tile<P> ys;
  __shared__ __attribute__((aligned(16))) double vsh[MODE == kCross ? kRows : 1][P + 2];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kRows * P;
  double acc[EPT];
  if constexpr (MODE == kCast) {
#pragma unroll
    for (int q = 0; q < EPT; ++q) acc[q] = (double)v0[base + tid + 256 * q];
  } else {
#pragma unroll
    for (int q = 0; q < EPT; ++q) acc[q] = 0.0;
    for (int s = 0; s < nslices; ++s) {
      const double* src = yp + (int64_t)s * K * P + base + tid;
#pragma unroll
      for (int q = 0; q < EPT; ++q) acc[q] += src[256 * q];
    }
  }
#pragma unroll
  for (int q = 0; q < EPT; ++q) {
    const int e = tid + 256 * q, i = e / P, c = e % P;
    if constexpr (MODE == kShift) acc[q] = fma(scal[0], v[base + e], acc[q]);
    if constexpr (MODE == kCross) vsh[i][c] = v[base + e];
    ys[i][c] = acc[q];
    y[base + e] = acc[q];
  }
  __syncthreads();
  block_gram<P>(MODE == kCross ? vsh : ys, ys, cp + (int64_t)blockIdx.x * P * P);
}

// c[e] = sum over blocks b (ascending) of cp[b][e].
template <int P>
__global__ void __launch_bounds__(64) k_eig_reduce(const double* __restrict__ cp, int nb,
                                                   double* __restrict__ c) {
  const int e = blockIdx.x * 64 + threadIdx.x;
  double s = 0.0;
#pragma unroll 8
  for (int b = 0; b < nb; ++b) s += cp[(int64_t)b * P * P + e];
  c[e] = s;
}

// vout = Y X^T for one 64-row block (X lower triangular, so column j of the
// output mixes Y's columns 0..j, in ascending order; the zeros above X's
// diagonal that a 4-wide block also reads add exactly nothing).  Thread t owns
// a 4 x 4 block of outputs.  With GRAM, also the Gram partial of vout.
template <int P, bool GRAM>
__global__ void __launch_bounds__(256) k_eig_apply(const double* __restrict__ yin,
                                                   const double* __restrict__ xm,
                                                   double* __restrict__ vout,
                                                   double* __restrict__ cp) {
  constexpr int NB = P / 4;
  __shared__ __attribute__((aligned(16))) Tile<P> ys;
  __shared__ __attribute__((aligned(16))) double xs[P][P + 2];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kRows * P;
  for (int e = tid; e < kRows * P; e += 256) ys[e / P][e % P] = yin[base + e];
  for (int e = tid; e < P * P; e += 256) xs[e / P][e % P] = xm[e];
  __syncthreads();
  const bool owner = tid < 16 * NB;
  const int i0 = (tid / NB) * 4, j0 = (tid % NB) * 4;
  double acc[4][4] = {};
  if (owner) {
    for (int k = 0; k < j0 + 4; ++k) {
      double a[4], b[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        a[x] = ys[i0 + x][k];
        b[x] = xs[j0 + x][k];
      }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = fma(a[x], b[y], acc[x][y]);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) vout[base + (int64_t)(i0 + x) * P + j0 + y] = acc[x][y];
  }
  if constexpr (GRAM) {
    __syncthreads();  // every thread is done reading ys
    if (owner) {
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) ys[i0 + x][j0 + y] = acc[x][y];
    }
    __syncthreads();
    block_gram<P>(ys, ys, cp + (int64_t)blockIdx.x * P * P);
  }
}

// --------------------------------------------------------- one-workgroup steps

__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)b, lane);
  const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(b >> 32), lane);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Cholesky C = L L^T and X = L^-1, blocked by 16 (P/16 block steps).
// Step jb: wave 0 factors the 16 x 16 diagonal block in registers (lane l
// holds row l; the pivot and each finished column element reach the other
// lanes by readlane, no barrier) and inverts it (lane c solves for column c);
// then all waves form the panel below it, L_ij = C_ij L_jj^-T, and update the
// trailing lower triangle, C_ik -= L_ij L_kj^T (right-looking order).  The
// inverse's off-diagonal blocks follow by block forward substitution,
// X_ij = -L_ii^-1 sum_{j <= k < i} L_ik X_kj, one block row at a time.  A pivot
// that is not a positive finite normal number is replaced by 1 and recorded in
// scal[1].
template <int P>
__global__ void __launch_bounds__(256) k_eig_chol(const double* __restrict__ cin,
                                                  double* __restrict__ xm,
                                                  double* __restrict__ scal) {
  constexpr int NB = P / 16;
  __shared__ double C[P][P + 1];
  __shared__ double X[P][P + 1];
  __shared__ double Pn[P][17];     // the panel of the current step / T blocks
  __shared__ int bad_flag;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < P * P; e += 256) {
    C[e / P][e % P] = cin[e];
    X[e / P][e % P] = 0.0;
  }
  if (tid == 0) bad_flag = 0;
  __syncthreads();
#pragma unroll 1
  for (int jb = 0; jb < NB; ++jb) {
    const int b0 = 16 * jb;
    if (wave == 0) {
      const int l = lane < 16 ? lane : 15;  // lanes past 16 mirror row 15 and store nothing
      double d[16], inv[16];
#pragma unroll
      for (int m = 0; m < 16; ++m) d[m] = C[b0 + l][b0 + m];
      bool bad_any = false;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        double pv = readlane_f64(d[k], k);
        const bool bad = !(pv >= 2.2250738585072014e-308) || __builtin_isinf(pv);
        if (bad) pv = 1.0;
        bad_any |= bad;
        inv[k] = rsqrt_nr(pv);
        const double piv = pv * inv[k];
        d[k] = l == k ? piv : (l > k ? d[k] * inv[k] : d[k]);
#pragma unroll
        for (int m = k + 1; m < 16; ++m) d[m] = fma(-d[k], readlane_f64(d[k], m), d[m]);
      }
      // column l of the block's inverse: x_r = (delta_{r,l} - sum_{t<r} L[r][t] x_t) / L[r][r]
      double x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        double acc = r == l ? 1.0 : 0.0;
#pragma unroll
        for (int t = 0; t < r; ++t) acc = fma(-readlane_f64(d[t], r), x[t], acc);
        x[r] = acc * inv[r];
      }
      if (lane < 16) {
#pragma unroll
        for (int m = 0; m < 16; ++m)
          if (m <= l) C[b0 + l][b0 + m] = d[m];
#pragma unroll
        for (int r = 0; r < 16; ++r) X[b0 + r][b0 + l] = x[r];
      }
      if (lane == 0 && bad_any) bad_flag = 1;
    }
    __syncthreads();
    const int lo = b0 + 16, rows = P - lo;
    // panel: Pn[i][c] = sum_{t <= c} C[i][b0 + t] Linv[c][t]
    for (int e = tid; e < rows * 16; e += 256) {
      const int i = lo + e / 16, c = e % 16;
      double acc = 0.0;
      for (int t = 0; t <= c; ++t) acc = fma(C[i][b0 + t], X[b0 + c][b0 + t], acc);
      Pn[i][c] = acc;
    }
    __syncthreads();
    // trailing lower triangle, and the panel into L
    for (int e = tid; e < rows * rows; e += 256) {
      const int i = lo + e / rows, k = lo + e % rows;
      if (k > i) continue;
      double acc = C[i][k];
#pragma unroll
      for (int c = 0; c < 16; ++c) acc = fma(-Pn[i][c], Pn[k][c], acc);
      C[i][k] = acc;
    }
    for (int e = tid; e < rows * 16; e += 256) {
      const int i = lo + e / 16, c = e % 16;
      C[i][b0 + c] = Pn[i][c];
    }
    __syncthreads();
  }
  // off-diagonal blocks of X, block row by block row
#pragma unroll 1
  for (int bi = 1; bi < NB; ++bi) {
    const int r0 = 16 * bi;
    // T_j = sum_{j <= k < bi} L[bi][k] X[k][j], for every block column j < bi, into Pn
    for (int e = tid; e < bi * 256; e += 256) {
      const int bj = e / 256, r = (e / 16) % 16, c = e % 16;
      double acc = 0.0;
      for (int t = 16 * bj; t < r0; ++t) acc = fma(C[r0 + r][t], X[t][16 * bj + c], acc);
      Pn[16 * bj + r][c] = acc;
    }
    __syncthreads();
    for (int e = tid; e < bi * 256; e += 256) {
      const int bj = e / 256, r = (e / 16) % 16, c = e % 16;
      double acc = 0.0;
      for (int t = 0; t <= r; ++t) acc = fma(-X[r0 + r][r0 + t], Pn[16 * bj + t][c], acc);
      X[r0 + r][16 * bj + c] = acc;
    }
    __syncthreads();
  }
  for (int e = tid; e < P * P; e += 256) xm[e] = X[e / P][e % P];
  if (tid == 0 && bad_flag) scal[1] = 1.0;
}

// mu = 2^-16 sqrt(sum of the Frobenius partials) (1 when that is 0); clears
// the breakdown flag.  One wave; fixed-order sums, so the result is the same
// on every run.
__global__ void __launch_bounds__(64) k_eig_mu(const double* __restrict__ fro, int nf,
                                               double* __restrict__ scal) {
  __shared__ double red[64];
  double s = 0.0;
  for (int b = threadIdx.x; b < nf; b += 64) s += fro[b];
  red[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x != 0) return;
  double t = 0.0;
  for (int i = 0; i < 64; ++i) t += red[i];
  const double mu = ldexp(sqrt(t), -16);
  scal[0] = mu > 0.0 ? mu : 1.0;
  scal[1] = 0.0;
}

constexpr int kFroRows = 8;  // rows of G per block of the Frobenius pass

// Sum of squares of kFroRows rows of G (float64; each thread's share in a
// fixed order, then a fixed-order tree in LDS).  K/8 blocks keep every CU
// streaming: the pass reads G once at close to the HBM rate.
__global__ void __launch_bounds__(256) k_eig_frob(const float* __restrict__ g, int K,
                                                  double* __restrict__ fro) {
  __shared__ double red[256];
  const f32x4_t* src = reinterpret_cast<const f32x4_t*>(g + (int64_t)blockIdx.x * kFroRows * K);
  const int n4 = kFroRows * K / 4;  // a multiple of 256 for K a multiple of 128
  double s = 0.0;
#pragma unroll 8
  for (int e = threadIdx.x; e < n4; e += 256) {
    const f32x4_t q = __builtin_nontemporal_load(src + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) s = fma((double)q[j], (double)q[j], s);
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) fro[blockIdx.x] = red[0];
}

// Symmetric eigendecomposition of T = (C + C^T)/2 (p x p) by cyclic Jacobi
// with the round-robin ordering: each step rotates p/2 disjoint index pairs
// at once (one thread computes each pair's rotation; then all threads apply
// them to 2 x 2 blocks of T and to Z).  Sweeps stop when the off-diagonal
// Frobenius norm falls to 1e-13 of the whole (rounding keeps it near 1e-16
// times a small factor, so a tighter bound might never be met), or after 40.  Outputs the
// eigenvalues largest first (equal ones in index order) and the matching
// eigenvector columns zs[:, m].
template <int P>
__global__ void __launch_bounds__(256) k_eig_jacobi(const double* __restrict__ cin,
                                                    double* __restrict__ theta,
                                                    double* __restrict__ zs,
                                                    double* __restrict__ scal) {
  constexpr int NP = P / 2;
  constexpr int NBLK = (NP * NP + 255) / 256;  // 2 x 2 blocks of T per thread
  constexpr int NZ = (NP * P + 255) / 256;     // (row, pair) items of Z per thread
  __shared__ double T[P][P + 1];
  __shared__ double Z[P][P + 1];
  __shared__ double cs[NP][2];
  __shared__ int pq[NP][2];
  __shared__ unsigned char sched[P - 1][NP][2];  // round-robin pairs, smaller index first
  __shared__ double red[256][2];
  __shared__ int perm[P];
  const int tid = threadIdx.x;
  for (int e = tid; e < P * P; e += 256) {
    const int a = e / P, b = e % P;
    T[a][b] = 0.5 * (cin[a * P + b] + cin[b * P + a]);
    Z[a][b] = a == b ? 1.0 : 0.0;
  }
  for (int e = tid; e < (P - 1) * NP; e += 256) {
    const int rnd = e / NP, i = e % NP;
    auto player = [&](int pos) { return pos == 0 ? 0 : 1 + (pos - 1 + rnd) % (P - 1); };
    const int a = player(i), b = player(P - 1 - i);
    sched[rnd][i][0] = (unsigned char)(a < b ? a : b);
    sched[rnd][i][1] = (unsigned char)(a < b ? b : a);
  }
  __syncthreads();
  for (int sweep = 0; sweep < 40; ++sweep) {
    double off = 0.0, all = 0.0;
    for (int e = tid; e < P * P; e += 256) {
      const double t = T[e / P][e % P];
      all = fma(t, t, all);
      if (e / P != e % P) off = fma(t, t, off);
    }
    red[tid][0] = off;
    red[tid][1] = all;
    __syncthreads();
    for (int w = 128; w > 0; w >>= 1) {
      if (tid < w) {
        red[tid][0] += red[tid + w][0];
        red[tid][1] += red[tid + w][1];
      }
      __syncthreads();
    }
    const bool done = !(red[0][0] > 1e-26 * red[0][1]);
    __syncthreads();  // everyone has read red before it is reused
    if (done) break;
    for (int rnd = 0; rnd < P - 1; ++rnd) {
      if (tid < NP) {
        const int a = sched[rnd][tid][0], b = sched[rnd][tid][1];
        const double app = T[a][a], aqq = T[b][b], apq = T[a][b];
        double c = 1.0, s = 0.0;
        if (fabs(apq) > 1e-300) {  // smaller entries are left as they are
          const double tau = (aqq - app) * rcp_nr(2.0 * apq);
          // the smaller root of t^2 + 2 tau t - 1 = 0; 1 / (2 tau) once tau^2 would overflow
          double t;
          if (fabs(tau) > 1e150) {
            t = 0.5 * rcp_nr(tau);
          } else {
            const double h = fma(tau, tau, 1.0);
            t = (tau >= 0.0 ? 1.0 : -1.0) * rcp_nr(fabs(tau) + h * rsqrt_nr(h));
          }
          c = rsqrt_nr(fma(t, t, 1.0));
          s = t * c;
        }
        cs[tid][0] = c;
        cs[tid][1] = s;
        pq[tid][0] = a;
        pq[tid][1] = b;
      }
      __syncthreads();
      // T = J^T T J, one 2 x 2 block (pair i's rows, pair i2's columns) per
      // item: each block is rebuilt from its own four entries (rows first,
      // then columns), so the blocks are independent; a diagonal block's
      // off-diagonal entries are the ones the rotation zeroes.  All of a
      // thread's loads are issued before its stores.
      {
        int ia[NBLK], ib[NBLK], ja[NBLK], jb[NBLK];
        double c1[NBLK], s1[NBLK], c2[NBLK], s2[NBLK], t4[NBLK][4];
#pragma unroll
        for (int n = 0; n < NBLK; ++n) {
          const int e = min(tid + 256 * n, NP * NP - 1), i = e / NP, i2 = e % NP;
          ia[n] = pq[i][0]; ib[n] = pq[i][1]; ja[n] = pq[i2][0]; jb[n] = pq[i2][1];
          c1[n] = cs[i][0]; s1[n] = cs[i][1]; c2[n] = cs[i2][0]; s2[n] = cs[i2][1];
        }
#pragma unroll
        for (int n = 0; n < NBLK; ++n) {
          t4[n][0] = T[ia[n]][ja[n]]; t4[n][1] = T[ia[n]][jb[n]];
          t4[n][2] = T[ib[n]][ja[n]]; t4[n][3] = T[ib[n]][jb[n]];
        }
#pragma unroll
        for (int n = 0; n < NBLK; ++n) {
          if (tid + 256 * n >= NP * NP) continue;
          const double c = c1[n], s = s1[n], cc = c2[n], ss = s2[n];
          const double raa = c * t4[n][0] - s * t4[n][2], rab = c * t4[n][1] - s * t4[n][3];
          const double rba = s * t4[n][0] + c * t4[n][2], rbb = s * t4[n][1] + c * t4[n][3];
          const bool diag_blk = ia[n] == ja[n];
          T[ia[n]][ja[n]] = cc * raa - ss * rab;
          T[ia[n]][jb[n]] = diag_blk ? 0.0 : ss * raa + cc * rab;
          T[ib[n]][ja[n]] = diag_blk ? 0.0 : cc * rba - ss * rbb;
          T[ib[n]][jb[n]] = ss * rba + cc * rbb;
        }
      }
      {  // Z = Z J: columns a and b of every row
        int za_[NZ], zb_[NZ], zk[NZ];
        double zc[NZ], zs_[NZ], va[NZ], vb[NZ];
#pragma unroll
        for (int n = 0; n < NZ; ++n) {
          const int e = min(tid + 256 * n, NP * P - 1), i = e / P;
          zk[n] = e % P; za_[n] = pq[i][0]; zb_[n] = pq[i][1];
          zc[n] = cs[i][0]; zs_[n] = cs[i][1];
        }
#pragma unroll
        for (int n = 0; n < NZ; ++n) {
          va[n] = Z[zk[n]][za_[n]];
          vb[n] = Z[zk[n]][zb_[n]];
        }
#pragma unroll
        for (int n = 0; n < NZ; ++n) {
          if (tid + 256 * n >= NP * P) continue;
          Z[zk[n]][za_[n]] = zc[n] * va[n] - zs_[n] * vb[n];
          Z[zk[n]][zb_[n]] = zs_[n] * va[n] + zc[n] * vb[n];
        }
      }
      __syncthreads();
    }
  }
  if (tid < P) {
    const double t = T[tid][tid];
    int rank = 0;
    for (int j = 0; j < P; ++j) {
      const double u = T[j][j];
      rank += (u > t) || (u == t && j < tid);
    }
    perm[rank] = tid;
  }
  __syncthreads();
  if (tid < P) theta[tid] = T[perm[tid]][perm[tid]];
  for (int e = tid; e < P * P; e += 256) zs[e] = Z[e / P][perm[e % P]];
  (void)scal;
}

// Ritz vectors of one 64-row block: vz = V z_m, residual G v - theta v =
// Y z_m - theta_m vz (Y = G V), for m < r.  Writes vz (float32) and per-block
// sums of squared residuals and the signed entry of largest |vz| (the first
// row on ties).
template <int P>
__global__ void __launch_bounds__(256) k_eig_ritz(const double* __restrict__ vin,
                                                  const double* __restrict__ yin,
                                                  const double* __restrict__ zs,
                                                  const double* __restrict__ theta, int r,
                                                  float* __restrict__ vout,
                                                  double* __restrict__ res2,
                                                  double* __restrict__ amv) {
  __shared__ double vsh[kRows][P + 1];
  __shared__ double ysh[kRows][P + 1];
  __shared__ double zsh[P][P + 1];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kRows * P;
  for (int e = tid; e < kRows * P; e += 256) {
    vsh[e / P][e % P] = vin[base + e];
    ysh[e / P][e % P] = yin[base + e];
  }
  for (int e = tid; e < P * P; e += 256) zsh[e / P][e % P] = zs[e];
  __syncthreads();
  const int i = tid >> 2;
  const int64_t row = (int64_t)blockIdx.x * kRows + i;
  double va[P / 4], ra[P / 4];
#pragma unroll
  for (int q = 0; q < P / 4; ++q) {
    const int m = (tid & 3) + 4 * q;
    va[q] = ra[q] = 0.0;
    if (m < r) {
      double a = 0.0, b = 0.0;
      for (int j = 0; j < P; ++j) {
        a = fma(vsh[i][j], zsh[j][m], a);
        b = fma(ysh[i][j], zsh[j][m], b);
      }
      const double res = fma(-theta[m], a, b);
      va[q] = a;
      ra[q] = res * res;
      vout[row * r + m] = (float)a;
    }
  }
  __syncthreads();  // every thread is done reading vsh and ysh
#pragma unroll
  for (int q = 0; q < P / 4; ++q) {
    const int m = (tid & 3) + 4 * q;
    if (m < r) {
      vsh[i][m] = va[q];
      ysh[i][m] = ra[q];
    }
  }
  __syncthreads();
  if (tid < r) {
    double s = 0.0, best = 0.0;
    for (int k = 0; k < kRows; ++k) {
      s += ysh[k][tid];
      if (fabs(vsh[k][tid]) > fabs(best)) best = vsh[k][tid];
    }
    res2[blockIdx.x * r + tid] = s;
    amv[blockIdx.x * r + tid] = best;
  }
}

// Combines the per-block residuals and largest entries (blocks ascending, so
// the first row wins ties), writes eigenvalues (NaN after a breakdown),
// residual norms and each column's sign.
__global__ void k_eig_final(const double* __restrict__ theta, const double* __restrict__ res2,
                            const double* __restrict__ amv, int nb, int r,
                            const double* __restrict__ scal, float* __restrict__ evals,
                            float* __restrict__ resid, double* __restrict__ sgn) {
  const int m = threadIdx.x;
  if (m >= r) return;
  double s = 0.0, best = 0.0;
  for (int b = 0; b < nb; ++b) {
    s += res2[b * r + m];
    if (fabs(amv[b * r + m]) > fabs(best)) best = amv[b * r + m];
  }
  evals[m] = scal[1] != 0.0 ? __builtin_nanf("") : (float)theta[m];
  if (resid) resid[m] = (float)sqrt(s);
  sgn[m] = best < 0.0 ? -1.0 : 1.0;
}

__global__ void __launch_bounds__(256) k_eig_flip(float* __restrict__ v, int64_t n, int r,
                                                  const double* __restrict__ sgn) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n && sgn[e % r] < 0.0) v[e] = -v[e];
}

// ----------------------------------------------------------------- host side

struct EigLayout {
  size_t va, vb, ya, yp, cp, cr, xm, zs, th, scal, fro, res2, amv, sgn, total;
  int slices, nb;
};

// K-slices of the G V product: as many as keep the partial sums' traffic
// (written and read back, float64) within G's own bytes, while the
// slices stay multiples of the 32-wide K chunk and the grid needs no more
// than ~2048 waves.
int eig_slices(int64_t K, int p) {
  int s = 1;
  while ((int64_t)(2 * s) * 4 * p <= K && (K / (2 * s)) % kBK == 0 && K % (2 * s) == 0 &&
         (K / kRows) * (2 * s) * 4 <= 2048)
    s *= 2;
  return s;
}

EigLayout eig_layout(int64_t K, int p, int r) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  EigLayout L;
  L.slices = eig_slices(K, p);
  L.nb = (int)(K / kRows);
  const size_t kp = (size_t)K * p * 8, pp = (size_t)p * p * 8;
  size_t o = 0;
  L.va = o; o += up(kp);
  L.vb = o; o += up(kp);
  L.ya = o; o += up(kp);
  L.yp = o; o += up(kp * L.slices);
  L.cp = o; o += up(pp * L.nb);
  L.cr = o; o += up(pp);
  L.xm = o; o += up(pp);
  L.zs = o; o += up(pp);
  L.th = o; o += up((size_t)p * 8);
  L.scal = o; o += up(8 * 8);
  L.fro = o; o += up((size_t)(K / kFroRows) * 8);
  L.res2 = o; o += up((size_t)L.nb * r * 8);
  L.amv = o; o += up((size_t)L.nb * r * 8);
  L.sgn = o; o += up((size_t)r * 8);
  L.total = o;
  return L;
}

int32_t eig_check(int64_t K, int32_t p, int32_t r, int32_t iters) {
  ASP_TRY(check_k(K));
  if (K > kEigMaxK) return fail(ASP_ERR_SHAPE, "K=%lld above %lld", (long long)K, (long long)kEigMaxK);
  if (p < 16 || p > kEigMaxP || p % 16 != 0)
    return fail(ASP_ERR_SHAPE, "block width p=%d must be 16, 32, 48 or 64", p);
  if (r < 1 || r > p) return fail(ASP_ERR_SHAPE, "r=%d outside [1, p=%d]", r, p);
  if (iters < 0 || iters > 100000) return fail(ASP_ERR_ARG, "iters=%d outside [0, 100000]", iters);
  return ASP_OK;
}

template <int P>
int32_t eig_run(const float* g, int64_t K, const float* v0, int r, int iters, float* vout,
                float* evals, float* resid, uint8_t* ws, const EigLayout& L, hipStream_t st) {
  auto d = [&](size_t off) { return reinterpret_cast<double*>(ws + off); };
  double *va = d(L.va), *vb = d(L.vb), *ya = d(L.ya), *yp = d(L.yp), *cp = d(L.cp),
         *cr = d(L.cr), *xm = d(L.xm), *zs = d(L.zs), *th = d(L.th), *scal = d(L.scal),
         *fro = d(L.fro), *res2 = d(L.res2), *amv = d(L.amv), *sgn = d(L.sgn);
  const int nb = L.nb, Ki = (int)K, slice = Ki / L.slices;
  const dim3 blk(256), rows(nb), gv_grid(nb, L.slices), red_grid(P * P / 64);

  auto chol_apply = [&](const double* yin, double* vo, bool gram) {
    k_eig_reduce<P><<<red_grid, 64, 0, st>>>(cp, nb, cr);
    k_eig_chol<P><<<1, blk, 0, st>>>(cr, xm, scal);
    if (gram)
      k_eig_apply<P, true><<<rows, blk, 0, st>>>(yin, xm, vo, cp);
    else
      k_eig_apply<P, false><<<rows, blk, 0, st>>>(yin, xm, vo, nullptr);
  };

  k_eig_frob<<<dim3(Ki / kFroRows), blk, 0, st>>>(g, Ki, fro);
  k_eig_mu<<<1, 64, 0, st>>>(fro, Ki / kFroRows, scal);
  k_eig_gram<P, kCast><<<rows, blk, 0, st>>>(v0, nullptr, 0, nullptr, scal, Ki, ya, cp);
  chol_apply(ya, va, iters == 0);
  for (int t = 0; t < iters; ++t) {
    k_eig_gv<P><<<gv_grid, blk, 0, st>>>(g, va, yp, Ki, slice);
    k_eig_gram<P, kShift><<<rows, blk, 0, st>>>(nullptr, yp, L.slices, va, scal, Ki, ya, cp);
    chol_apply(ya, va, t == iters - 1);
  }
  chol_apply(va, vb, false);  // second Cholesky QR pass
  k_eig_gv<P><<<gv_grid, blk, 0, st>>>(g, vb, yp, Ki, slice);
  k_eig_gram<P, kCross><<<rows, blk, 0, st>>>(nullptr, yp, L.slices, vb, scal, Ki, ya, cp);
  k_eig_reduce<P><<<red_grid, 64, 0, st>>>(cp, nb, cr);
  k_eig_jacobi<P><<<1, blk, 0, st>>>(cr, th, zs, scal);
  k_eig_ritz<P><<<rows, blk, 0, st>>>(vb, ya, zs, th, r, vout, res2, amv);
  k_eig_final<<<1, 64, 0, st>>>(th, res2, amv, nb, r, scal, evals, resid, sgn);
  const int64_t n = K * r;
  k_eig_flip<<<(unsigned)((n + 255) / 256), blk, 0, st>>>(vout, n, r, sgn);
  return launch_status("top eigenspace");
}

}  // namespace
}  // namespace asp

using namespace asp;

extern "C" {

int32_t asp_top_eigenspace_workspace_bytes(int64_t K, int32_t p, int32_t r, size_t* bytes) {
  clear_error();
  ASP_TRY(eig_check(K, p, r, 0));
  if (!bytes) return fail(ASP_ERR_ARG, "null output pointer");
  *bytes = eig_layout(K, p, r).total;
  return ASP_OK;
}

int32_t asp_top_eigenspace_slices(int64_t K, int32_t p, int32_t* slices) {
  clear_error();
  ASP_TRY(eig_check(K, p, 1, 0));
  if (!slices) return fail(ASP_ERR_ARG, "null output pointer");
  *slices = eig_slices(K, p);
  return ASP_OK;
}

int32_t asp_metric_product_partials(const float* g, int64_t K, const double* v, int32_t p,
                                    double* yp, void* stream) {
  clear_error();
  ASP_TRY(eig_check(K, p, 1, 0));
  ASP_TRY(check_ptr(g, "g", true));
  ASP_TRY(check_ptr(v, "v", true));
  ASP_TRY(check_ptr(yp, "yp", true));
  const int S = eig_slices(K, p), nb = (int)(K / kRows), Ki = (int)K;
  const dim3 grid(nb, S), blk(256);
  const hipStream_t st = (hipStream_t)stream;
  switch (p) {
    case 16: k_eig_gv<16><<<grid, blk, 0, st>>>(g, v, yp, Ki, Ki / S); break;
    case 32: k_eig_gv<32><<<grid, blk, 0, st>>>(g, v, yp, Ki, Ki / S); break;
    case 48: k_eig_gv<48><<<grid, blk, 0, st>>>(g, v, yp, Ki, Ki / S); break;
    default: k_eig_gv<64><<<grid, blk, 0, st>>>(g, v, yp, Ki, Ki / S); break;
  }
  return launch_status("metric product");
}

int32_t asp_top_eigenspace(const float* g, int64_t K, const float* v0, int32_t p, int32_t r,
                           int32_t iters, float* v, float* evals, float* resid, void* workspace,
                           size_t workspace_bytes, void* stream) {
  clear_error();
  ASP_TRY(eig_check(K, p, r, iters));
  ASP_TRY(check_ptr(g, "g", true));
  ASP_TRY(check_ptr(v0, "v0", true));
  ASP_TRY(check_ptr(v, "v", true));
  ASP_TRY(check_ptr(evals, "evals", true));
  ASP_TRY(check_ptr(resid, "resid", false));
  if (!workspace) return fail(ASP_ERR_ARG, "workspace is NULL");
  if (((uintptr_t)workspace & 255u) != 0) return fail(ASP_ERR_ALIGN, "workspace must be 256-byte aligned");
  const EigLayout L = eig_layout(K, p, r);
  if (workspace_bytes < L.total)
    return fail(ASP_ERR_WORKSPACE, "workspace: %zu bytes, need %zu", workspace_bytes, L.total);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  const hipStream_t st = (hipStream_t)stream;
  switch (p) {
    case 16: return eig_run<16>(g, K, v0, r, iters, v, evals, resid, ws, L, st);
    case 32: return eig_run<32>(g, K, v0, r, iters, v, evals, resid, ws, L, st);
    case 48: return eig_run<48>(g, K, v0, r, iters, v, evals, resid, ws, L, st);
    default: return eig_run<64>(g, K, v0, r, iters, v, evals, resid, ws, L, st);
  }
}

}  // extern "C"
