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

// Partial Gram sums of one 64-row block: part[a][b] = sum_rows L[row][a] R[row][b],
// rows in ascending order (L = R gives an exactly symmetric result).
template <int P>
__device__ __forceinline__ void block_gram(const double (*L)[P + 1], const double (*R)[P + 1],
                                           double* __restrict__ part) {
  for (int e = threadIdx.x; e < P * P; e += 256) {
    const int a = e / P, b = e % P;
    double s = 0.0;
#pragma unroll 8
    for (int i = 0; i < kRows; ++i) s = fma(L[i][a], R[i][b], s);
    part[e] = s;
  }
}

enum GramMode { kCast = 0, kShift = 1, kCross = 2 };

// Forms one 64-row block of Y and its Gram partial:
//   kCast : Y = float64(v0)                      part = Y^T Y
//   kShift: Y = sum_s yp[s] + mu V               part = Y^T Y
//   kCross: Y = sum_s yp[s]                      part = V^T Y
// slices are added in ascending order.
template <int P, int MODE>
__global__ void __launch_bounds__(256) k_eig_gram(const float* __restrict__ v0,
                                                  const double* __restrict__ yp, int nslices,
                                                  const double* __restrict__ v,
                                                  const double* __restrict__ scal, int K,
                                                  double* __restrict__ y, double* __restrict__ cp) {
  __shared__ double ys[kRows][P + 1];
  __shared__ double vsh[MODE == kCross ? kRows : 1][P + 1];
  const int64_t base = (int64_t)blockIdx.x * kRows * P;
  const double mu = MODE == kShift ? scal[0] : 0.0;
  for (int e = threadIdx.x; e < kRows * P; e += 256) {
    const int i = e / P, c = e % P;
    double val;
    if constexpr (MODE == kCast) {
      val = (double)v0[base + e];
    } else {
      val = 0.0;
      for (int s = 0; s < nslices; ++s) val += yp[(int64_t)s * K * P + base + e];
      if constexpr (MODE == kShift) val = fma(mu, v[base + e], val);
      if constexpr (MODE == kCross) vsh[i][c] = v[base + e];
    }
    ys[i][c] = val;
    y[base + e] = val;
  }
  __syncthreads();
  block_gram<P>(MODE == kCross ? vsh : ys, ys, cp + (int64_t)blockIdx.x * P * P);
}

// c[e] = sum over blocks b (ascending) of cp[b][e].
template <int P>
__global__ void __launch_bounds__(256) k_eig_reduce(const double* __restrict__ cp, int nb,
                                                    double* __restrict__ c) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= P * P) return;
  double s = 0.0;
  for (int b = 0; b < nb; ++b) s += cp[(int64_t)b * P * P + e];
  c[e] = s;
}

// vout = Y X^T for one 64-row block (X lower triangular, so column j of the
// output mixes Y's columns 0..j); with GRAM, also the Gram partial of vout.
template <int P, bool GRAM>
__global__ void __launch_bounds__(256) k_eig_apply(const double* __restrict__ yin,
                                                   const double* __restrict__ xm,
                                                   double* __restrict__ vout,
                                                   double* __restrict__ cp) {
  __shared__ double ys[kRows][P + 1];
  __shared__ double xs[P][P + 1];
  const int tid = threadIdx.x;
  const int64_t base = (int64_t)blockIdx.x * kRows * P;
  for (int e = tid; e < kRows * P; e += 256) ys[e / P][e % P] = yin[base + e];
  for (int e = tid; e < P * P; e += 256) xs[e / P][e % P] = xm[e];
  __syncthreads();
  const int i = tid >> 2;
  double o[P / 4];
#pragma unroll
  for (int m = 0; m < P / 4; ++m) {
    const int j = (tid & 3) + 4 * m;
    double s = 0.0;
    for (int k = 0; k <= j; ++k) s = fma(ys[i][k], xs[j][k], s);
    o[m] = s;
    vout[base + (int64_t)i * P + j] = s;
  }
  if constexpr (GRAM) {
    __syncthreads();  // every thread is done reading ys
#pragma unroll
    for (int m = 0; m < P / 4; ++m) ys[i][(tid & 3) + 4 * m] = o[m];
    __syncthreads();
    block_gram<P>(ys, ys, cp + (int64_t)blockIdx.x * P * P);
  }
}

// --------------------------------------------------------- one-workgroup steps

// Cholesky C = L L^T (right-looking, in LDS) and X = L^-1 (column c solved by
// thread c, forward substitution).  A pivot that is not a positive finite
// number is replaced by 1 and recorded in scal[1].
template <int P>
__global__ void __launch_bounds__(256) k_eig_chol(const double* __restrict__ cin,
                                                  double* __restrict__ xm,
                                                  double* __restrict__ scal) {
  __shared__ double C[P][P + 1];
  __shared__ double X[P][P + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e < P * P; e += 256) C[e / P][e % P] = cin[e];
  __syncthreads();
  bool bad_any = false;
  for (int j = 0; j < P; ++j) {
    double d = C[j][j];
    const bool bad = !(d > 0.0) || __builtin_isinf(d);
    if (bad) d = 1.0;
    bad_any |= bad;
    const double piv = sqrt(d), inv = 1.0 / piv;
    for (int i = j + 1 + tid; i < P; i += 256) C[i][j] *= inv;
    __syncthreads();
    if (tid == 0) C[j][j] = piv;
    const int m = P - 1 - j;
    for (int e = tid; e < m * m; e += 256) {
      const int i = j + 1 + e / m, k = j + 1 + e % m;
      if (k <= i) C[i][k] = fma(-C[i][j], C[k][j], C[i][k]);
    }
    __syncthreads();
  }
  if (tid < P) {
    const int c = tid;
    for (int i = 0; i < c; ++i) X[i][c] = 0.0;
    X[c][c] = 1.0 / C[c][c];
    for (int i = c + 1; i < P; ++i) {
      double s = 0.0;
      for (int k = c; k < i; ++k) s = fma(C[i][k], X[k][c], s);
      X[i][c] = -s / C[i][i];
    }
  }
  __syncthreads();
  for (int e = tid; e < P * P; e += 256) xm[e] = X[e / P][e % P];
  if (tid == 0 && bad_any) scal[1] = 1.0;
}

// mu = 2^-16 sqrt(sum of the Frobenius partials) (1 when that is 0); clears
// the breakdown flag.
__global__ void k_eig_mu(const double* __restrict__ fro, int nb, double* __restrict__ scal) {
  if (threadIdx.x != 0) return;
  double s = 0.0;
  for (int b = 0; b < nb; ++b) s += fro[b];
  const double mu = ldexp(sqrt(s), -16);
  scal[0] = mu > 0.0 ? mu : 1.0;
  scal[1] = 0.0;
}

// Sum of squares of 64 rows of G (float64, fixed-order tree in LDS).
__global__ void __launch_bounds__(256) k_eig_frob(const float* __restrict__ g, int K,
                                                  double* __restrict__ fro) {
  __shared__ double red[256];
  const f32x4_t* src = reinterpret_cast<const f32x4_t*>(g + (int64_t)blockIdx.x * kRows * K);
  const int n4 = kRows * K / 4;
  double s = 0.0;
  for (int e = threadIdx.x; e < n4; e += 256) {
    const f32x4_t q = src[e];
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
// at once (one thread computes each pair's rotation; all threads apply the
// row and then the column updates).  Sweeps stop when the off-diagonal
// Frobenius norm falls to 1e-15 of the whole, or after 40.  Outputs the
// eigenvalues largest first (equal ones in index order) and the matching
// eigenvector columns zs[:, m].
template <int P>
__global__ void __launch_bounds__(256) k_eig_jacobi(const double* __restrict__ cin,
                                                    double* __restrict__ theta,
                                                    double* __restrict__ zs,
                                                    double* __restrict__ scal) {
  __shared__ double T[P][P + 1];
  __shared__ double Z[P][P + 1];
  __shared__ double cs[P / 2][2];
  __shared__ int pq[P / 2][2];
  __shared__ double red[256][2];
  __shared__ int perm[P];
  const int tid = threadIdx.x;
  for (int e = tid; e < P * P; e += 256) {
    const int a = e / P, b = e % P;
    T[a][b] = 0.5 * (cin[a * P + b] + cin[b * P + a]);
    Z[a][b] = a == b ? 1.0 : 0.0;
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
    const bool done = !(red[0][0] > 1e-30 * red[0][1]);
    __syncthreads();  // everyone has read red before it is reused
    if (done) break;
    for (int rnd = 0; rnd < P - 1; ++rnd) {
      if (tid < P / 2) {
        auto player = [&](int pos) { return pos == 0 ? 0 : 1 + (pos - 1 + rnd) % (P - 1); };
        int a = player(tid), b = player(P - 1 - tid);
        if (a > b) { const int t = a; a = b; b = t; }
        const double app = T[a][a], aqq = T[b][b], apq = T[a][b];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double tau = (aqq - app) / (2.0 * apq);
          // the smaller root of t^2 + 2 tau t - 1 = 0; 1 / (2 tau) once tau^2 would overflow
          const double t = fabs(tau) > 1e150 ? 0.5 / tau
                                             : (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        cs[tid][0] = c;
        cs[tid][1] = s;
        pq[tid][0] = a;
        pq[tid][1] = b;
      }
      __syncthreads();
      for (int e = tid; e < (P / 2) * P; e += 256) {  // rows a and b of T
        const int i = e / P, k = e % P, a = pq[i][0], b = pq[i][1];
        const double c = cs[i][0], s = cs[i][1];
        const double ta = T[a][k], tb = T[b][k];
        T[a][k] = c * ta - s * tb;
        T[b][k] = s * ta + c * tb;
      }
      __syncthreads();
      for (int e = tid; e < (P / 2) * P; e += 256) {  // columns a and b of T and Z
        const int i = e / P, k = e % P, a = pq[i][0], b = pq[i][1];
        const double c = cs[i][0], s = cs[i][1];
        const double ta = T[k][a], tb = T[k][b];
        T[k][a] = c * ta - s * tb;
        T[k][b] = s * ta + c * tb;
        if (k == a) T[a][b] = 0.0;
        if (k == b) T[b][a] = 0.0;
        const double za = Z[k][a], zb = Z[k][b];
        Z[k][a] = c * za - s * zb;
        Z[k][b] = s * za + c * zb;
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
  L.fro = o; o += up((size_t)L.nb * 8);
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
  const dim3 blk(256), rows(nb), gv_grid(nb, L.slices), red_grid((P * P + 255) / 256);

  auto chol_apply = [&](const double* yin, double* vo, bool gram) {
    k_eig_reduce<P><<<red_grid, blk, 0, st>>>(cp, nb, cr);
    k_eig_chol<P><<<1, blk, 0, st>>>(cr, xm, scal);
    if (gram)
      k_eig_apply<P, true><<<rows, blk, 0, st>>>(yin, xm, vo, cp);
    else
      k_eig_apply<P, false><<<rows, blk, 0, st>>>(yin, xm, vo, nullptr);
  };

  k_eig_frob<<<rows, blk, 0, st>>>(g, Ki, fro);
  k_eig_mu<<<1, 64, 0, st>>>(fro, nb, scal);
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
  k_eig_reduce<P><<<red_grid, blk, 0, st>>>(cp, nb, cr);
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
