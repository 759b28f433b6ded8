// Per-layer smoothing search (model card "FastWAM UR3 3-task -- 4-bit
// quantisations", section "What ASP is, and what the deflated form means": the
// per-layer (alpha, beta) of the smoothing vector is chosen from a grid of
// candidates by the layer's own deflated-ASP NVFP4 output error on calibration
// activations).
//
// For each candidate the smoothing vector is
//     s_k = max_m |x_mk|^alpha / max_n |W_nk|^beta
// (float64, a zero maximum replaced by 1e-5, then rounded to float32), the
// weight is packed on the host with that s, the layer runs on the device
// (asp_forward, float32 output) and the squared error against the unquantised
// output x W^T + b (a float32 reference GEMM on the device) is summed in a
// fixed order.  The candidate with the smallest mean squared error wins; ties
// go to the earlier one.
#include "asp_device.h"

#include <cmath>
#include <vector>

namespace asp {
namespace {

constexpr int kErrBlocks = 1024;  // partial sums of the squared error (fixed: deterministic)

// Column-wise max |x| over the M rows (threads run along K: coalesced rows).
template <typename XT>
__global__ void __launch_bounds__(256) k_colmax(const XT* __restrict__ x, int M, int K,
                                                float* __restrict__ out) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= K) return;
  float m = 0.0f;
  for (int i = 0; i < M; ++i) {
    float v;
    if constexpr (sizeof(XT) == 2)
      v = bits_f32((uint32_t)x[(int64_t)i * K + k] << 16);
    else
      v = x[(int64_t)i * K + k];
    m = fmaxf(m, fabsf(v));
  }
  out[k] = m;
}

// Reference y = x W^T + b in float32: 64 x 64 output tiles, K in chunks of 16
// through LDS, 4 x 4 outputs per thread, products added in ascending K.
template <typename XT>
__global__ void __launch_bounds__(256) k_ref_gemm(const XT* __restrict__ x,
                                                  const float* __restrict__ w,
                                                  const float* __restrict__ bias, int M, int N,
                                                  int K, float* __restrict__ y) {
  __shared__ float xs[64][17], ws[64][17];
  const int tid = threadIdx.x, tr = tid / 16, tc = tid % 16;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = tid + 256 * j, row = e / 16, col = e % 16;
      const int m = m0 + row, n = n0 + row;
      float xv = 0.0f;
      if (m < M) {
        if constexpr (sizeof(XT) == 2)
          xv = bits_f32((uint32_t)x[(int64_t)m * K + k0 + col] << 16);
        else
          xv = x[(int64_t)m * K + k0 + col];
      }
      xs[row][col] = xv;
      ws[row][col] = n < N ? w[(int64_t)n * K + k0 + col] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = fmaf(xs[tr + 16 * a][kk], ws[tc + 16 * b][kk], acc[a][b]);
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int m = m0 + tr + 16 * a, n = n0 + tc + 16 * b;
      if (m < M && n < N) y[(int64_t)m * N + n] = acc[a][b] + (bias ? bias[n] : 0.0f);
    }
}

// Sum of (a - b)^2 in float64: block b takes elements b*256 + t, b*256 + t +
// kErrBlocks*256, ...; a fixed tree inside the block; then one block adds the
// kErrBlocks partial sums in a fixed tree.
__device__ __forceinline__ double block_sum(double v, double* red) {
  const int t = threadIdx.x;
  red[t] = v;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (t < h) red[t] += red[t + h];
    __syncthreads();
  }
  return red[0];
}

__global__ void __launch_bounds__(256) k_sqerr_partial(const float* __restrict__ a,
                                                       const float* __restrict__ b, int64_t n,
                                                       double* __restrict__ partial) {
  __shared__ double red[256];
  double s = 0.0;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)kErrBlocks * 256) {
    const double d = (double)a[i] - (double)b[i];
    s += d * d;
  }
  const double t = block_sum(s, red);
  if (threadIdx.x == 0) partial[blockIdx.x] = t;
}

__global__ void __launch_bounds__(256) k_sqerr_final(const double* __restrict__ partial,
                                                     double* __restrict__ out) {
  __shared__ double red[256];
  double s = 0.0;
  for (int i = threadIdx.x; i < kErrBlocks; i += 256) s += partial[i];
  const double t = block_sum(s, red);
  if (threadIdx.x == 0) *out = t;
}

size_t up256(size_t b) { return (b + 255) & ~(size_t)255; }

struct SearchLayout {
  size_t w, bias, yref, yq, xmax, codes, scales, wv, prep, fwd, partial, mse, total;
  size_t fwd_bytes, prep_bytes;
};

int32_t search_layout(int64_t M, int64_t N, int64_t K, int32_t r, int32_t n_cand, SearchLayout& L) {
  ASP_TRY(asp_workspace_bytes(M, N, K, r, &L.fwd_bytes));
  ASP_TRY(asp_prep_pack_bytes(K, r, &L.prep_bytes));
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o += up256(bytes);
    return at;
  };
  L.w = take((size_t)N * K * 4);
  L.bias = take((size_t)N * 4);
  L.yref = take((size_t)M * N * 4);
  L.yq = take((size_t)M * N * 4);
  L.xmax = take((size_t)K * 4);
  L.codes = take((size_t)N * K / 2);
  L.scales = take((size_t)N * K / 16);
  L.wv = take((size_t)N * (r > 0 ? r : 1) * 2);
  L.prep = take(L.prep_bytes);
  L.fwd = take(L.fwd_bytes);
  L.partial = take((size_t)kErrBlocks * 8);
  L.mse = take((size_t)n_cand * 8);
  L.total = o;
  return ASP_OK;
}

int32_t hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(ASP_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ASP_OK;
}

}  // namespace
}  // namespace asp

using namespace asp;

extern "C" {

int32_t asp_smoothing_search_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t r,
                                             int32_t n_candidates, size_t* bytes) {
  clear_error();
  ASP_TRY(check_mk(M, K));
  ASP_TRY(check_rank(r));
  if (M < 1 || N < 1 || N > INT32_MAX) return fail(ASP_ERR_SHAPE, "M=%lld N=%lld", (long long)M, (long long)N);
  if (n_candidates < 1) return fail(ASP_ERR_ARG, "n_candidates=%d", n_candidates);
  if (!bytes) return fail(ASP_ERR_ARG, "null output pointer");
  SearchLayout L;
  ASP_TRY(search_layout(M, N, K, r, n_candidates, L));
  *bytes = L.total;
  return ASP_OK;
}

int32_t asp_smoothing_search(const void* x, int32_t x_dtype, int64_t M, int64_t K,
                             const float* w, const float* bias, int64_t N, const float* v,
                             int32_t r, const float* alphas, const float* betas,
                             int32_t n_candidates, double* mse, int32_t* best,
                             void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  ASP_TRY(check_mk(M, K));
  ASP_TRY(check_rank(r));
  if (M < 1 || N < 1 || N > INT32_MAX || M * N > ((int64_t)1 << 40))
    return fail(ASP_ERR_SHAPE, "M=%lld N=%lld", (long long)M, (long long)N);
  if (x_dtype != ASP_F32 && x_dtype != ASP_BF16) return fail(ASP_ERR_ARG, "x_dtype=%d", x_dtype);
  if (n_candidates < 1) return fail(ASP_ERR_ARG, "n_candidates=%d", n_candidates);
  if (!w || !alphas || !betas || !mse || !best || (r > 0 && !v))
    return fail(ASP_ERR_ARG, "null host pointer");
  ASP_TRY(check_ptr(x, "x", true));
  ASP_TRY(check_ptr(workspace, "workspace", true));
  if (((uintptr_t)workspace & 255u) != 0)
    return fail(ASP_ERR_ALIGN, "workspace must be 256-byte aligned");
  SearchLayout L;
  ASP_TRY(search_layout(M, N, K, r, n_candidates, L));
  if (workspace_bytes < L.total)
    return fail(ASP_ERR_WORKSPACE, "workspace %zu bytes, need %zu", workspace_bytes, L.total);
  hipStream_t st = (hipStream_t)stream;
  uint8_t* base = static_cast<uint8_t*>(workspace);
  float* wdev = reinterpret_cast<float*>(base + L.w);
  float* bdev = bias ? reinterpret_cast<float*>(base + L.bias) : nullptr;
  float* yref = reinterpret_cast<float*>(base + L.yref);
  float* yq = reinterpret_cast<float*>(base + L.yq);
  float* xmax_d = reinterpret_cast<float*>(base + L.xmax);
  double* partial = reinterpret_cast<double*>(base + L.partial);
  double* mse_d = reinterpret_cast<double*>(base + L.mse);
  const int Mi = (int)M, Ni = (int)N, Ki = (int)K;

  // the unquantised reference and the activation channel maxima, once
  ASP_TRY(hip_ok(hipMemcpyAsync(wdev, w, (size_t)N * K * 4, hipMemcpyHostToDevice, st), "copy W"));
  if (bias)
    ASP_TRY(hip_ok(hipMemcpyAsync(bdev, bias, (size_t)N * 4, hipMemcpyHostToDevice, st), "copy bias"));
  const dim3 gref((unsigned)((N + 63) / 64), (unsigned)((M + 63) / 64));
  if (x_dtype == ASP_BF16) {
    hipLaunchKernelGGL(k_colmax<uint16_t>, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), Mi, Ki, xmax_d);
    hipLaunchKernelGGL(k_ref_gemm<uint16_t>, gref, dim3(256), 0, st,
                       static_cast<const uint16_t*>(x), wdev, bdev, Mi, Ni, Ki, yref);
  } else {
    hipLaunchKernelGGL(k_colmax<float>, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st,
                       static_cast<const float*>(x), Mi, Ki, xmax_d);
    hipLaunchKernelGGL(k_ref_gemm<float>, gref, dim3(256), 0, st, static_cast<const float*>(x),
                       wdev, bdev, Mi, Ni, Ki, yref);
  }
  ASP_TRY(launch_status("search reference"));
  std::vector<float> xmax(K);
  ASP_TRY(hip_ok(hipMemcpyAsync(xmax.data(), xmax_d, (size_t)K * 4, hipMemcpyDeviceToHost, st), "copy maxima"));
  ASP_TRY(hip_ok(hipStreamSynchronize(st), "synchronize"));
  std::vector<double> wmax(K, 0.0);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) wmax[k] = std::max(wmax[k], std::fabs((double)w[n * K + k]));

  std::vector<float> s(K);
  std::vector<uint8_t> codes((size_t)N * K / 2), scales((size_t)N * K / 16), prep(L.prep_bytes);
  std::vector<uint16_t> wv((size_t)N * (r > 0 ? r : 1));
  for (int32_t c = 0; c < n_candidates; ++c) {
    const double a = alphas[c], b = betas[c];
    for (int64_t k = 0; k < K; ++k) {
      const double xm = xmax[k] > 0.0f ? (double)xmax[k] : 1e-5;
      const double wm = wmax[k] > 0.0 ? wmax[k] : 1e-5;
      s[k] = (float)(std::pow(xm, a) / std::pow(wm, b));
    }
    ASP_TRY(asp_pack_weight(N, K, r, w, s.data(), v, codes.data(), scales.data(),
                            r > 0 ? wv.data() : nullptr, nullptr, 0));
    ASP_TRY(asp_pack_prep(K, r, s.data(), v, prep.data()));
    ASP_TRY(hip_ok(hipMemcpyAsync(base + L.codes, codes.data(), codes.size(), hipMemcpyHostToDevice, st), "copy codes"));
    ASP_TRY(hip_ok(hipMemcpyAsync(base + L.scales, scales.data(), scales.size(), hipMemcpyHostToDevice, st), "copy scales"));
    if (r > 0)
      ASP_TRY(hip_ok(hipMemcpyAsync(base + L.wv, wv.data(), (size_t)N * r * 2, hipMemcpyHostToDevice, st), "copy wv"));
    ASP_TRY(hip_ok(hipMemcpyAsync(base + L.prep, prep.data(), prep.size(), hipMemcpyHostToDevice, st), "copy prep"));
    ASP_TRY(asp_forward(x, x_dtype, M, N, K, r, base + L.prep, base + L.codes, base + L.scales,
                        r > 0 ? reinterpret_cast<const uint16_t*>(base + L.wv) : nullptr, bdev,
                        yq, ASP_F32, base + L.fwd, L.fwd_bytes, stream));
    hipLaunchKernelGGL(k_sqerr_partial, dim3(kErrBlocks), dim3(256), 0, st, yq, yref, M * N, partial);
    hipLaunchKernelGGL(k_sqerr_final, dim3(1), dim3(256), 0, st, partial, mse_d + c);
    ASP_TRY(launch_status("search error"));
    // the host buffers are refilled for the next candidate
    ASP_TRY(hip_ok(hipStreamSynchronize(st), "synchronize"));
  }
  std::vector<double> sums(n_candidates);
  ASP_TRY(hip_ok(hipMemcpyAsync(sums.data(), mse_d, (size_t)n_candidates * 8, hipMemcpyDeviceToHost, st), "copy errors"));
  ASP_TRY(hip_ok(hipStreamSynchronize(st), "synchronize"));
  int32_t arg = 0;
  for (int32_t c = 0; c < n_candidates; ++c) {
    mse[c] = sums[c] / ((double)M * (double)N);
    if (mse[c] < mse[arg]) arg = c;
  }
  *best = arg;
  return ASP_OK;
}

}  // extern "C"
