// Host side of the SVDQuant-style INT4 (group 64) W4A4 arm (model card
// "FastWAM UR3 3-task -- 4-bit quantisations", method table: INT4 with groups
// of 64 for weights and activations, contracted on INT8 tensor cores):
//   - the Gram matrix (W diag(s))^T (W diag(s)) whose top-r eigenvectors are
//     the smoothed weight's top right singular vectors (the rank-r branch);
//   - the weight pack: L1 = W_hat V_r, the residual R = W_hat - L1 V_r^T
//     quantised to INT4 per group of 64 with bfloat16 scales, L1 in bfloat16,
//     and the activation-side constants (1/s and V'' = diag(1/s) V_r, split
//     into bfloat16 high and low parts for the u = x V'' contraction).
// float64 arithmetic; the quantiser's decisions are float32 (amax, the
// bfloat16 scale of amax / 7, the quotient v / scale rounded half to even).
#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "asp.h"
#include "asp_internal.h"

namespace asp {
namespace {

constexpr int kGroup = 64;

uint32_t bits_of(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}
float float_of(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
uint16_t bf16_rne(float f) {
  const uint32_t u = bits_of(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
float bf16_value(uint16_t b) { return float_of((uint32_t)b << 16); }

// float64 -> bfloat16 bits, round to nearest even, directly from the double.
uint16_t bf16_of_double(double v) {
  const uint16_t sign = std::signbit(v) ? 0x8000u : 0u;
  const double a = std::fabs(v);
  if (a == 0.0) return sign;
  int e;
  std::frexp(a, &e);                      // a = f 2^e, f in [0.5, 1)
  const int lead = std::max(e - 1, -126);  // exponent of the leading bit (gradual underflow)
  const double quantum = std::ldexp(1.0, lead - 7);
  const double r = std::nearbyint(a / quantum) * quantum;  // a / quantum is exact
  return (uint16_t)(bits_of((float)r) >> 16) | sign;
}

// One row of float32 values -> INT4 codes (two per byte, element 2j in the low
// nibble, two's complement) and one bfloat16 scale per group of 64.  The
// scales go to scales[g * stride].
void quantize_row(const float* v, int64_t K, uint8_t* codes, uint16_t* scales, int64_t stride) {
  for (int64_t g = 0; g < K / kGroup; ++g) {
    const float* p = v + g * kGroup;
    float amax = 0.0f;
    for (int i = 0; i < kGroup; ++i) amax = std::max(amax, std::fabs(p[i]));
    const uint16_t sb = bf16_rne(amax / 7.0f);
    const float sc = bf16_value(sb);
    scales[g * stride] = sb;
    for (int i = 0; i < kGroup; i += 2) {
      int c[2];
      for (int t = 0; t < 2; ++t) {
        int q = 0;
        if (sc > 0.0f) q = (int)std::nearbyint(p[i + t] / sc);
        c[t] = std::min(7, std::max(-8, q));
      }
      codes[g * (kGroup / 2) + i / 2] = (uint8_t)((c[0] & 15) | ((c[1] & 15) << 4));
    }
  }
}

template <typename F>
void parallel_rows(int64_t n, F&& f) {
  const int64_t nt = std::max<int64_t>(1, std::min<int64_t>(n, std::thread::hardware_concurrency()));
  std::vector<std::thread> pool;
  for (int64_t t = 0; t < nt; ++t)
    pool.emplace_back([&, t] { f(n * t / nt, n * (t + 1) / nt); });
  for (auto& th : pool) th.join();
}

int32_t svdq_check(int64_t N, int64_t K, int32_t r) {
  if (int32_t st = check_k(K)) return st;
  if (int32_t st = check_rank(r)) return st;
  if (N < 1 || N > INT32_MAX) return fail(ASP_ERR_SHAPE, "N=%lld", (long long)N);
  return ASP_OK;
}

}  // namespace
}  // namespace asp

using namespace asp;

extern "C" {

int32_t asp_svdq_packed_sizes(int64_t N, int64_t K, int32_t r, size_t* code_bytes,
                              size_t* scale_bytes, size_t* l1_bytes, size_t* prep_bytes) {
  clear_error();
  if (int32_t st = svdq_check(N, K, r)) return st;
  if (!code_bytes || !scale_bytes || !l1_bytes || !prep_bytes)
    return fail(ASP_ERR_ARG, "null output pointer");
  const PrepPackLayout P = prep_pack_layout(K, r);
  *code_bytes = (size_t)N * K / 2;
  *scale_bytes = (size_t)((N + 127) / 128 * 128) * (K / kGroup) * 2;
  *l1_bytes = (size_t)N * P.rp32 * 2;
  *prep_bytes = P.total;
  return ASP_OK;
}

int32_t asp_svdq_gram(int64_t N, int64_t K, const float* w, const float* s, float* g) {
  clear_error();
  if (int32_t st = svdq_check(N, K, 0)) return st;
  if (!w || !s || !g) return fail(ASP_ERR_ARG, "null host pointer");
  for (int64_t k = 0; k < K; ++k)
    if (!(s[k] > 0.0f) || !std::isfinite(s[k]))
      return fail(ASP_ERR_ARG, "s[%lld] = %g is not a positive finite number", (long long)k, s[k]);
  // W_hat^T, column k of W_hat contiguous
  std::vector<double> wt((size_t)K * N);
  parallel_rows(K, [&](int64_t k0, int64_t k1) {
    for (int64_t k = k0; k < k1; ++k)
      for (int64_t n = 0; n < N; ++n) wt[(size_t)k * N + n] = (double)w[n * K + k] * (double)s[k];
  });
  // rows i of the upper triangle, spread so every thread gets a similar share
  parallel_rows(K, [&](int64_t t0, int64_t t1) {
    for (int64_t t = t0; t < t1; ++t) {
      const int64_t i = (t % 2 == 0) ? t / 2 : K - 1 - t / 2;
      const double* a = &wt[(size_t)i * N];
      for (int64_t j = i; j < K; ++j) {
        const double* b = &wt[(size_t)j * N];
        double acc = 0.0;
        for (int64_t n = 0; n < N; ++n) acc += a[n] * b[n];
        g[i * K + j] = g[j * K + i] = (float)acc;
      }
    }
  });
  return ASP_OK;
}

int32_t asp_svdq_pack_weight(int64_t N, int64_t K, int32_t r, const float* w, const float* s,
                             const float* v, uint8_t* codes, uint16_t* scales, uint16_t* l1,
                             uint8_t* prep) {
  clear_error();
  if (int32_t st = svdq_check(N, K, r)) return st;
  if (!w || !s || !codes || !scales || !prep || (r > 0 && (!v || !l1)))
    return fail(ASP_ERR_ARG, "null host pointer");
  for (int64_t k = 0; k < K; ++k)
    if (!(s[k] > 0.0f) || !std::isfinite(s[k]))
      return fail(ASP_ERR_ARG, "s[%lld] = %g is not a positive finite number", (long long)k, s[k]);
  const PrepPackLayout P = prep_pack_layout(K, r);
  const int64_t N128 = (N + 127) / 128 * 128;  // scale rows are padded with zeros to this
  std::memset(scales, 0, (size_t)N128 * (K / kGroup) * 2);
  // weight side, row by row: L1 = W_hat V, R = W_hat - L1 V^T, INT4 codes of R
  parallel_rows(N, [&](int64_t n0, int64_t n1) {
    std::vector<double> wh(K), low(r > 0 ? r : 1);
    std::vector<float> res(K);
    for (int64_t n = n0; n < n1; ++n) {
      for (int64_t k = 0; k < K; ++k) wh[k] = (double)w[n * K + k] * (double)s[k];
      for (int j = 0; j < r; ++j) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += wh[k] * (double)v[k * r + j];
        low[j] = acc;
      }
      for (int64_t k = 0; k < K; ++k) {
        double t = wh[k];
        for (int j = 0; j < r; ++j) t -= low[j] * (double)v[k * r + j];
        res[k] = (float)t;
      }
      quantize_row(res.data(), K, codes + n * (K / 2), scales + n, N128);
      if (r > 0) {
        for (int j = 0; j < P.rp32; ++j) l1[n * P.rp32 + j] = j < r ? bf16_of_double(low[j]) : 0;
      }
    }
  });
  // activation side: 1/s (float32), V'' = diag(1/s) V transposed, as three bf16 terms
  std::memset(prep, 0, P.total);
  float* cvec = reinterpret_cast<float*>(prep + P.cvec);
  uint16_t* vt[kSplit];
  for (int t = 0; t < kSplit; ++t) vt[t] = reinterpret_cast<uint16_t*>(prep + P.vt[t]);
  uint16_t parts[kSplit];
  for (int64_t k = 0; k < K; ++k) {
    const float rs = (float)(1.0 / (double)s[k]);
    cvec[k] = rs;
    for (int j = 0; j < r; ++j) {
      split_bf16x3((double)v[k * r + j] * (double)rs, parts);
      for (int t = 0; t < kSplit; ++t) vt[t][(int64_t)j * K + k] = parts[t];
    }
  }
  return ASP_OK;
}

}  // extern "C"
