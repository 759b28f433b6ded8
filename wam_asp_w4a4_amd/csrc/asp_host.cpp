// Host half of libasp: status/error plumbing, size queries, the NVFP4
// quantiser on the CPU and the float64 weight packer.
//
// Weight side of the deflated contract (model card "FastWAM UR3 3-task --
// 4-bit quantisations", section "What ASP is, and what the deflated form
// means"): the 4-bit weight holds W_tilde (I - V V^T) and the low-rank branch
// the exact W_tilde V, kept in bf16.  W_tilde = W diag(s) H includes the
// block Hadamard so that it meets the rotated activation (x / s) H.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <string>
#include <thread>
#include <vector>

#include "asp.h"
#include "asp_internal.h"
#include "nvfp4_codec.h"

namespace asp {

static thread_local std::string g_last_error;

int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(asp_status_string(status)) + ": " + buf;
  return status;
}

void clear_error() { g_last_error.clear(); }

int32_t check_k(int64_t K) {
  if (K <= 0 || K % ASP_HADAMARD_BLOCK != 0)
    return fail(ASP_ERR_SHAPE, "K=%lld must be a positive multiple of %d", (long long)K,
                ASP_HADAMARD_BLOCK);
  return ASP_OK;
}

int32_t check_rank(int32_t r) {
  if (r < 0 || r > ASP_MAX_RANK)
    return fail(ASP_ERR_SHAPE, "rank r=%d outside [0, %d]", r, ASP_MAX_RANK);
  return ASP_OK;
}

// ---------------------------------------------------------------------------
// NVFP4 quantisation of one float32 row on the host.
static void quantize_row(const float* in, int64_t cols, uint8_t* codes, uint8_t* scales) {
  for (int64_t b = 0; b < cols / 16; ++b) {
    const float* v = in + 16 * b;
    float amax = 0.0f;
    for (int i = 0; i < 16; ++i) amax = std::max(amax, fabsf(v[i]));
    uint32_t sc = block_scale_code(amax);
    float sd = e4m3_decode(sc);
    scales[b] = (uint8_t)sc;
    for (int i = 0; i < 16; i += 2) {
      uint32_t lo = e2m1_code(v[i], sd), hi = e2m1_code(v[i + 1], sd);
      codes[8 * b + i / 2] = (uint8_t)(lo | (hi << 4));
    }
  }
}

// float64 -> bfloat16 bits, round to nearest even (no overflow handling: the
// low-rank factor is far inside the bf16 range).
static uint16_t bf16_from_double(double v) {
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  double a = fabs(v);
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);                      // a = f * 2^e, f in [0.5, 1)
  int lead = std::max(e - 1, -126);  // exponent of the leading bit (gradual underflow)
  double quantum = ldexp(1.0, lead - 7);
  double r = nearbyint(a / quantum) * quantum;  // a / quantum is exact
  return (uint16_t)(f32_bits((float)r) >> 16) | sign;
}

static double bf16_value(uint16_t b) { return (double)bits_f32((uint32_t)b << 16); }

// v as the sum of three bf16 numbers, each the RNE bf16 rounding of what the
// earlier ones leave (computed in float64, where every difference is exact
// for the magnitudes met here): about 26 significant bits, and every float32
// value exactly.
void split_bf16x3(double v, uint16_t (&out)[kSplit]) {
  double rest = v;
  for (int t = 0; t < kSplit; ++t) {
    out[t] = bf16_from_double(rest);
    rest -= bf16_value(out[t]);
  }
}

// In-place Sylvester-ordered Walsh-Hadamard transform of 128 doubles,
// scaled by 1/sqrt(128).
static void fwht128(double* a) {
  for (int h = 1; h < 128; h <<= 1)
    for (int i = 0; i < 128; i += 2 * h)
      for (int j = i; j < i + h; ++j) {
        double x = a[j], y = a[j + h];
        a[j] = x + y;
        a[j + h] = x - y;
      }
  const double inv = 1.0 / sqrt(128.0);
  for (int i = 0; i < 128; ++i) a[i] *= inv;
}

struct PackJob {
  int64_t N, K;
  int32_t r;
  const float *w, *s, *v;
  uint8_t *codes, *scales;
  uint16_t* wv;
  float* pre;
  bool shared;  // the shared-weight arm: W_tilde itself is quantised, L = DQ(W_q) V
};

static void pack_rows(const PackJob& j, int64_t row0, int64_t row1) {
  const int64_t K = j.K;
  const int r = j.r;
  std::vector<double> t(K), low(r > 0 ? r : 1);
  std::vector<float> d32(K);
  for (int64_t n = row0; n < row1; ++n) {
    const float* wr = j.w + n * K;
    for (int64_t k = 0; k < K; ++k) t[k] = (double)wr[k] * (double)j.s[k];
    for (int64_t b = 0; b < K; b += 128) fwht128(&t[b]);
    uint8_t* crow = j.codes + n * (K / 2);
    uint8_t* srow = j.scales + n * (K / 16);
    for (int c = 0; c < r; ++c) low[c] = 0.0;
    if (!j.shared) {
      for (int64_t k = 0; k < K; ++k)
        for (int c = 0; c < r; ++c) low[c] += t[k] * (double)j.v[k * r + c];
      for (int64_t k = 0; k < K; ++k) {
        double d = t[k];
        double proj = 0.0;
        for (int c = 0; c < r; ++c) proj += low[c] * (double)j.v[k * r + c];
        d32[k] = (float)(d - proj);
      }
      quantize_row(d32.data(), K, crow, srow);
    } else {
      // one weight: W_tilde itself; the low-rank factor is that quantised
      // weight (decoded exactly) times V
      for (int64_t k = 0; k < K; ++k) d32[k] = (float)t[k];
      quantize_row(d32.data(), K, crow, srow);
      for (int64_t k = 0; k < K; ++k) {
        const uint32_t code = (crow[k >> 1] >> (4 * (k & 1))) & 0xFu;
        const double dq = (double)e2m1_decode(code) * (double)e4m3_decode(srow[k >> 4]);
        for (int c = 0; c < r; ++c) low[c] += dq * (double)j.v[k * r + c];
      }
    }
    for (int c = 0; c < r; ++c) j.wv[n * r + c] = bf16_from_double(low[c]);
    if (j.pre) memcpy(j.pre + n * K, d32.data(), K * sizeof(float));
  }
}

}  // namespace asp

using namespace asp;

extern "C" {

int32_t asp_abi_version(void) { return 8; }

#ifndef ASP_SOURCE_DIGEST
#define ASP_SOURCE_DIGEST "unknown"
#endif
const char* asp_source_digest(void) { return ASP_SOURCE_DIGEST; }

const char* asp_status_string(int32_t status) {
  switch (status) {
    case ASP_OK: return "ASP_OK";
    case ASP_ERR_ARG: return "ASP_ERR_ARG";
    case ASP_ERR_SHAPE: return "ASP_ERR_SHAPE";
    case ASP_ERR_ALIGN: return "ASP_ERR_ALIGN";
    case ASP_ERR_UNSUPPORTED: return "ASP_ERR_UNSUPPORTED";
    case ASP_ERR_WORKSPACE: return "ASP_ERR_WORKSPACE";
    case ASP_ERR_HIP: return "ASP_ERR_HIP";
    case ASP_ERR_INTERNAL: return "ASP_ERR_INTERNAL";
    default: return "ASP_ERR_UNKNOWN";
  }
}

const char* asp_last_error(void) { return g_last_error.c_str(); }

int32_t asp_packed_sizes(int64_t N, int64_t K, int32_t r, size_t* code_bytes,
                         size_t* scale_bytes, size_t* wv_bytes) {
  clear_error();
  if (int32_t st = check_k(K)) return st;
  if (int32_t st = check_rank(r)) return st;
  if (N < 1) return fail(ASP_ERR_SHAPE, "N=%lld must be >= 1", (long long)N);
  if (!code_bytes || !scale_bytes || !wv_bytes)
    return fail(ASP_ERR_ARG, "null output pointer");
  *code_bytes = (size_t)N * (size_t)K / 2;
  *scale_bytes = (size_t)N * (size_t)K / 16;
  *wv_bytes = (size_t)N * (size_t)r * 2;
  return ASP_OK;
}

int32_t asp_prep_pack_bytes(int64_t K, int32_t r, size_t* bytes) {
  clear_error();
  if (int32_t st = check_k(K)) return st;
  if (int32_t st = check_rank(r)) return st;
  if (!bytes) return fail(ASP_ERR_ARG, "null output pointer");
  *bytes = prep_pack_layout(K, r).total;
  return ASP_OK;
}

int32_t asp_pack_prep(int64_t K, int32_t r, const float* s, const float* v, uint8_t* prep_pack) {
  clear_error();
  if (int32_t st = check_k(K)) return st;
  if (int32_t st = check_rank(r)) return st;
  if (!s || !prep_pack) return fail(ASP_ERR_ARG, "null pointer");
  if (r > 0 && !v) return fail(ASP_ERR_ARG, "r=%d needs v", r);
  for (int64_t k = 0; k < K; ++k)
    if (!(s[k] > 0.0f) || !isfinite(s[k]))
      return fail(ASP_ERR_ARG, "s[%lld]=%g must be finite and > 0", (long long)k, (double)s[k]);
  const PrepPackLayout L = prep_pack_layout(K, r);
  memset(prep_pack, 0, L.total);
  double* cvec = reinterpret_cast<double*>(prep_pack + L.cvec64);
  uint16_t* vt[kSplit];
  uint16_t* vs[kSplit];
  for (int t = 0; t < kSplit; ++t) {
    vt[t] = reinterpret_cast<uint16_t*>(prep_pack + L.vt[t]);
    vs[t] = reinterpret_cast<uint16_t*>(prep_pack + L.v[t]);
  }
  const double root = sqrt(128.0);
  for (int64_t k = 0; k < K; ++k) cvec[k] = 1.0 / ((double)s[k] * root);
  std::vector<double> col(K);
  uint16_t parts[kSplit];
  for (int c = 0; c < r; ++c) {
    // V'' = diag(1/s) H V, one column at a time
    for (int64_t k = 0; k < K; ++k) col[k] = (double)v[k * r + c];
    for (int64_t b = 0; b < K; b += 128) fwht128(&col[b]);
    for (int64_t k = 0; k < K; ++k) {
      split_bf16x3(col[k] / (double)s[k], parts);
      for (int t = 0; t < kSplit; ++t) vt[t][(int64_t)c * K + k] = parts[t];
      split_bf16x3((double)v[k * r + c], parts);
      for (int t = 0; t < kSplit; ++t) vs[t][k * L.rp32 + c] = parts[t];
    }
  }
  return ASP_OK;
}

int32_t asp_quantize_nvfp4_host(const float* in, int64_t rows, int64_t cols,
                                uint8_t* codes, uint8_t* scales) {
  clear_error();
  if (rows < 0 || cols <= 0 || cols % 16)
    return fail(ASP_ERR_SHAPE, "rows=%lld cols=%lld: need rows >= 0, cols a positive multiple of 16",
                (long long)rows, (long long)cols);
  if (rows == 0) return ASP_OK;
  if (!in || !codes || !scales) return fail(ASP_ERR_ARG, "null pointer");
  for (int64_t i = 0; i < rows; ++i)
    quantize_row(in + i * cols, cols, codes + i * (cols / 2), scales + i * (cols / 16));
  return ASP_OK;
}

static int32_t pack_weight_impl(bool shared, int64_t N, int64_t K, int32_t r, const float* w,
                                const float* s, const float* v, uint8_t* w_codes,
                                uint8_t* w_scales, uint16_t* wv, float* w_prequant,
                                int32_t n_threads) {
  clear_error();
  if (int32_t st = check_k(K)) return st;
  if (int32_t st = check_rank(r)) return st;
  if (N < 1) return fail(ASP_ERR_SHAPE, "N=%lld must be >= 1", (long long)N);
  if (!w || !s || !w_codes || !w_scales) return fail(ASP_ERR_ARG, "null pointer");
  if (r > 0 && (!v || !wv)) return fail(ASP_ERR_ARG, "r=%d needs v and wv", r);
  for (int64_t k = 0; k < K; ++k)
    if (!(s[k] > 0.0f) || !isfinite(s[k]))
      return fail(ASP_ERR_ARG, "s[%lld]=%g must be finite and > 0", (long long)k, (double)s[k]);
  PackJob job{N, K, r, w, s, v, w_codes, w_scales, wv, w_prequant, shared};
  int64_t nt = n_threads > 0 ? n_threads : (int64_t)std::thread::hardware_concurrency();
  nt = std::max<int64_t>(1, std::min<int64_t>(nt, N));
  if (nt == 1) {
    pack_rows(job, 0, N);
    return ASP_OK;
  }
  std::vector<std::thread> pool;
  int64_t per = (N + nt - 1) / nt;
  for (int64_t t = 0; t < nt; ++t) {
    int64_t a = t * per, b = std::min(N, a + per);
    if (a >= b) break;
    pool.emplace_back(pack_rows, std::cref(job), a, b);
  }
  for (auto& th : pool) th.join();
  return ASP_OK;
}

int32_t asp_pack_weight(int64_t N, int64_t K, int32_t r, const float* w, const float* s,
                        const float* v, uint8_t* w_codes, uint8_t* w_scales, uint16_t* wv,
                        float* w_prequant, int32_t n_threads) {
  return pack_weight_impl(false, N, K, r, w, s, v, w_codes, w_scales, wv, w_prequant, n_threads);
}

int32_t asp_pack_weight_shared(int64_t N, int64_t K, int32_t r, const float* w, const float* s,
                               const float* v, uint8_t* w_codes, uint8_t* w_scales,
                               uint16_t* wv, float* w_prequant, int32_t n_threads) {
  return pack_weight_impl(true, N, K, r, w, s, v, w_codes, w_scales, wv, w_prequant, n_threads);
}

}  // extern "C"
