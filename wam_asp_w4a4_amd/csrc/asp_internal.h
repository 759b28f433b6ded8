// Internal helpers shared by the host translation unit and the HIP kernels:
// thread-local error reporting and argument validation.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "asp.h"

namespace asp {

// Record a failure for asp_last_error() and return its status.
int32_t fail(int32_t status, const char* fmt, ...)
#if defined(__GNUC__)
    __attribute__((format(printf, 2, 3)))
#endif
    ;

// Clear the thread's last error (called at the start of every entry point).
void clear_error();

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Shared shape checks; return ASP_OK or a recorded failure.
int32_t check_k(int64_t K);
int32_t check_rank(int32_t r);

// Byte layout of a layer's prep constants (written by asp_pack_prep on the
// host, read by the activation-prep kernels).  Each section starts on a
// 256-byte boundary.
//   cvec      K float32          the SVDQuant-style arm's 1 / s_k (unused by
//                                the NVFP4 arm)
//   cvec64    K float64          1 / (s_k * sqrt(128)), the NVFP4 arm's
//                                smoothing and Hadamard normalisation
//   vt[0..2]  rp32 x K bf16      V'' = diag(1/s) H V, transposed, as three
//                                bf16 terms (hi, mid, lo: each the bf16
//                                rounding of what the earlier terms leave)
//   v[0..2]   K x rp32 bf16      V as three bf16 terms (exact for float32 V)
// with rp32 = r rounded up to 32 and the padding zero.  Three bf16 terms hold
// 24 or more significant bits, so products on bf16 MFMA reach float32
// accuracy when every cross term of combined order <= 2 is formed.
constexpr int kSplit = 3;

struct PrepPackLayout {
  size_t cvec, cvec64, vt[kSplit], v[kSplit], total;
  size_t plane_bytes;  // distance between consecutive term planes (V'' and V alike)
  int rp16, rp32;
};

inline PrepPackLayout prep_pack_layout(int64_t K, int32_t r) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  PrepPackLayout L;
  L.rp16 = (r + 15) / 16 * 16;
  L.rp32 = (r + 31) / 32 * 32;
  L.cvec = 0;
  L.cvec64 = up((size_t)K * 4);
  size_t at = L.cvec64 + up((size_t)K * 8);
  L.plane_bytes = up((size_t)L.rp32 * K * 2);  // rp32 x K and K x rp32 planes alike
  for (int t = 0; t < kSplit; ++t) {
    L.vt[t] = at;
    at += L.plane_bytes;
  }
  for (int t = 0; t < kSplit; ++t) {
    L.v[t] = at;
    at += L.plane_bytes;
  }
  L.total = at;
  return L;
}

// v as three bf16 terms (host side of the prep and SVDQuant-style packers).
void split_bf16x3(double v, uint16_t (&out)[kSplit]);

}  // namespace asp
