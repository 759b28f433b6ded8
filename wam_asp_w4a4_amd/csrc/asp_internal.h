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
//   cvec   K float32          1 / (s_k * sqrt(128))
//   vt_hi  rp32 x K bf16      V'' = diag(1/s) H V, transposed, high part
//   vt_lo  rp32 x K bf16      V'' low part (V'' - hi, rounded to bf16)
//   v_hi   K x rp32 bf16      V, high part
//   v_lo   K x rp32 bf16      V, low part
// with rp32 = r rounded up to 32 and the padding zero.
struct PrepPackLayout {
  size_t cvec, vt_hi, vt_lo, v_hi, v_lo, total;
  int rp16, rp32;
};

inline PrepPackLayout prep_pack_layout(int64_t K, int32_t r) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  PrepPackLayout L;
  L.rp16 = (r + 15) / 16 * 16;
  L.rp32 = (r + 31) / 32 * 32;
  L.cvec = 0;
  L.vt_hi = up((size_t)K * 4);
  L.vt_lo = L.vt_hi + up((size_t)L.rp32 * K * 2);
  L.v_hi = L.vt_lo + up((size_t)L.rp32 * K * 2);
  L.v_lo = L.v_hi + up((size_t)K * L.rp32 * 2);
  L.total = L.v_lo + up((size_t)K * L.rp32 * 2);
  return L;
}

}  // namespace asp
