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

}  // namespace asp
