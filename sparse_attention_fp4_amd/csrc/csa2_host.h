// Host-side helpers of the CSA2 library: status reporting and argument checks.
#pragma once
#include <hip/hip_runtime.h>
#include <stdarg.h>
#include <stdio.h>

#include "../../include/csa2.h"

namespace csa2 {

// Records a thread-local detail message and returns the status.
csa2_status_t fail(csa2_status_t s, const char* fmt, ...);

// Checks the launch status of the kernels just enqueued.
csa2_status_t check_launch(const char* what);

inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace csa2

#define CSA2_REQUIRE(cond, status, ...) \
    do { if (!(cond)) return ::csa2::fail((status), __VA_ARGS__); } while (0)
