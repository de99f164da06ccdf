// sconv_host.h -- host-side helpers of the libsconv C ABI: error reporting,
// argument checks and launch-error capture.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sconv.h"

namespace sconv {

// Record a formatted message for sconv_last_error() and return `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// After a launch: map a HIP launch error to SCONV_ERR_HIP.
int check_launch(const char* what);

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
// p is a multiple of `bytes` (a power of two).
inline bool aligned_to(const void* p, int64_t bytes) {
  return ((uintptr_t)p & (uintptr_t)(bytes - 1)) == 0;
}

inline int64_t elem_size(int32_t dtype) { return dtype == SCONV_F32 ? 4 : 2; }

inline bool valid_dtype(int32_t d) { return d == SCONV_F32 || d == SCONV_BF16; }
inline bool valid_act(int32_t a) { return a == SCONV_ACT_NONE || a == SCONV_ACT_SILU; }

// Byte ranges [a, a+na) and [b, b+nb) intersect.
inline bool overlap(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na > 0 && nb > 0 && x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace sconv
