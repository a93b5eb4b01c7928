// fa_api_util.hpp -- host-side helpers shared by the C ABI's translation
// units (fa_api.hip: forward entry points; fa_api_bwd.hip: backward).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa.h"

namespace fa_api {

// Rows past the end that a kernel may address (rounded-up tiles) before its
// buffer range check turns them into zeros; every such byte offset must
// still fit in 32 bits.
inline constexpr int64_t kRowSlack = 1024;

inline bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

inline bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

inline bool valid_dtype(fa_dtype t) { return (int)t >= (int)FA_F32 && (int)t <= (int)FA_F16; }

inline int64_t elem_bytes(fa_dtype t) { return t == FA_F32 ? 4 : 2; }

inline fa_status launch_status(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH; }

}  // namespace fa_api
