// fa_api.hip -- the C ABI of libfa (declared in include/fa.h): argument
// validation on the host, choice of kernel instance, launch on the caller's
// stream.  No allocation, no synchronisation, no global mutable state.
//
// The error surface follows the GitHub README "CUDA Flash Attention...",
// "Correctness Audit": a fixed head size is checked instead of assumed
// (there an assert(d==64); here a status code), pointers are non-aliasing
// (restrict there; an overlap check here), and launch errors are reported
// right after the launch.
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_device.hpp"

#define LIBFA_VERSION_MAJOR 0
#define LIBFA_VERSION_MINOR 1
#define LIBFA_VERSION_PATCH 0

namespace {

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  if (!a || !b || na <= 0 || nb <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

bool aligned(const void* p, uintptr_t n) { return ((uintptr_t)p % n) == 0; }

}  // namespace

extern "C" fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                            fa_dtype dtype, void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  if (B < 0 || H < 0 || N < 0) return FA_ERR_SHAPE;
  if ((int)dtype < (int)FA_F32 || (int)dtype > (int)FA_F16) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  if (B == 0 || H == 0 || N == 0) return FA_OK;

  // Sizes: N and B*H must fit the kernels' 32-bit per-head indices (element
  // offsets are 64-bit), byte counts must not overflow, and the workgroup
  // count must fit the grid.
  if (N > INT32_MAX || B > INT32_MAX / H) return FA_ERR_SHAPE;
  const int64_t bh = B * H;
  const int64_t elem = dtype == FA_F32 ? 4 : 2;
  if (bh > INT64_MAX / N || bh * N > INT64_MAX / (d * elem)) return FA_ERR_SHAPE;
  const int64_t rows = bh * N;
  // one head's rows are addressed with 32-bit byte offsets (buffer loads)
  if ((N + 256) * d * elem > INT32_MAX) return FA_ERR_SHAPE;
  const int64_t grid = dtype == FA_F32 ? fa_impl::f32_grid_blocks(bh, N)
                                       : fa_impl::h16_grid_blocks(bh, N);
  if (grid > INT32_MAX) return FA_ERR_SHAPE;

  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return FA_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return FA_ERR_ALIGN;

  const int64_t tbytes = rows * d * elem;
  const int64_t lbytes = rows * 4;
  if (overlaps(o, tbytes, q, tbytes) || overlaps(o, tbytes, k, tbytes) ||
      overlaps(o, tbytes, v, tbytes))
    return FA_ERR_ALIAS;
  if (lse && (overlaps(lse, lbytes, q, tbytes) || overlaps(lse, lbytes, k, tbytes) ||
              overlaps(lse, lbytes, v, tbytes) || overlaps(lse, lbytes, o, tbytes)))
    return FA_ERR_ALIAS;

  fa_impl::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.bh = (int)bh;
  a.n = (int)N;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);

  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = dtype == FA_F32
                           ? fa_impl::launch_fwd_f32((int)d, causal != 0, a, s)
                           : fa_impl::launch_fwd_h16(dtype == FA_BF16, (int)d, causal != 0, a, s);
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

extern "C" const char* fa_strerror(fa_status s) {
  switch (s) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "q, k, v or o is a null pointer";
    case FA_ERR_SHAPE: return "B, H or N is negative or the problem exceeds the supported size";
    case FA_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
    case FA_ERR_DTYPE: return "dtype is not FA_F32, FA_BF16 or FA_F16";
    case FA_ERR_SCALE: return "scale must be finite and greater than zero";
    case FA_ERR_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_ALIAS: return "o or lse overlaps another argument buffer";
    case FA_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
  }
  return "unknown fa_status value";
}

extern "C" int fa_version(void) {
  return LIBFA_VERSION_MAJOR * 10000 + LIBFA_VERSION_MINOR * 100 + LIBFA_VERSION_PATCH;
}
