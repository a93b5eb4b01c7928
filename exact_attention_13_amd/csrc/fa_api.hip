// fa_api.hip -- the C ABI of libfa (declared in include/fa.h): argument
// validation on the host, choice of kernel instance, launch on the caller's
// stream.  No allocation and no synchronisation; the only global state is the
// cached device address of the static scratch of fa_fwd_ex_noalloc (set once
// per device under a mutex).
//
// The error surface follows the GitHub README "CUDA Flash Attention...",
// "Correctness Audit": a fixed head size is checked instead of assumed
// (there an assert(d==64); here a status code), pointers are non-aliasing
// (restrict there; an overlap check here), and launch errors are reported
// right after the launch.
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "fa.h"
#include "fa_api_util.hpp"
#include "fa_device.hpp"

#define LIBFA_VERSION_MAJOR 0
#define LIBFA_VERSION_MINOR 5
#define LIBFA_VERSION_PATCH 0

using namespace fa_api;

namespace {

// Keys per split are a multiple of this.  A kernel whose key tile is larger
// masks the keys past its range's end and skips compute steps that start
// there.
constexpr int64_t kSplitGranule = 64;
// Most key ranges per problem a split launch uses.
constexpr int64_t kMaxSplits = 256;
// How the (batch, head) problems of a call are laid out for the kernels.
struct Plan {
  bool causal;       // a mask remains after the reductions below
  int64_t problems;  // independent problems
  int64_t nq;        // query rows per problem
  int64_t hp, hkv, grp;
  int64_t rows;      // B * H * N_q, the rows of o and lse
  int64_t rpb;       // query rows per workgroup of the chosen instance
  int64_t blocks;    // workgroups of an unsplit launch
};

// Shapes are assumed validated (non-negative, H_kv > 0, H % H_kv == 0).
Plan make_plan(int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t d, int causal,
               fa_dtype dtype) {
  Plan p;
  // One query row aligned to the end of the keys sees every key: no mask.
  p.causal = causal != 0 && N_q > 1;
  const int64_t g = H / H_kv;
  // Without a row-dependent mask the query heads of a group are packed into
  // the rows of one problem: they are adjacent in memory and share K/V.
  const bool packed = g > 1 && !p.causal;
  p.problems = B * (packed ? H_kv : H);
  p.nq = packed ? g * N_q : N_q;
  p.hp = packed ? H_kv : H;
  p.hkv = H_kv;
  p.grp = packed ? 1 : g;
  p.rows = B * H * N_q;
  p.rpb = dtype == FA_F32 ? fa_impl::f32_rows_per_block()
                          : fa_impl::h16_rows_per_block((int)d, p.causal, p.nq, p.problems);
  p.blocks = p.problems * ((p.nq + p.rpb - 1) / p.rpb);
  return p;
}

// Effective number of key ranges and keys per range for a requested count.
void split_keys(int64_t N_kv, int64_t want, int64_t* splits, int64_t* chunk) {
  const int64_t granules = (N_kv + kSplitGranule - 1) / kSplitGranule;
  if (want <= 1 || granules <= 1) {
    *splits = 1;
    *chunk = granules * kSplitGranule;
    return;
  }
  if (want > kMaxSplits) want = kMaxSplits;
  const int64_t per = (granules + want - 1) / want;
  *splits = (granules + per - 1) / per;
  *chunk = per * kSplitGranule;
}

// Shared validation of the extended call; fills the plan on success.
fa_status check_ex(const void* q, const void* k, const void* v, void* o, int64_t B, int64_t H,
                   int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t d, float scale,
                   fa_dtype dtype) {
  // k and v are never read when there are no keys
  if (!q || !o || ((!k || !v) && N_kv != 0)) return FA_ERR_NULL;
  if (B < 0 || H < 0 || H_kv < 0 || N_q < 0 || N_kv < 0) return FA_ERR_SHAPE;
  if (!valid_dtype(dtype)) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  if (H_kv == 0 ? H != 0 : H % H_kv != 0) return FA_ERR_SHAPE;
  return FA_OK;
}

// Size limits of a non-empty call: 32-bit per-head indices and byte
// offsets, no overflow of byte counts, grids that fit.
fa_status check_sizes(int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t d,
                      fa_dtype dtype, const Plan& p, int64_t splits) {
  const int64_t e = elem_bytes(dtype);
  if (N_q > INT32_MAX || N_kv > INT32_MAX || H > INT32_MAX || B > INT32_MAX / H)
    return FA_ERR_SHAPE;
  const int64_t bh = B * H, bhkv = B * H_kv;
  if (bh > INT64_MAX / N_q || bh * N_q > INT64_MAX / (d * 4 * kMaxSplits)) return FA_ERR_SHAPE;
  if (N_kv > 0 && (bhkv > INT64_MAX / N_kv || bhkv * N_kv > INT64_MAX / (d * e)))
    return FA_ERR_SHAPE;
  if (p.problems > INT32_MAX || p.nq > INT32_MAX) return FA_ERR_SHAPE;
  if ((p.nq + kRowSlack) * d * e > INT32_MAX || (N_kv + kRowSlack) * d * e > INT32_MAX)
    return FA_ERR_SHAPE;
  if (p.blocks > INT32_MAX / splits) return FA_ERR_SHAPE;
  if (splits > 1 && fa_impl::combine_grid_blocks(p.rows, (int)d) > INT32_MAX) return FA_ERR_SHAPE;
  return FA_OK;
}

void* device_scratch_for(void* stream);

// The whole extended forward call.  `workspace` is the caller's buffer
// (fa_fwd_ex); with static_ws (fa_fwd_ex_noalloc) the partials go to the
// static scratch of the stream's device instead, whose address is looked up
// only after every argument has been validated, and partials larger than
// workspace_bytes (the scratch size) report FA_ERR_SCRATCH.
fa_status fwd_ex_impl(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t d,
                      float scale, int causal, fa_dtype dtype, int64_t num_splits,
                      void* workspace, int64_t workspace_bytes, void* stream, bool static_ws) {
  fa_status st = check_ex(q, k, v, o, B, H, H_kv, N_q, N_kv, d, scale, dtype);
  if (st != FA_OK) return st;
  if (num_splits < 1) return FA_ERR_WORKSPACE;
  if (B == 0 || H == 0 || N_q == 0) return FA_OK;

  const Plan p = make_plan(B, H, H_kv, N_q, d, causal, dtype);
  int64_t splits, chunk;
  split_keys(N_kv, num_splits, &splits, &chunk);
  st = check_sizes(B, H, H_kv, N_q, N_kv, d, dtype, p, splits);
  if (st != FA_OK) return st;

  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16))
    return FA_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return FA_ERR_ALIGN;

  const int64_t e = elem_bytes(dtype);
  const int64_t qbytes = p.rows * d * e;
  const int64_t kvbytes = B * H_kv * N_kv * d * e;
  const int64_t lbytes = p.rows * 4;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kvbytes) ||
      overlaps(o, qbytes, v, kvbytes))
    return FA_ERR_ALIAS;
  if (lse && (overlaps(lse, lbytes, q, qbytes) || overlaps(lse, lbytes, k, kvbytes) ||
              overlaps(lse, lbytes, v, kvbytes) || overlaps(lse, lbytes, o, qbytes)))
    return FA_ERR_ALIAS;

  const int64_t wbytes = splits > 1 ? splits * p.rows * (d + 1) * 4 : 0;
  if (splits > 1 && static_ws) {
    if (wbytes > workspace_bytes) return FA_ERR_SCRATCH;
    workspace = device_scratch_for(stream);
    if (!workspace) return FA_ERR_LAUNCH;
  }
  if (splits > 1) {
    if (!workspace || workspace_bytes < wbytes || !aligned(workspace, 16))
      return FA_ERR_WORKSPACE;
    if (overlaps(workspace, wbytes, q, qbytes) || overlaps(workspace, wbytes, k, kvbytes) ||
        overlaps(workspace, wbytes, v, kvbytes) || overlaps(workspace, wbytes, o, qbytes) ||
        (lse && overlaps(workspace, wbytes, lse, lbytes)))
      return FA_ERR_ALIAS;
  }

  fa_impl::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.problems = (int)p.problems;
  a.nq = (int)p.nq;
  a.nk = (int)N_kv;
  a.hp = (int)p.hp;
  a.hkv = (int)p.hkv;
  a.grp = (int)p.grp;
  a.causal_off = (int)(N_kv - N_q);
  a.splits = (int)splits;
  a.kv_chunk = (int)chunk;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  float* ws_o = (float*)workspace;
  float* ws_lse = splits > 1 ? ws_o + splits * p.rows * d : nullptr;
  a.o = splits > 1 ? (void*)ws_o : o;
  a.lse = splits > 1 ? ws_lse : lse;

  hipStream_t s = (hipStream_t)stream;
  const bool split = splits > 1;
  st = launch_status(dtype == FA_F32
                         ? fa_impl::launch_fwd_f32((int)d, p.causal, split, a, s)
                         : fa_impl::launch_fwd_h16(dtype == FA_BF16, (int)d, p.causal, split, a, s));
  if (st != FA_OK || !split) return st;
  return launch_status(fa_impl::launch_lse_combine(ws_o, ws_lse, (int)splits, p.rows, (int)d, o,
                                                   lse, (int)dtype, s));
}

// ---------------------------------------------------------------------------
// Static scratch for callers that cannot allocate (fa_fwd_ex_noalloc).
//
// `scratch` is a device array in the library's code object: every GPU the
// library runs on holds its own copy, at its own address, from the first
// use until the process ends.  In host code the name is only a stand-in for
// the symbol; the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and cached here, and only
// that address is ever passed to a kernel.  The split kernels write every
// partial row of their ranges before the combine reads it, so nothing has to
// be cleared between calls.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on `dev` (nullptr when the lookup fails).
void* device_scratch(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr) return ptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (ptr) return ptr;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  void* addr = nullptr;
  const hipError_t e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || !addr) return nullptr;
  g_scratch_ptr[dev].store(addr, std::memory_order_release);
  return addr;
}

// The scratch of the device that runs `stream` (the current device for the
// null stream).
void* device_scratch_for(void* stream) {
  int dev = -1;
  if (stream ? hipStreamGetDevice((hipStream_t)stream, &dev) != hipSuccess
             : hipGetDevice(&dev) != hipSuccess)
    return nullptr;
  return device_scratch(dev);
}

}  // namespace

extern "C" fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t B, int64_t H, int64_t H_kv, int64_t N_q, int64_t N_kv,
                               int64_t d, float scale, int causal, fa_dtype dtype,
                               int64_t num_splits, void* workspace, int64_t workspace_bytes,
                               void* stream) {
  return fwd_ex_impl(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale, causal, dtype, num_splits,
                     workspace, workspace_bytes, stream, false);
}

extern "C" fa_status fa_fwd_ex_noalloc(const void* q, const void* k, const void* v, void* o,
                                       float* lse, int64_t B, int64_t H, int64_t H_kv,
                                       int64_t N_q, int64_t N_kv, int64_t d, float scale,
                                       int causal, fa_dtype dtype, int64_t num_splits,
                                       void* stream) {
  return fwd_ex_impl(q, k, v, o, lse, B, H, H_kv, N_q, N_kv, d, scale, causal, dtype, num_splits,
                     nullptr, FA_NOALLOC_SCRATCH_BYTES, stream, true);
}

extern "C" fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                            int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                            fa_dtype dtype, void* stream) {
  if (!q || !k || !v || !o) return FA_ERR_NULL;
  return fa_fwd_ex(q, k, v, o, lse, B, H, H, N, N, d, scale, causal, dtype, 1, nullptr, 0,
                   stream);
}

extern "C" int64_t fa_fwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t N_q, int64_t N_kv,
                                             int64_t d, int64_t num_splits) {
  if (B <= 0 || H <= 0 || N_q <= 0 || N_kv < 0 || d <= 0 || num_splits < 1) return 0;
  int64_t splits, chunk;
  split_keys(N_kv, num_splits, &splits, &chunk);
  if (splits <= 1) return 0;
  if (B > INT64_MAX / H || B * H > INT64_MAX / N_q ||
      B * H * N_q > INT64_MAX / ((d + 1) * 4 * splits))
    return -1;
  return splits * B * H * N_q * (d + 1) * 4;
}

extern "C" int64_t fa_fwd_ex_default_splits(int64_t B, int64_t H, int64_t H_kv, int64_t N_q,
                                            int64_t N_kv, int64_t d, int causal,
                                            fa_dtype dtype) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || N_q <= 0 || N_kv <= 0) return 1;
  if ((d != 64 && d != 128) || !valid_dtype(dtype)) return 1;
  const Plan p = make_plan(B, H, H_kv, N_q, d, causal, dtype);
  // fp32 problems that the unsplit launch hands to the small-problem kernel
  // stay unsplit while each 16-row block's key chain is short: measured on
  // MI355X, up to N_kv d = 64 Ki the one kernel beats the split call and its
  // combine (one 512-row head, d = 64: 11.0 against 15.1 us with 8 ranges;
  // 2 x 4 heads of 256 rows: 9.4 against 15.4), beyond it splitting gains
  // (2048 keys at d = 64: 22.8 against 25.1 us; d = 128: 30.4 against 47.5).
  if (dtype == FA_F32 && fa_impl::f32_small_kernel(p.nq, p.problems, p.causal, (int)d) &&
      N_kv * d <= 65536)
    return 1;
  // Aim for about two workgroups per compute unit (256 CUs) where several
  // fit on one (fp32, and the one-wave workgroups of short bf16/fp16 rows,
  // which stream K/V), one per compute unit for the multi-wave bf16/fp16
  // tiles (eight-wave d = 64 tiles fill a compute unit; the split call's
  // partial results and combine then cost more than the rest of the chip
  // gains).  More ranges do not stream K/V faster (a decoding step already
  // reads at the rate a plain streaming read reaches) but cost partial
  // results and a longer combine.  Each range keeps enough keys that its
  // fixed costs (Q load, partial write) stay small; short key sequences
  // of problems of at most 2048 query rows in all take shorter ranges.  (Measured on MI355X over 1-32 heads, N_q 1-2048,
  // N_kv 512-65536: one 512-row bf16 head at d = 64 21.2 -> 18.3 us,
  // 16 heads of 2048 rows 59.7 -> 45.2 us, d = 128 with 128 row blocks
  // 34.5 -> 28.6 us unsplit; decoding shapes unchanged.)
  const bool multi_wave = dtype != FA_F32 && p.rpb > 32;
  const int64_t target = multi_wave ? 256 : 512;
  if (p.blocks >= target / 2) return 1;
  int64_t want = (target + p.blocks - 1) / p.blocks;
  const int64_t min_keys = dtype == FA_F32 ? 64 : (N_kv <= 1024 && p.rows <= 2048 ? 128 : 256);
  int64_t most = N_kv / min_keys;
  if (most < 1) most = 1;
  if (want > most) want = most;
  if (want > kMaxSplits) want = kMaxSplits;
  int64_t splits, chunk;
  split_keys(N_kv, want, &splits, &chunk);
  return splits;
}

extern "C" fa_status fa_lse_combine(const float* o_part, const float* lse_part, int64_t splits,
                                    int64_t rows, int64_t d, void* o, float* lse,
                                    fa_dtype dtype, void* stream) {
  if (!o_part || !lse_part || !o) return FA_ERR_NULL;
  if (rows < 0 || splits < 1 || splits > INT32_MAX) return FA_ERR_SHAPE;
  if (!valid_dtype(dtype)) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (rows == 0) return FA_OK;
  if (rows > INT64_MAX / (splits * (d + 1) * 4)) return FA_ERR_SHAPE;
  if (fa_impl::combine_grid_blocks(rows, (int)d) > INT32_MAX) return FA_ERR_SHAPE;
  if (!aligned(o_part, 16) || !aligned(o, 16) || !aligned(lse_part, 4)) return FA_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return FA_ERR_ALIGN;
  const int64_t pbytes = splits * rows * d * 4, plbytes = splits * rows * 4;
  const int64_t obytes = rows * d * elem_bytes(dtype), lbytes = rows * 4;
  if (overlaps(o, obytes, o_part, pbytes) || overlaps(o, obytes, lse_part, plbytes))
    return FA_ERR_ALIAS;
  if (lse && (overlaps(lse, lbytes, o_part, pbytes) || overlaps(lse, lbytes, lse_part, plbytes) ||
              overlaps(lse, lbytes, o, obytes)))
    return FA_ERR_ALIAS;
  return launch_status(fa_impl::launch_lse_combine(o_part, lse_part, (int)splits, rows, (int)d, o,
                                                   lse, (int)dtype, (hipStream_t)stream));
}

extern "C" const char* fa_strerror(fa_status s) {
  switch (s) {
    case FA_OK: return "success";
    case FA_ERR_NULL: return "a required pointer argument is null";
    case FA_ERR_SHAPE:
      return "a size is negative, H is not a multiple of H_kv, or the problem exceeds the "
             "supported size";
    case FA_ERR_HEAD_DIM: return "head dimension d must be 64 or 128";
    case FA_ERR_DTYPE: return "dtype is not FA_F32, FA_BF16 or FA_F16";
    case FA_ERR_SCALE: return "scale must be finite and greater than zero";
    case FA_ERR_ALIGN: return "tensor pointers must be 16-byte aligned and lse 4-byte aligned";
    case FA_ERR_ALIAS: return "an output or workspace buffer overlaps another argument buffer";
    case FA_ERR_LAUNCH: return "the HIP runtime refused the kernel launch";
    case FA_ERR_WORKSPACE:
      return "num_splits is below 1, or the workspace is null, too small or misaligned";
    case FA_ERR_SCRATCH:
      return "the split partials exceed the static scratch of fa_fwd_ex_noalloc "
             "(FA_NOALLOC_SCRATCH_BYTES); use fewer splits or fa_fwd_ex with a workspace";
  }
  return "unknown fa_status value";
}

extern "C" int fa_version(void) {
  return LIBFA_VERSION_MAJOR * 10000 + LIBFA_VERSION_MINOR * 100 + LIBFA_VERSION_PATCH;
}
