// fa_api_bwd.hip -- the backward entry points of libfa's C ABI (declared in
// include/fa.h): argument validation on the host, choice of kernel family,
// launch on the caller's stream.  No allocation, no synchronisation, no
// global mutable state; validation follows the forward entry points.
#include <math.h>
#include <stdint.h>

#include "fa.h"
#include "fa_api_util.hpp"
#include "fa_bwd.hpp"

using namespace fa_api;

namespace {

// dK/dV workgroups the 256 CUs hold at once: one per wave a SIMD holds
// (bf16/fp16: three at d = 64, two at d = 128; fp32: two, one).
int64_t dkdv_slots(int64_t d, fa_dtype dtype) {
  const int64_t waves = dtype == FA_F32 ? (d == 64 ? 2 : 1) : (d == 64 ? 3 : 2);
  return waves * 256;
}

// Parts a call's head groups are actually split into: at most the group
// size, and 1 when there is nothing to split (no keys or no queries).
int64_t head_parts(int64_t H, int64_t H_kv, int64_t N_q, int64_t N_kv, int64_t num_splits) {
  if (H_kv <= 0 || H % H_kv != 0 || N_q <= 0 || N_kv <= 0 || num_splits <= 1) return 1;
  const int64_t grp = H / H_kv;
  return num_splits < grp ? num_splits : grp;
}

// fp32 partial dK and dV of every part: 2 * parts * B*H_kv*N_kv*d floats;
// -1 when that overflows.
int64_t part_bytes(int64_t B, int64_t H_kv, int64_t N_kv, int64_t d, int64_t parts) {
  if (parts <= 1) return 0;
  const int64_t per = 2 * d * 4;
  if (B > INT64_MAX / H_kv / N_kv || B * H_kv * N_kv > INT64_MAX / per / parts) return -1;
  return parts * B * H_kv * N_kv * per;
}

}  // namespace

extern "C" int64_t fa_bwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t N_q,
                                             int64_t N_kv, int64_t d, int64_t num_splits) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || N_q < 0 || N_kv < 0 || (d != 64 && d != 128)) return 0;
  return part_bytes(B, H_kv, N_kv, d, head_parts(H, H_kv, N_q, N_kv, num_splits));
}

extern "C" int64_t fa_bwd_ex_default_splits(int64_t B, int64_t H, int64_t H_kv, int64_t N_q,
                                            int64_t N_kv, int64_t d, int causal,
                                            fa_dtype dtype) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || N_q <= 0 || N_kv <= 0 ||
      (d != 64 && d != 128) || !valid_dtype(dtype) || N_kv > INT32_MAX || B > INT32_MAX / H)
    return 1;
  const int64_t grp = H / H_kv;
  if (grp == 1) return 1;
  const int64_t blocks = fa_impl::bwd_dkdv_blocks(B * H_kv, N_kv);
  const int64_t slots = dkdv_slots(d, dtype);
  // Without a mask every dK/dV workgroup has the same work: split a grid of
  // less than two workgroups per slot (one wave of equal workgroups ends on
  // its slowest CU).  Under the causal mask the first key tiles carry the
  // most work; four workgroups per slot let the light ones fill in behind.
  const int64_t per_slot = causal ? 4 : 2;
  int64_t want = blocks >= per_slot * slots ? 1 : (per_slot * slots + blocks - 1) / blocks;
  // Parts of equal size only (a group of 4 cut in 3 leaves one part with two
  // heads, and the grid waits for it): the smallest divisor of the group
  // size that reaches `want`.
  for (int64_t p = want < 1 ? 1 : want; p < grp; ++p)
    if (grp % p == 0) return p;
  return grp;
}

extern "C" fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o,
                               const void* dout, const float* lse, void* dq, void* dk, void* dv,
                               float* delta, int64_t B, int64_t H, int64_t H_kv, int64_t N_q,
                               int64_t N_kv, int64_t d, float scale, int causal, fa_dtype dtype,
                               int64_t num_splits, void* workspace, int64_t workspace_bytes,
                               void* stream) {
  // the query side is not touched when N_q = 0, nor the key side when N_kv = 0
  if ((N_q != 0 && (!q || !o || !dout || !lse || !dq || !delta)) ||
      (N_kv != 0 && (!k || !v || !dk || !dv)))
    return FA_ERR_NULL;
  if (B < 0 || H < 0 || H_kv < 0 || N_q < 0 || N_kv < 0) return FA_ERR_SHAPE;
  if (!valid_dtype(dtype)) return FA_ERR_DTYPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (!isfinite(scale) || !(scale > 0.f)) return FA_ERR_SCALE;
  if (H_kv == 0 ? H != 0 : H % H_kv != 0) return FA_ERR_SHAPE;
  if (num_splits < 1) return FA_ERR_WORKSPACE;
  if (B == 0 || H == 0 || (N_q == 0 && N_kv == 0)) return FA_OK;
  const int64_t e = elem_bytes(dtype);
  if (N_q > INT32_MAX || N_kv > INT32_MAX || H > INT32_MAX || B > INT32_MAX / H)
    return FA_ERR_SHAPE;
  const int64_t bh = B * H, bkv = B * H_kv;
  if (N_q > 0 && (bh > INT64_MAX / N_q || bh * N_q > INT64_MAX / (d * e))) return FA_ERR_SHAPE;
  if (N_kv > 0 && (bkv > INT64_MAX / N_kv || bkv * N_kv > INT64_MAX / (d * e)))
    return FA_ERR_SHAPE;
  if ((N_q + kRowSlack) * d * e > INT32_MAX || (N_kv + kRowSlack) * d * e > INT32_MAX)
    return FA_ERR_SHAPE;
  const int64_t parts = head_parts(H, H_kv, N_q, N_kv, num_splits);
  const int64_t wbytes = part_bytes(B, H_kv, N_kv, d, parts);
  if (wbytes < 0) return FA_ERR_SHAPE;
  if (fa_impl::bwd_grid_blocks(bh, bkv, N_q, N_kv, parts) > INT32_MAX) return FA_ERR_SHAPE;
  if ((bh * N_q + 255) / 256 * (d / 4) > INT32_MAX) return FA_ERR_SHAPE;  // row-dot grid

  if (N_q != 0) {
    const void* qs[4] = {q, o, dout, dq};
    for (int i = 0; i < 4; ++i)
      if (!aligned(qs[i], 16)) return FA_ERR_ALIGN;
    if (!aligned(lse, 4) || !aligned(delta, 4)) return FA_ERR_ALIGN;
  }
  if (N_kv != 0 && (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16)))
    return FA_ERR_ALIGN;

  const int64_t qb = bh * N_q * d * e, kvb = bkv * N_kv * d * e, lb = bh * N_q * 4;
  const void* in[6] = {q, k, v, o, dout, lse};
  const int64_t in_bytes[6] = {qb, kvb, kvb, qb, qb, lb};
  void* out[4] = {dq, dk, dv, delta};
  const int64_t out_bytes[4] = {qb, kvb, kvb, lb};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(out[i], out_bytes[i], in[j], in_bytes[j])) return FA_ERR_ALIAS;
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(out[i], out_bytes[i], out[j], out_bytes[j])) return FA_ERR_ALIAS;
  }
  if (parts > 1) {
    if (!workspace || workspace_bytes < wbytes || !aligned(workspace, 16)) return FA_ERR_WORKSPACE;
    for (int j = 0; j < 6; ++j)
      if (overlaps(workspace, wbytes, in[j], in_bytes[j])) return FA_ERR_ALIAS;
    for (int j = 0; j < 4; ++j)
      if (overlaps(workspace, wbytes, out[j], out_bytes[j])) return FA_ERR_ALIAS;
  }

  fa_impl::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.bh = (int)bh;
  a.hq = (int)H;
  a.hkv = (int)H_kv;
  a.hgrp = (int)(H / H_kv);
  a.bkv = (int)bkv;
  a.nq = (int)N_q;
  a.nk = (int)N_kv;
  a.off = (int)(N_kv - N_q);
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
  a.hsplit = (int)parts;
  a.dk_part = parts > 1 ? (float*)workspace : nullptr;
  a.dv_part = parts > 1 ? (float*)workspace + wbytes / 8 : nullptr;
  if (dtype == FA_F32)
    return launch_status(
        fa_impl::launch_bwd_f32((int)d, causal != 0, a, o, delta, (hipStream_t)stream));
  return launch_status(fa_impl::launch_bwd_h16(dtype == FA_BF16, (int)d, causal != 0, a, o, delta,
                                               (hipStream_t)stream));
}

extern "C" fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o,
                            const void* dout, const float* lse, void* dq, void* dk, void* dv,
                            float* delta, int64_t B, int64_t H, int64_t N, int64_t d,
                            float scale, int causal, fa_dtype dtype, void* stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !delta) return FA_ERR_NULL;
  return fa_bwd_ex(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, H, N, N, d, scale, causal,
                   dtype, 1, nullptr, 0, stream);
}

