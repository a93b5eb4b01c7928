// fa_bwd.hpp -- device-side arguments and host launchers of the backward
// pass (fa_bwd_h16.hip, fa_bwd_f32.hip), kept apart from the forward's.
#pragma once

#include "fa_device.hpp"

namespace fa_impl {

// Arguments of the backward kernels: q, dout, dq are [B, H, N_q, d], k, v,
// dk, dv [B, H_kv, N_kv, d], lse and delta [B, H, N_q].
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;   // upstream gradient dO
  const float* lse;   // the forward pass's logsumexp, natural log
  const float* delta;  // D_i = dO_i . O_i, filled by the first backward kernel
  void* dq;
  void* dk;
  void* dv;
  int bh;          // B*H query heads
  int hq;          // H, query heads per batch entry
  int hkv;         // H_kv, K/V heads per batch entry; query head h uses K/V head h / hgrp
  int hgrp;        // H / H_kv
  int bkv;         // B*H_kv
  int nq;          // query rows per head (q, o, dout, dq, lse, delta)
  int nk;          // keys per K/V head (k, v, dk, dv)
  int off;         // causal alignment N_kv - N_q: key j is visible to row i when j <= i + off
  float scale;     // multiplier of q.k
  float scale_log2;  // scale * log2(e)
  // Parts a group's query heads are divided into for dK/dV (1: one
  // workgroup per key tile sums the whole group and writes dK, dV).  With
  // hsplit > 1 each part writes fp32 partial sums, unscaled, to
  // dk_part / dv_part ([hsplit][B*H_kv][N_kv][d]) and a reduce kernel adds
  // the parts in order.
  int hsplit;
  float* dk_part;
  float* dv_part;
};

// Backward pass (bf16/fp16): delta, then dK/dV, then dQ on stream s.
hipError_t launch_bwd_h16(bool bf16, int d, bool causal, const BwdArgs& a, const void* o,
                          float* delta, hipStream_t s);
// Backward pass for fp32 inputs (fp32 MFMA), same three kernels and arguments.
hipError_t launch_bwd_f32(int d, bool causal, const BwdArgs& a, const void* o, float* delta,
                          hipStream_t s);
// Largest workgroup count of the backward launches (dK/dV over the K/V heads'
// key tiles and head parts, dQ over the query heads' row tiles).
int64_t bwd_grid_blocks(int64_t bh, int64_t bkv, int64_t nq, int64_t nk, int64_t hsplit);
// Workgroups of the dK/dV launch without head parts (B*H_kv key-tile rows).
int64_t bwd_dkdv_blocks(int64_t bkv, int64_t nk);

}  // namespace fa_impl
