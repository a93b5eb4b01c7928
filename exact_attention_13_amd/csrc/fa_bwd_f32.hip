// fa_bwd_f32.hip -- FlashAttention backward pass, fp32 in / fp32 MFMA / fp32
// out, for MI355X (gfx950).
//
// The same recomputation as the bf16/fp16 backward ("FlashAttention
// dissected", section "Memory complexity: from O(N^2) to O(N)": the weights
// are rebuilt from Q, K and the forward pass's logsumexp instead of being
// stored), with P_ij = exp(scale q_i.k_j - LSE_i) (0 where masked):
//     D_i = dO_i . O_i,   dS_ij = P_ij (dO_i . v_j - D_i),
//     dV_j = sum_i P_ij dO_i,   dK_j = scale sum_i dS_ij q_i,
//     dQ_i = scale sum_j dS_ij k_j.
// Three kernels, no atomics (bitwise reproducible), all products on
// v_mfma_f32_32x32x2_f32 with the fp32 forward kernel's operand scheme: a
// 2-deep contraction per instruction whose order is permuted so that lane
// half g takes elements 8j + 4g + e, e = 0..3, of four consecutive
// instructions from one 16-byte read, and an accumulator's register r
// (rows 8(r/4) + 4g + r%4) is, unchanged, the B operand of instruction r of
// the next product:
//   * bwd_delta_f32_kernel: D_i, d/4 lanes per row;
//   * bwd_dkdv_f32_kernel: one workgroup per (128 keys, K/V head, part of
//     the group's query heads), four waves of 32 keys holding their K and V
//     rows in registers; 32-query tiles of Q and dO of every query head of
//     the part pass through double-buffered
//     LDS row-major (S = Q K^T, dP = dO V^T: each lane holds one key) and
//     transposed (Q^T, dO^T: the A operands of dK^T += Q^T dS and
//     dV^T += dO^T P);
//   * bwd_dq_f32_kernel: one workgroup per (query head, 128 queries), the
//     forward's shape: Q and dO rows in registers, S^T = K Q^T and
//     dP^T = V dO^T give each lane one query; 32-key tiles of K (row-major and
//     transposed) and V (row-major) in LDS; dQ^T += K^T dS^T.
// Causal masking (key j visible to row i when j <= i + N_kv - N_q), ragged
// tails and rows without a visible key follow the bf16/fp16 backward.
#include "fa_bwd.hpp"

namespace fa_impl {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // keys (dK/dV) or queries (dQ) per workgroup
constexpr int kBT = 32;             // rows of a streamed tile
constexpr float kLog2e = 1.44269504088896340736f;

template <int D>
struct Tile32 {
  static constexpr int kRowStride = D + 4;  // row-major tile: floats per row (+16 B)
  static constexpr int kTStride = kBT + 4;  // transposed tile: floats per row (+16 B)
  static constexpr int kRowFloats = kBT * kRowStride;
  static constexpr int kTFloats = D * kTStride;
  // staging unit: 4 consecutive rows x 4 consecutive columns (four 16-byte loads)
  static constexpr int kUnits = (kBT / 4) * (D / 4);
};

__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 ld4(__amdgpu_buffer_rsrc_t r, int float_off) {
  return __builtin_bit_cast(f32x4, buf_load16(r, float_off * 4));
}

// logsumexp in exp2 units; a row without a visible key (LSE = -inf) gets +inf
// so that every weight exp2(s c - lse2) is 0.
__device__ __forceinline__ float lse2_of(float lse) {
  return lse == kNegInf ? __builtin_inff() : lse * kLog2e;
}

// One staging unit: rows r0 .. r0+3, columns 4cc .. 4cc+3 of a [rows, D] array.
template <int D>
__device__ __forceinline__ void load_unit(__amdgpu_buffer_rsrc_t r, int r0, int cc, f32x4* x) {
#pragma unroll
  for (int h = 0; h < 4; ++h) x[h] = ld4(r, (r0 + h) * D + cc * 4);
}

// Unit u of a tile: row group and column group.
template <int D>
__device__ __forceinline__ void unit_pos(int u, int& rq, int& cc) {
  rq = u % (kBT / 4);
  cc = u / (kBT / 4);
}

// Store a unit row-major (rows 4rq .. +3) and transposed (columns become rows).
template <int D>
__device__ __forceinline__ void store_unit(float* rm, float* tm, int rq, int cc, const f32x4* x) {
  using T = Tile32<D>;
#pragma unroll
  for (int h = 0; h < 4; ++h) *(f32x4*)(rm + (4 * rq + h) * T::kRowStride + cc * 4) = x[h];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const f32x4 w = {x[0][e], x[1][e], x[2][e], x[3][e]};
    *(f32x4*)(tm + (cc * 4 + e) * T::kTStride + rq * 4) = w;
  }
}

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_f32_kernel(const float* __restrict__ o,
                                                            const float* __restrict__ dout,
                                                            float* __restrict__ delta,
                                                            int64_t rows) {
  constexpr int kLanes = D / 4;
  constexpr int kRowsPerBlock = 256 / kLanes;
  const int sub = threadIdx.x % kLanes;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanes;
  float acc = 0.f;
  if (row < rows) {
    const f32x4 x = *(const f32x4*)(o + row * D + sub * 4);
    const f32x4 y = *(const f32x4*)(dout + row * D + sub * 4);
    acc = x[0] * y[0] + x[1] * y[1] + x[2] * y[2] + x[3] * y[3];
  }
#pragma unroll
  for (int off = kLanes / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && sub == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (128 keys, K/V head, head part), summing the
// query heads of its part in registers (the whole group with one part).  At
// d = 64 two waves share a SIMD.
// ---------------------------------------------------------------------------
template <bool CAUSAL, int D>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 64 ? 2 : 1))) void bwd_dkdv_f32_kernel(BwdArgs a) {
  using T = Tile32<D>;
  constexpr int kStage = 2 * (T::kRowFloats + T::kTFloats);  // Qr, Qt, dOr, dOt
  constexpr int kPer = 2 * T::kUnits / kThreads;             // Q and dO units per thread
  static_assert(T::kUnits % 64 == 0 && kPer >= 1 && kPer * kThreads == 2 * T::kUnits,
                "unit split");
  __shared__ __attribute__((aligned(16))) float lds[2 * kStage];
  __shared__ __attribute__((aligned(16))) float stat[2][2][kBT];  // [stage][lse2, D][query]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, grp = lane >> 5;
  const int nq = a.nq, nk = a.nk, off = a.off;

  // workgroup -> (key tile, K/V head, part of the group's query heads), key
  // tiles outermost (as in the bf16/fp16 kernel)
  const int units = a.bkv * a.hsplit;
  const int kt = blockIdx.x / units;
  const int unit = blockIdx.x - kt * units;
  const int bkv = unit / a.hsplit, sp = unit - bkv * a.hsplit;
  const int k0 = kt * kRows;
  const int kw0 = k0 + wave * 32;
  const int b = bkv / a.hkv;
  const int h_lo = sp * a.hgrp / a.hsplit, h_hi = (sp + 1) * a.hgrp / a.hsplit;
  const int bh0 = b * a.hq + (bkv - b * a.hkv) * a.hgrp + h_lo;

  const int64_t kvhead = (int64_t)bkv * nk * D;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const float*)a.k + kvhead, nk * D * 4);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const float*)a.v + kvhead, nk * D * 4);

  // K and V rows of this lane's key as B operands: kf[j][e] = K[key][8j + 4g + e].
  f32x4 kf[D / 8], vf[D / 8];
#pragma unroll
  for (int j = 0; j < D / 8; ++j) {
    kf[j] = ld4(kr, (kw0 + col) * D + j * 8 + grp * 4);
    vf[j] = ld4(vr, (kw0 + col) * D + j * 8 + grp * 4);
  }

  const int n_qt = (nq + kBT - 1) / kBT;
  const int qt_begin = CAUSAL ? max(0, (k0 - off) / kBT) : 0;
  const int n_iter = max(0, n_qt - qt_begin);
  const int total_it = n_iter * (h_hi - h_lo);

  // Units [0, kUnits) are Q's, [kUnits, 2 kUnits) dO's; whole waves take one
  // kind, so the buffer resource is wave-uniform.
  f32x4 sx[kPer][4];
  float st = 0.f;
  auto load_tile = [&](int hh, int q0) {
    const int64_t bhq = bh0 + hh;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc((const float*)a.q + bhq * nq * D, nq * D * 4);
    const __amdgpu_buffer_rsrc_t gr = make_rsrc((const float*)a.dout + bhq * nq * D, nq * D * 4);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * kThreads;
      int rq, cc;
      unit_pos<D>(u % T::kUnits, rq, cc);
      if (wave * 64 + i * kThreads < T::kUnits)
        load_unit<D>(qr, q0 + 4 * rq, cc, sx[i]);
      else
        load_unit<D>(gr, q0 + 4 * rq, cc, sx[i]);
    }
    const __amdgpu_buffer_rsrc_t lr = make_rsrc(a.lse + bhq * nq, nq * 4);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(a.delta + bhq * nq, nq * 4);
    if (tid < kBT)
      st = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lr, (q0 + tid) * 4, 0, 0));
    else if (tid < 2 * kBT)
      st = __builtin_bit_cast(float,
                              __builtin_amdgcn_raw_buffer_load_b32(dr, (q0 + tid - kBT) * 4, 0, 0));
  };
  auto store_tile = [&](int buf) {
    float* base = lds + buf * kStage;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * kThreads;
      int rq, cc;
      unit_pos<D>(u % T::kUnits, rq, cc);
      float* rm = base + (wave * 64 + i * kThreads < T::kUnits ? 0 : T::kRowFloats + T::kTFloats);
      store_unit<D>(rm, rm + T::kRowFloats, rq, cc, sx[i]);
    }
    if (tid < 2 * kBT) stat[buf][tid / kBT][tid % kBT] = tid < kBT ? lse2_of(st) : -st;
  };

  const float c = a.scale_log2;
  f32x16 dkT[D / 32], dvT[D / 32];  // dK^T, dV^T: lane holds key kw0 + col
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dkT[db] = dvT[db] = (f32x16){};

  load_tile(0, qt_begin * kBT);
  store_tile(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int key = kw0 + col;
  int hh = 0, qt = qt_begin;
  for (int it = 0; it < total_it; ++it) {
    const int buf = it & 1;
    const int q0 = qt * kBT;
    const bool more = it + 1 < total_it;
    const bool wrap = qt + 1 == n_qt;
    const int hh_next = wrap ? hh + 1 : hh;
    const int qt_next = wrap ? qt_begin : qt + 1;
    if (more) load_tile(hh_next, qt_next * kBT);

    if (!(CAUSAL && q0 + kBT - 1 + off < kw0)) {
      const float* qrm = lds + buf * kStage;
      const float* qtm = qrm + T::kRowFloats;
      const float* grm = qtm + T::kTFloats;
      const float* gtm = grm + T::kRowFloats;

      // S = Q K^T, dP - D = dO V^T - D: lane holds key `key`, register r
      // the query q0 + 8(r/4) + 4g + r%4; the dP product starts from -D.
      f32x16 s = {}, dp;
#pragma unroll
      for (int jr = 0; jr < 4; ++jr) {
        const f32x4 nd = *(const f32x4*)(&stat[buf][1][8 * jr + 4 * grp]);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * jr + e] = nd[e];
      }
#pragma unroll
      for (int j = 0; j < D / 8; ++j) {
        const f32x4 qa = *(const f32x4*)(qrm + col * T::kRowStride + j * 8 + grp * 4);
        const f32x4 ga = *(const f32x4*)(grm + col * T::kRowStride + j * 8 + grp * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = mfma32(qa[e], kf[j][e], s);
          dp = mfma32(ga[e], vf[j][e], dp);
        }
      }

      // Only the causal mask is applied: a query row past the end has zero
      // Q and dO rows and a zero lse and D, so its weights add exact zeros,
      // and a key past the end only touches its own dK/dV column, which is
      // never stored.  key > query + off reads kq > 8 (r/4) + r%4.
      const bool diag = CAUSAL && q0 + off < kw0 + 31;
      const int kq = key - q0 - off - 4 * grp;
#pragma unroll
      for (int jr = 0; jr < 4; ++jr) {
        const f32x4 l4 = *(const f32x4*)(&stat[buf][0][8 * jr + 4 * grp]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * jr + e;
          float p = fast_exp2(fmaf(s[r], c, -l4[e]));
          if (diag) p = kq > 8 * jr + e ? 0.f : p;
          s[r] = p;                       // P
          dp[r] = p * dp[r];              // dS
        }
      }

      // dV^T += dO^T P and dK^T += Q^T dS: instruction r takes register r.
#pragma unroll
      for (int jr = 0; jr < 4; ++jr)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const f32x4 ga = *(const f32x4*)(gtm + (db * 32 + col) * T::kTStride + 8 * jr + 4 * grp);
          const f32x4 qa = *(const f32x4*)(qtm + (db * 32 + col) * T::kTStride + 8 * jr + 4 * grp);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            dvT[db] = mfma32(ga[e], s[4 * jr + e], dvT[db]);
            dkT[db] = mfma32(qa[e], dp[4 * jr + e], dkT[db]);
          }
        }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
    hh = hh_next;
    qt = qt_next;
  }

  // dK = scale (Q^T dS)^T, dV = (dO^T P)^T; lane holds key `key`, register r
  // the column db*32 + 8(r/4) + 4g + r%4.
  if (key < nk) {
    const bool parts = a.hsplit > 1;  // this part's sums, unscaled, for the reduce kernel
    const int64_t prow = ((int64_t)sp * a.bkv + bkv) * nk + key;
    float* dkg = parts ? a.dk_part + prow * D : (float*)a.dk + kvhead + (int64_t)key * D;
    float* dvg = parts ? a.dv_part + prow * D : (float*)a.dv + kvhead + (int64_t)key * D;
    const float ks = parts ? 1.f : a.scale;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jr = 0; jr < 4; ++jr) {
        const int d0 = db * 32 + 8 * jr + 4 * grp;
        const f32x4 wk = {dkT[db][4 * jr] * ks, dkT[db][4 * jr + 1] * ks,
                          dkT[db][4 * jr + 2] * ks, dkT[db][4 * jr + 3] * ks};
        const f32x4 wv = {dvT[db][4 * jr], dvT[db][4 * jr + 1], dvT[db][4 * jr + 2],
                          dvT[db][4 * jr + 3]};
        *(f32x4*)(dkg + d0) = wk;
        *(f32x4*)(dvg + d0) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (query head, 128 queries)
// ---------------------------------------------------------------------------
template <bool CAUSAL, int D>
__global__ __launch_bounds__(kThreads) void bwd_dq_f32_kernel(BwdArgs a, int n_qt, int total) {
  using T = Tile32<D>;
  constexpr int kStage = 2 * T::kRowFloats + T::kTFloats;  // Kr, Kt, Vr
  constexpr int kPer = 2 * T::kUnits / kThreads;            // K and V units per thread
  static_assert(T::kUnits % 64 == 0 && kPer >= 1 && kPer * kThreads == 2 * T::kUnits,
                "unit split");
  __shared__ __attribute__((aligned(16))) float lds[2 * kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, grp = lane >> 5;
  const int nq = a.nq, nk = a.nk, off = a.off;

  const int L = xcd_remap(blockIdx.x, total);
  int bh, qt;
  tile_of<CAUSAL>(L, total, n_qt, bh, qt);
  const int q0 = qt * kRows;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + col;
  const int b = bh / a.hq;
  const int bkv = b * a.hkv + (bh - b * a.hq) / a.hgrp;

  const int64_t qhead = (int64_t)bh * nq * D, kvhead = (int64_t)bkv * nk * D;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc((const float*)a.q + qhead, nq * D * 4);
  const __amdgpu_buffer_rsrc_t gr = make_rsrc((const float*)a.dout + qhead, nq * D * 4);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const float*)a.k + kvhead, nk * D * 4);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const float*)a.v + kvhead, nk * D * 4);
  const __amdgpu_buffer_rsrc_t lr = make_rsrc(a.lse + (int64_t)bh * nq, nq * 4);
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(a.delta + (int64_t)bh * nq, nq * 4);

  // Q and dO rows of this lane's query as B operands: qf[j][e] = Q[my_q][8j + 4g + e].
  f32x4 qf[D / 8], gf[D / 8];
#pragma unroll
  for (int j = 0; j < D / 8; ++j) {
    qf[j] = ld4(qr, my_q * D + j * 8 + grp * 4);
    gf[j] = ld4(gr, my_q * D + j * 8 + grp * 4);
  }
  const float lse2 =
      lse2_of(__builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lr, my_q * 4, 0, 0)));
  const float drow =
      __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dr, my_q * 4, 0, 0));
  f32x16 ndrow;  // -D of the lane's row in every register: the start of dP - D
#pragma unroll
  for (int r = 0; r < 16; ++r) ndrow[r] = -drow;

  // causal: row i sees keys j <= i + off
  const int kv_end = CAUSAL ? max(0, min(q0 + kRows + off, nk)) : nk;
  const int n_kv = (kv_end + kBT - 1) / kBT;
  const int wave_kv_end = CAUSAL ? max(0, min(qw0 + 32 + off, nk)) : nk;

  f32x4 sx[kPer][4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * kThreads;
      int rq, cc;
      unit_pos<D>(u % T::kUnits, rq, cc);
      if (wave * 64 + i * kThreads < T::kUnits)
        load_unit<D>(kr, k0 + 4 * rq, cc, sx[i]);
      else
        load_unit<D>(vr, k0 + 4 * rq, cc, sx[i]);
    }
  };
  auto store_tile = [&](int buf) {
    float* base = lds + buf * kStage;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int u = tid + i * kThreads;
      int rq, cc;
      unit_pos<D>(u % T::kUnits, rq, cc);
      if (wave * 64 + i * kThreads < T::kUnits) {
        store_unit<D>(base, base + T::kRowFloats, rq, cc, sx[i]);  // Kr, Kt
      } else {
        float* vm = base + T::kRowFloats + T::kTFloats;  // Vr
#pragma unroll
        for (int h = 0; h < 4; ++h) *(f32x4*)(vm + (4 * rq + h) * T::kRowStride + cc * 4) = sx[i][h];
      }
    }
  };

  const float c = a.scale_log2;
  f32x16 dqT[D / 32];  // dQ^T: lane holds query my_q
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dqT[db] = (f32x16){};

  load_tile(0);
  store_tile(0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < n_kv; ++t) {
    const int k0 = t * kBT, buf = t & 1;
    const bool more = t + 1 < n_kv;
    if (more) load_tile(k0 + kBT);

    if (k0 < wave_kv_end) {
      const float* krm = lds + buf * kStage;
      const float* ktm = krm + T::kRowFloats;
      const float* vrm = ktm + T::kTFloats;

      // S^T = K Q^T, dP^T - D = V dO^T - D: lane holds query my_q, register
      // r the key k0 + 8(r/4) + 4g + r%4; the dP product starts from -D.
      f32x16 s = {}, dp = ndrow;
#pragma unroll
      for (int j = 0; j < D / 8; ++j) {
        const f32x4 ka = *(const f32x4*)(krm + col * T::kRowStride + j * 8 + grp * 4);
        const f32x4 va = *(const f32x4*)(vrm + col * T::kRowStride + j * 8 + grp * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = mfma32(ka[e], qf[j][e], s);
          dp = mfma32(va[e], gf[j][e], dp);
        }
      }

      // Masked keys (past the end, or after the row's last visible key):
      // register r holds key k0 + 8 (r/4) + 4 grp + r%4, masked when
      // 8 (r/4) + r%4 exceeds one per-lane limit.
      const bool edge = k0 + kBT > nk || (CAUSAL && k0 + kBT - 1 > qw0 + off);
      const int lim = (CAUSAL ? min(nk - 1, my_q + off) : nk - 1) - k0 - 4 * grp;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(fmaf(s[r], c, -lse2));
        if (edge) p = 8 * (r >> 2) + (r & 3) > lim ? 0.f : p;
        dp[r] = p * dp[r];  // dS^T
      }

      // dQ^T += K^T dS^T: instruction r takes register r.
#pragma unroll
      for (int jr = 0; jr < 4; ++jr)
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const f32x4 ka = *(const f32x4*)(ktm + (db * 32 + col) * T::kTStride + 8 * jr + 4 * grp);
#pragma unroll
          for (int e = 0; e < 4; ++e) dqT[db] = mfma32(ka[e], dp[4 * jr + e], dqT[db]);
        }
    }

    if (more) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (my_q < nq) {
    float* g = (float*)a.dq + qhead + (int64_t)my_q * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int jr = 0; jr < 4; ++jr) {
        const f32x4 w = {dqT[db][4 * jr] * a.scale, dqT[db][4 * jr + 1] * a.scale,
                         dqT[db][4 * jr + 2] * a.scale, dqT[db][4 * jr + 3] * a.scale};
        *(f32x4*)(g + db * 32 + 8 * jr + 4 * grp) = w;
      }
  }
}

// dK, dV from the parts of split head groups (sum in part order, dK times
// scale), fp32.
__global__ __launch_bounds__(256) void bwd_part_sum_f32_kernel(const float* __restrict__ dk_part,
                                                               const float* __restrict__ dv_part,
                                                               int parts, int64_t quads,
                                                               float scale, float* __restrict__ dk,
                                                               float* __restrict__ dv) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= quads) return;
  f32x4 sk = *(const f32x4*)(dk_part + i * 4);
  f32x4 sv = *(const f32x4*)(dv_part + i * 4);
  for (int p = 1; p < parts; ++p) {
    sk += *(const f32x4*)(dk_part + (p * quads + i) * 4);
    sv += *(const f32x4*)(dv_part + (p * quads + i) * 4);
  }
  *(f32x4*)(dk + i * 4) = sk * scale;
  *(f32x4*)(dv + i * 4) = sv;
}

template <bool CAUSAL, int D>
hipError_t launch(const BwdArgs& a, const void* o, float* delta, hipStream_t s) {
  BwdArgs args = a;
  hipError_t e;
  const int64_t rows = (int64_t)a.bh * a.nq;
  if (rows > 0) {
    constexpr int kRowsPerBlock = 256 / (D / 4);
    const float* op = (const float*)o;
    const float* gp = (const float*)a.dout;
    int64_t rows_arg = rows;
    void* p0[] = {&op, &gp, &delta, &rows_arg};
    e = hipLaunchKernel((const void*)&bwd_delta_f32_kernel<D>,
                        dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(256),
                        p0, 0, s);
    if (e != hipSuccess) return e;
  }
  int n_kt = (a.nk + kRows - 1) / kRows;
  int total_kv = (int)((int64_t)n_kt * a.bkv * a.hsplit);
  if (total_kv > 0) {
    void* p1[] = {&args};
    e = hipLaunchKernel((const void*)&bwd_dkdv_f32_kernel<CAUSAL, D>, dim3(total_kv),
                        dim3(kThreads), p1, 0, s);
    if (e != hipSuccess) return e;
    if (a.hsplit > 1) {
      const float* kp = a.dk_part;
      const float* vp = a.dv_part;
      int parts = a.hsplit;
      int64_t quads = (int64_t)a.bkv * a.nk * (D / 4);
      float scale = a.scale;
      float* dkp = (float*)a.dk;
      float* dvp = (float*)a.dv;
      void* p3[] = {&kp, &vp, &parts, &quads, &scale, &dkp, &dvp};
      e = hipLaunchKernel((const void*)&bwd_part_sum_f32_kernel,
                          dim3((unsigned)((quads + 255) / 256)), dim3(256), p3, 0, s);
      if (e != hipSuccess) return e;
    }
  }
  int n_qt = (a.nq + kRows - 1) / kRows;
  int total_q = (int)((int64_t)n_qt * a.bh);
  if (total_q > 0) {
    void* p2[] = {&args, &n_qt, &total_q};
    e = hipLaunchKernel((const void*)&bwd_dq_f32_kernel<CAUSAL, D>, dim3(total_q),
                        dim3(kThreads), p2, 0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd_f32(int d, bool causal, const BwdArgs& a, const void* o, float* delta,
                          hipStream_t s) {
  if (d == 64) return causal ? launch<true, 64>(a, o, delta, s) : launch<false, 64>(a, o, delta, s);
  return causal ? launch<true, 128>(a, o, delta, s) : launch<false, 128>(a, o, delta, s);
}

}  // namespace fa_impl
