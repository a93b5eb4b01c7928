// fa_bwd_h16.hip -- FlashAttention backward pass, bf16 / fp16 inputs, fp32
// accumulate, for MI355X (gfx950).
//
// The attention weights are never stored: they are recomputed from Q, K and
// the forward pass's logsumexp ("FlashAttention dissected", section "Memory
// complexity: from O(N^2) to O(N)": the backward pass recomputes the blocks
// it needs from Q, K, V and the saved softmax statistics).  With
// P_ij = exp(scale q_i.k_j - LSE_i) (0 where masked):
//     D_i   = dO_i . O_i
//     dS_ij = P_ij (dO_i . v_j - D_i)
//     dV_j  = sum_i P_ij dO_i
//     dK_j  = scale sum_i dS_ij q_i
//     dQ_i  = scale sum_j dS_ij k_j
// Three kernels, no atomics (the result is bitwise reproducible):
//   * bwd_delta_kernel: D_i, one row per d/8 lanes, v_dot2 on the stored pairs;
//   * bwd_dkdv_kernel: a workgroup owns 128 keys (four waves x 32), keeps its
//     K and V fragments in registers and streams 32-query tiles of Q and dO
//     through double-buffered LDS, row-major: S = Q K^T and dP = dO V^T read
//     them as A operands (their accumulators give every lane one key), and
//     dV^T += dO^T P, dK^T += Q^T dS read the transposed operands straight
//     from the same rows with the LDS transpose load, in the query order in
//     which the P and dS accumulators are, unchanged, the B operands.  The
//     Q and dO tiles go HBM -> LDS directly, two stages deep, in unpadded
//     swizzled rows (row_swz), and at d = 128 the V rows wait in LDS in the
//     same layout (against register staging into padded rows: C3 backward
//     1.99 -> 1.91 ms, C5 3.69 -> 3.55, G2 1.94 -> 1.89; at d = 64 within
//     1 %);
//   * bwd_dq_kernel: the forward kernel's shape: a workgroup owns 128 (d = 128)
//     or 256 (d = 64, two 32-query blocks per wave) queries (Q and dO
//     fragments in registers, one query per lane in S^T = K Q^T and
//     dP^T = V dO^T) and streams 32-key tiles of K and V (row-major); dS^T is
//     the B operand of dQ^T += K^T dS^T, whose K^T operand comes from the K
//     rows through the transpose load.  The tiles go HBM -> LDS directly,
//     three stages deep, in unpadded swizzled rows (row_swz): the
//     single-buffered register staging sat on the critical path (C3 backward
//     2.06 -> 1.99 ms, C5 3.76 -> 3.70, G2 1.96 -> 1.92; at d = 64 against
//     double-buffered staging into padded rows, C4 3.63 -> 3.58).
// Causal masking, ragged tails and the -inf guard follow the forward kernels.
#include <type_traits>

#include "fa_bwd.hpp"
#include "fa_lds_dma.hpp"
#include "fa_h16.hpp"

namespace fa_impl {
namespace {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdRows = 32 * kBwdWaves;  // keys (dK/dV) or queries (dQ) per workgroup
constexpr int kBT = 32;                   // rows of a streamed tile

// Slot swizzle of a tile row of D bf16/fp16 columns: 256-byte rows
// (d = 128) take chunk_swz; 128-byte rows (d = 64, 8 chunks) take
// (r1, r0 ^ r2, r0 ^ r3), which keeps both the 16-row reads and the
// transpose reads free of bank conflicts.
template <int D>
__device__ __forceinline__ int row_swz(int r) {
  if constexpr (D == 128)
    return chunk_swz(r);
  else
    return (((r >> 1) & 1) << 2) | (((r ^ (r >> 2)) & 1) << 1) | ((r ^ (r >> 3)) & 1);
}
constexpr float kLog2e = 1.44269504088896340736f;

// Waves per SIMD that the register allocation must leave room for.  Both
// kernels keep a wave's rows (K and V, or Q and dO) and its gradient
// accumulators in registers.  At d = 128 the dK/dV kernel would need a few
// more than half the register file; its V rows wait in LDS instead, so that
// two waves share a SIMD without spills (two waves instead of one are worth
// +37-51 %: one wave's exponentials and packing hide under the other's
// MFMAs).  At d = 64 the dK/dV kernel runs three waves per SIMD.
template <int D> constexpr int kDkdvWaves = D == 64 ? 3 : 2;
template <int D> constexpr int kDqWaves = 2;
// 32-query blocks per wave in the dQ kernel, and queries per workgroup.  At
// d = 64 two blocks share every K and V operand read from LDS (half the LDS
// reads per MFMA, like the forward's two row blocks) at two waves per SIMD
// instead of three: 1-1.5 % faster backward (C4, G1).
template <int D> constexpr int kDqBlocks = D == 64 ? 2 : 1;
template <int D> constexpr int kDqRows = 32 * kBwdWaves * kDqBlocks<D>;
#ifndef FA_BWD_DQ_SHORT_GRID
#define FA_BWD_DQ_SHORT_GRID 256
#endif
constexpr int64_t kDqShortGrid = FA_BWD_DQ_SHORT_GRID;

// logsumexp in exp2 units; a row without a visible key (LSE = -inf) gets +inf
// so that every weight exp2(s c - lse2) is 0 instead of inf.
__device__ __forceinline__ float lse_log2(float lse) {
  return lse == kNegInf ? __builtin_inff() : lse * kLog2e;
}

// ---------------------------------------------------------------------------
// D_i = dO_i . O_i
// ---------------------------------------------------------------------------
template <bool BF16, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const uint16_t* __restrict__ o,
                                                        const uint16_t* __restrict__ dout,
                                                        float* __restrict__ delta,
                                                        int64_t rows) {
  using HH = Half<BF16>;
  constexpr int kLanes = D / 8;
  constexpr int kRowsPerBlock = 256 / kLanes;
  const int sub = threadIdx.x % kLanes;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanes;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 x = *(const u32x4*)(o + row * D + sub * 8);
    const u32x4 y = *(const u32x4*)(dout + row * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc = HH::dot2(x[e], y[e], acc);
  }
#pragma unroll
  for (int off = kLanes / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && sub == 0) delta[row] = acc;
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup per (128 keys, K/V head, head part).  With grouped
// heads the workgroup walks the query tiles of every query head of its part
// (the whole group with one part) in turn and sums their contributions in
// its registers; several parts write fp32 partials that bwd_part_sum_kernel
// adds in part order (no atomics: deterministic).
// ---------------------------------------------------------------------------
template <bool BF16, bool CAUSAL, int D>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(kDkdvWaves<D>))) void bwd_dkdv_kernel(BwdArgs a) {
  using HH = Half<BF16>;
  // Q and dO tiles go HBM -> LDS directly into two stages of unpadded
  // swizzled rows (row_swz, fa_lds_dma.hpp)
  constexpr int kTileElems = kBT * D;
  constexpr int kDmaPer = kTileElems * 2 / (kBwdThreads * 16);  // loads per thread per tile
  static_assert(kDmaPer * kBwdThreads * 16 == kTileElems * 2 && kBwdWaves % 4 == 0,
                "DMA tile split");
  // At d = 128 the V rows of the workgroup's keys wait in LDS (see below).
  constexpr bool kVLds = D == 128;
  // One LDS array holds the Q / dO stages, the V rows and the per-query
  // statistics [stage][lse2, D][query].  (With several arrays the compiler
  // tags the direct loads with an alias scope, and then makes every LDS read
  // after one wait for it.)  The statistics are aligned to their size, so
  // that an offset inside them can be applied as an XOR.
  constexpr int kQgBytes = 2 * 2 * kTileElems * 2;
  constexpr int kVBytes = kVLds ? kBwdRows * D * 2 : 0;
  constexpr int kStatBytes = 2 * 2 * kBT * 4;
  static_assert((kQgBytes + kVBytes) % kStatBytes == 0 && kQgBytes % 1024 == 0, "LDS regions");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[kQgBytes + kVBytes + kStatBytes];
  uint16_t* const lds = (uint16_t*)smem;
  uint16_t* const vlds = (uint16_t*)(smem + kQgBytes);
  float(*const stat)[2][kBT] = (float(*)[2][kBT])(smem + kQgBytes + kVBytes);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, grp = lane >> 5;
  const int nq = a.nq, nk = a.nk, off = a.off;

  // Workgroup -> (key tile, K/V head, part of the group's query heads), key
  // tiles outermost: under causal masking the low key tiles see the most
  // queries, and dispatching them first lets the light ones fill in behind.
  // Consecutive workgroups (same key tile) land on consecutive XCDs, so with
  // a multiple of 8 (head, part) units each unit stays on one XCD.
  const int units = a.bkv * a.hsplit;
  const int kt = blockIdx.x / units;
  const int unit = blockIdx.x - kt * units;
  const int bkv = unit / a.hsplit, sp = unit - bkv * a.hsplit;
  const int k0 = kt * kBwdRows;
  const int kw0 = k0 + wave * 32;  // this wave's first key
  const int b = bkv / a.hkv;
  const int h_lo = sp * a.hgrp / a.hsplit, h_hi = (sp + 1) * a.hgrp / a.hsplit;
  const int bh0 = b * a.hq + (bkv - b * a.hkv) * a.hgrp + h_lo;  // first query head of the part

  const int64_t kvhead = (int64_t)bkv * nk * D;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const uint16_t*)a.k + kvhead, nk * D * 2);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const uint16_t*)a.v + kvhead, nk * D * 2);

  // K and V rows of this wave's keys as B operands: lane (col, grp) holds
  // row kw0 + col, columns 16 kc + 8 grp .. + 8 (zero past the end).  At
  // d = 128 the V rows wait in LDS instead (each wave reads back only its own
  // rows, so no barrier is needed): 32 registers fewer, which keeps the
  // kernel from spilling at two waves per SIMD.
  // Unpadded 256-byte rows with the chunk swizzle (lane (col, grp) reads
  // row wave * 32 + col, chunk (2 kc + grp) ^ chunk_swz(col), i.e. one base
  // XOR 32 kc: conflict-free like the Q and dO row reads).
  const int vrow_off = kVLds ? ((wave * 32 + col) * D * 2 + 16 * (grp ^ chunk_swz(col))) : 0;
  u32x4 kf[D / 16], vf[kVLds ? 1 : D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) {
    kf[kc] = buf_load16(kr, ((kw0 + col) * D + kc * 16 + grp * 8) * 2);
    const u32x4 x = buf_load16(vr, ((kw0 + col) * D + kc * 16 + grp * 8) * 2);
    if constexpr (kVLds)
      *(u32x4*)((char*)vlds + (vrow_off ^ (32 * kc))) = x;
    else
      vf[kc] = x;
  }

  // Query tiles qt_begin .. n_qt - 1 of each of the hgrp query heads, walked
  // as one sequence (head by head, tiles upward).  Causal: a query row i sees
  // key k0 only if i + off >= k0, so earlier tiles see none of these keys.
  const int n_qt = (nq + kBT - 1) / kBT;
  const int qt_begin = CAUSAL ? max(0, (k0 - off) / kBT) : 0;
  const int n_iter = max(0, n_qt - qt_begin);
  const int total_it = n_iter * (h_hi - h_lo);

  float st = 0.f;  // this thread's lse or D value of the next tile

  // Direct loads of the Q and dO tile of (query head hh, rows q0 ..) into
  // stage `stage`: wave w's load i fills the kLoadRows rows from
  // kLoadRows (4 i + w) on, lane l the 16 bytes at l * 16 of that block,
  // fetching the chunk the swizzle puts there.  The tile's lse and D values still go through a register
  // (load_stat / store_stat: they are transformed on the way).
  constexpr int kChunks = D / 8;           // 16-byte chunks per tile row
  constexpr int kLoadRows = 64 / kChunks;  // tile rows one wave's load fills
  const int dma_row = kLoadRows * wave + lane / kChunks;
  const int dma_off = dma_row * D * 2 + 16 * ((lane % kChunks) ^ row_swz<D>(dma_row));
  // The resources start at the tile's first row and end with the head, so
  // that the per-lane offsets stay loop-invariant and rows past the end
  // still read as zeros (the range check covers the per-lane offset only).
  auto dma_tile = [&](int hh, int q0, int stage) {
    const int64_t row0 = (bh0 + hh) * (int64_t)nq + q0;
    const int bytes = (nq - q0) * D * 2;
    const __amdgpu_buffer_rsrc_t qr = make_rsrc((const uint16_t*)a.q + row0 * D, bytes);
    const __amdgpu_buffer_rsrc_t gr = make_rsrc((const uint16_t*)a.dout + row0 * D, bytes);
    uint16_t* qt_ = lds + stage * 2 * kTileElems;
    uint16_t* gt_ = qt_ + kTileElems;
#pragma unroll
    for (int i = 0; i < kDmaPer; ++i) {
      const int rows = kLoadRows * (i * kBwdWaves + wave);
      buf_load16_lds(qr, qt_ + rows * D, dma_off + i * kBwdWaves * 1024);
      buf_load16_lds(gr, gt_ + rows * D, dma_off + i * kBwdWaves * 1024);
    }
  };
  auto load_stat = [&](int hh, int q0) {
    const int64_t bhq = bh0 + hh;
    const __amdgpu_buffer_rsrc_t lr = make_rsrc(a.lse + bhq * nq, nq * 4);
    const __amdgpu_buffer_rsrc_t dr = make_rsrc(a.delta + bhq * nq, nq * 4);
    if (tid < kBT)
      st = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lr, (q0 + tid) * 4, 0, 0));
    else if (tid < 2 * kBT)
      st = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(dr, (q0 + tid - kBT) * 4, 0, 0));
  };
  auto store_stat = [&](int buf) {
    if (tid < 2 * kBT) stat[buf][tid / kBT][tid % kBT] = tid < kBT ? lse_log2(st) : -st;
  };
  // LDS byte offsets of this lane's operands inside a DMA stage: Q and dO
  // rows (row col, chunk 2 kc + grp; the 2 kc part applied per read as an
  // XOR of 32 kc) and the transposed Q^T / dO^T reads (rows 4 grp +
  // (lane % 16) / 4 and that + 8 of each 16-query chunk, bytes 64 db +
  // 32 ((lane / 16) % 2) + 8 (lane % 4); the 64 db part applied as an XOR).
  // The reads go through LDS byte addresses, with the swizzled part and
  // the per-read offsets applied as XORs on aligned bases.  The bases pass
  // through an empty asm, which keeps the compiler from folding them back
  // into per-read address arithmetic (more instructions and registers).
  uint32_t stat_b = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) float*)&stat[0][0][0];
  uint32_t vrow_b = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)vlds + vrow_off;
  uint32_t lds_b = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)lds;
  asm("" : "+v"(stat_b), "+v"(vrow_b), "+v"(lds_b));
  auto lds_f32x4 = [](uint32_t addr) {
    return *(const __attribute__((address_space(3))) f32x4*)(uintptr_t)addr;
  };
  const int trow = 4 * grp + ((lane & 15) >> 2);
  const int tx = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const uint32_t r_off = col * D * 2 + 16 * (grp ^ row_swz<D>(col));
  const uint32_t t_off0 = trow * D * 2 + 16 * (tx ^ row_swz<D>(trow)) + 8 * (lane & 1);
  const uint32_t t_off1 = (trow + 8) * D * 2 + 16 * (tx ^ row_swz<D>(trow + 8)) + 8 * (lane & 1);

  const float c = a.scale_log2;
  f32x16 dkT[D / 32], dvT[D / 32];  // dK^T, dV^T: lane holds key kw0 + col
#pragma unroll
  for (int db = 0; db < D / 32; ++db) dkT[db] = dvT[db] = (f32x16){};

  if (total_it > 0) {
    dma_tile(0, qt_begin * kBT, 0);
    load_stat(0, qt_begin * kBT);
  }
  __builtin_amdgcn_s_waitcnt(kVmcntWait<0>);
  if (total_it > 0) store_stat(0);
  __syncthreads();
  // nothing is pending on any path into the loop (the compiler merges the
  // two total_it tests above and would leave the K fragments "pending" on
  // the path that skips them, then wait for them inside every iteration)
  __builtin_amdgcn_s_waitcnt(kVmcntWait<0>);

  int hh = 0, qt = qt_begin;  // query head (within the group) and tile of step `it`
  for (int it = 0; it < total_it; ++it) {
    const int buf = it & 1;
    const int q0 = qt * kBT;
    const bool more = it + 1 < total_it;
    const bool wrap = qt + 1 == n_qt;
    const int hh_next = wrap ? hh + 1 : hh;
    const int q0_next = (wrap ? qt_begin : qt + 1) * kBT;
    // the next tile goes to the other stage, read last in the previous
    // iteration (the barrier at its end has passed)
    if (more) {
      dma_tile(hh_next, q0_next, buf ^ 1);
      load_stat(hh_next, q0_next);
    }

    // causal: a tile whose last query sees none of this wave's keys is empty
    const bool active = !(CAUSAL && q0 + kBT - 1 + off < kw0);
    const uint32_t stage_b = lds_b + buf * 2 * kTileElems * 2;
    const uint32_t qr_b = stage_b + r_off, gr_b = stage_b + kTileElems * 2 + r_off;
    const uint32_t qt0_b = stage_b + t_off0, qt1_b = stage_b + t_off1;
    const uint32_t gt0_b = qt0_b + kTileElems * 2, gt1_b = qt1_b + kTileElems * 2;

    // S = Q K^T and dP - D = dO V^T - D: lane holds key kw0 + col of the
    // queries q0 + 8 (r/4) + 4 grp + r%4; the dP product starts from -D, so
    // that dS = P (dP - D) is one multiply per score.
    f32x16 s = {}, dp = {};
    if (active) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 nd = lds_f32x4(stat_b ^ (((buf * 2 + 1) * kBT + 8 * j + 4 * grp) * 4));
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * j + e] = nd[e];
      }
      // the 2 D / 16 MFMAs of S and dP as one sequence, each operand read
      // from LDS two MFMAs ahead of its use (the barriers keep the
      // scheduler from sinking the reads to their uses)
      constexpr int KC = D / 16;
      auto rd_a = [&](int op) {
        return *(const lds_u32x4*)(uintptr_t)((op < KC ? qr_b : gr_b) ^ (32u * (op % KC)));
      };
      auto rd_b = [&](int op) {
        return *(const lds_u32x4*)(uintptr_t)(vrow_b ^ (32u * (op - KC)));
      };
      u32x4 ra[2], rb[2];
      ra[0] = rd_a(0);
      ra[1] = rd_a(1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int op = 0; op < 2 * KC; ++op) {
        const u32x4 a_ = ra[op % 2];
        u32x4 b_;
        if constexpr (kVLds)
          b_ = op < KC ? kf[op % KC] : rb[op % 2];
        else
          b_ = op < KC ? kf[op % KC] : vf[op % KC];
        if (op + 2 < 2 * KC) {
          ra[op % 2] = rd_a(op + 2);
          if (kVLds && op + 2 >= KC) rb[op % 2] = rd_b(op + 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (op < KC)
          s = HH::mfma(a_, b_, s);
        else
          dp = HH::mfma(a_, b_, dp);
        __builtin_amdgcn_sched_barrier(0);
      }

    }

    // Only the causal mask is applied.  A query row past the end has zero Q
    // and dO rows and a zero lse and D (the buffer range check), so its
    // weights are finite and add exact zeros; a key past the end only
    // touches its own dK/dV column, which is never stored.  Register r holds
    // query q0 + 8 (r/4) + 4 grp + r%4, so key > query + off reads
    // kq0 > 8 (r/4) + r%4 with one per-lane offset kq0.
    const bool diag = CAUSAL && q0 + off < kw0 + 31;  // the tile crosses this wave's diagonal
    const int kq0 = kw0 + col - q0 - off - 4 * grp;
    // One 16-query chunk at a time (registers 8 ch .. 8 ch + 7): P, dS,
    // their packed pairs, then dV^T += dO^T P and dK^T += Q^T dS for the
    // chunk, so only one chunk's weights are live.
    // The masked form is its own wave-uniform branch, taken only by diagonal
    // tiles (folded into every tile, the test would add two VALU
    // instructions per score).
    auto weights = [&](auto masked, int ch, uint32_t* pp, uint32_t* pd) {
      constexpr bool M = decltype(masked)::value;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = 2 * ch + jj;
        const f32x4 l4 = lds_f32x4(stat_b ^ (((buf * 2 + 0) * kBT + 8 * j + 4 * grp) * 4));
        float pv[4], dsv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * j + e;
          float p = fast_exp2(fmaf(s[r], c, -l4[e]));
          if (CAUSAL && M) p = kq0 > 8 * j + e ? 0.f : p;
          pv[e] = p;
          dsv[e] = p * dp[r];
        }
        pp[2 * jj] = HH::pack(pv[0], pv[1]);
        pp[2 * jj + 1] = HH::pack(pv[2], pv[3]);
        pd[2 * jj] = HH::pack(dsv[0], dsv[1]);
        pd[2 * jj + 1] = HH::pack(dsv[2], dsv[3]);
      }
    };
    auto chunk = [&](auto chc) {
      const int ch = chc;
      uint32_t pp[4], pd[4];
      if (diag)
        weights(std::true_type{}, ch, pp, pd);
      else
        weights(std::false_type{}, ch, pp, pd);
      const u32x4 bp = {pp[0], pp[1], pp[2], pp[3]};
      const u32x4 bd = {pd[0], pd[1], pd[2], pd[3]};
      // dO^T and Q^T by transpose reads in inline assembly (the
      // compiler's own transpose-load intrinsic would wait for every load
      // into LDS in flight), each d block's four reads issued two blocks
      // ahead of its MFMAs; the scheduling barriers keep the MFMAs from
      // sinking below later waits
      auto tread = [&](int db, u32x2 (&r)[4]) {
        constexpr int o = decltype(chc)::value * 16 * D * 2;
        r[0] = lds_read_tr16_b64<o>(gt0_b ^ (64u * db));
        r[1] = lds_read_tr16_b64<o>(gt1_b ^ (64u * db));
        r[2] = lds_read_tr16_b64<o>(qt0_b ^ (64u * db));
        r[3] = lds_read_tr16_b64<o>(qt1_b ^ (64u * db));
      };
      auto tmma = [&](int db, const u32x2 (&r)[4]) {
        const u32x4 ga = {r[0][0], r[0][1], r[1][0], r[1][1]};
        const u32x4 qa = {r[2][0], r[2][1], r[3][0], r[3][1]};
        dvT[db] = HH::mfma(ga, bp, dvT[db]);
        dkT[db] = HH::mfma(qa, bd, dkT[db]);
      };
      if constexpr (D / 32 == 2) {
        u32x2 r0[4], r1[4];
        tread(0, r0);
        tread(1, r1);
        __builtin_amdgcn_sched_barrier(0);
        lds_wait_keep4(r0[0], r0[1], r0[2], r0[3]);
        tmma(0, r0);
        __builtin_amdgcn_sched_barrier(0);
        lds_wait_all(r1[0], r1[1], r1[2], r1[3]);
        tmma(1, r1);
      } else {
      static_assert(D / 32 == 4, "two or four d blocks");
      u32x2 r0[4], r1[4], r2[4];
      tread(0, r0);
      tread(1, r1);
      __builtin_amdgcn_sched_barrier(0);
      lds_wait_keep4(r0[0], r0[1], r0[2], r0[3]);
      tread(2, r2);
      tmma(0, r0);
      __builtin_amdgcn_sched_barrier(0);
      lds_wait_keep4(r1[0], r1[1], r1[2], r1[3]);
      tread(3, r0);
      tmma(1, r1);
      __builtin_amdgcn_sched_barrier(0);
      lds_wait_keep4(r2[0], r2[1], r2[2], r2[3]);
      tmma(2, r2);
      __builtin_amdgcn_sched_barrier(0);
      lds_wait_all(r0[0], r0[1], r0[2], r0[3]);
      tmma(3, r0);
      }

    };
    if (active) {
      chunk(std::integral_constant<int, 0>{});
      chunk(std::integral_constant<int, 1>{});
    }
    if (more) store_stat(buf ^ 1);
    // the next tile's loads have landed (this thread's share) before the
    // barrier that hands the stage over
    __builtin_amdgcn_s_waitcnt(kVmcntWait<0>);
    __syncthreads();
    hh = hh_next;
    qt = wrap ? qt_begin : qt + 1;
  }

  // dK = scale * (Q^T dS)^T, dV = (dO^T P)^T; lane holds key kw0 + col.
  const int key = kw0 + col;
  if (a.hsplit > 1) {
    // this part's sums, fp32 and unscaled, for the reduce kernel
    if (key < nk) {
      const int64_t row = ((int64_t)sp * a.bkv + bkv) * nk + key;
      float* dkp = a.dk_part + row * D;
      float* dvp = a.dv_part + row * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d0 = db * 32 + 8 * j + 4 * grp;
          *(f32x4*)(dkp + d0) = (f32x4){dkT[db][4 * j], dkT[db][4 * j + 1], dkT[db][4 * j + 2],
                                        dkT[db][4 * j + 3]};
          *(f32x4*)(dvp + d0) = (f32x4){dvT[db][4 * j], dvT[db][4 * j + 1], dvT[db][4 * j + 2],
                                        dvT[db][4 * j + 3]};
        }
    }
  } else if (key < nk) {
    uint16_t* dkg = (uint16_t*)a.dk + kvhead + (int64_t)key * D;
    uint16_t* dvg = (uint16_t*)a.dv + kvhead + (int64_t)key * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = db * 32 + 8 * j + 4 * grp;
        const u32x2 wk = {HH::pack(dkT[db][4 * j] * a.scale, dkT[db][4 * j + 1] * a.scale),
                          HH::pack(dkT[db][4 * j + 2] * a.scale, dkT[db][4 * j + 3] * a.scale)};
        const u32x2 wv = {HH::pack(dvT[db][4 * j], dvT[db][4 * j + 1]),
                          HH::pack(dvT[db][4 * j + 2], dvT[db][4 * j + 3])};
        *(u32x2*)(dkg + d0) = wk;
        *(u32x2*)(dvg + d0) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup per (query head, kDqRows queries)
// ---------------------------------------------------------------------------
// QB_: 32-row query blocks per wave (kDqBlocks by default; one for the short
// d = 64 grids below).
template <bool BF16, bool CAUSAL, int D, int QB_ = kDqBlocks<D>>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(kDqWaves<D>))) void bwd_dq_kernel(BwdArgs a, int n_qt, int total) {
  using HH = Half<BF16>;
  constexpr int QB = QB_;
  constexpr int kRows = 32 * kBwdWaves * QB;
  // K and V tiles loaded HBM -> LDS directly into three stages of unpadded
  // swizzled rows (row_swz)
  constexpr int kTileElems = kBT * D;
  constexpr int kDmaPer = kTileElems * 2 / (kBwdThreads * 16);  // loads per thread per tile
  static_assert(kDmaPer * kBwdThreads * 16 == kTileElems * 2 && kBwdWaves % 4 == 0,
                "DMA tile split");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[3 * 2 * kTileElems];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, grp = lane >> 5;
  const int nq = a.nq, nk = a.nk, off = a.off;

  const int L = xcd_remap(blockIdx.x, total);
  int bh, qt;
  tile_of<CAUSAL>(L, total, n_qt, bh, qt);
  const int q0 = qt * kRows;
  const int qw0 = q0 + wave * 32 * QB;  // block qb: queries qw0 + 32 qb .. + 31
  const int b = bh / a.hq;
  const int bkv = b * a.hkv + (bh - b * a.hq) / a.hgrp;  // this query head's K/V head

  const int64_t qhead = (int64_t)bh * nq * D, kvhead = (int64_t)bkv * nk * D;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc((const uint16_t*)a.q + qhead, nq * D * 2);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const uint16_t*)a.k + kvhead, nk * D * 2);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const uint16_t*)a.v + kvhead, nk * D * 2);
  const __amdgpu_buffer_rsrc_t gr = make_rsrc((const uint16_t*)a.dout + qhead, nq * D * 2);
  const __amdgpu_buffer_rsrc_t lr = make_rsrc(a.lse + (int64_t)bh * nq, nq * 4);
  const __amdgpu_buffer_rsrc_t dr = make_rsrc(a.delta + (int64_t)bh * nq, nq * 4);

  // causal: row i sees keys j <= i + off
  const int kv_end = CAUSAL ? max(0, min(q0 + kRows + off, nk)) : nk;
  const int n_kv = (kv_end + kBT - 1) / kBT;
  const int wave_kv_end = CAUSAL ? max(0, min(qw0 + 32 * QB + off, nk)) : nk;

  // Direct HBM -> LDS loads: wave w's load i fills the kLoadRows tile rows
  // from kLoadRows (4 i + w) on, lane l the 16 bytes at l * 16 of that
  // block, fetching the chunk the swizzle puts there.
  constexpr int kChunks = D / 8;           // 16-byte chunks per tile row
  constexpr int kLoadRows = 64 / kChunks;  // tile rows one wave's load fills
  const int dma_row = kLoadRows * wave + lane / kChunks;
  const int dma_off = dma_row * D * 2 + 16 * ((lane % kChunks) ^ row_swz<D>(dma_row));
  auto dma_tile = [&](int k0, int stage) {
    uint16_t* kt = lds + stage * 2 * kTileElems;
    uint16_t* vt = kt + kTileElems;
    const int g = k0 * D * 2 + dma_off;
#pragma unroll
    for (int i = 0; i < kDmaPer; ++i) {
      const int rows = kLoadRows * (i * kBwdWaves + wave);
      buf_load16_lds(kr, kt + rows * D, g + i * kBwdWaves * 1024);
      buf_load16_lds(vr, vt + rows * D, g + i * kBwdWaves * 1024);
    }
  };
  if (n_kv > 0) dma_tile(0, 0);

  // Q and dO rows of this lane's queries as B operands.
  u32x4 qf[QB][D / 16], gf[QB][D / 16];
  float lse2[QB], drow[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int my_q = qw0 + 32 * qb + col;
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc) {
      qf[qb][kc] = buf_load16(qr, (my_q * D + kc * 16 + grp * 8) * 2);
      gf[qb][kc] = buf_load16(gr, (my_q * D + kc * 16 + grp * 8) * 2);
    }
    lse2[qb] = lse_log2(
        __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(lr, my_q * 4, 0, 0)));
    drow[qb] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(dr, my_q * 4, 0, 0));
  }
  // With one block per wave the dP product starts from -D of the lane's row
  // (16 registers), so that dS = P (dP - D) is one multiply; with two blocks
  // the registers go to the second block and dS takes a subtract as well.
  f32x16 ndrow = {};
  if constexpr (QB == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) ndrow[r] = -drow[0];
  }

  const float c = a.scale_log2;
  f32x16 dqT[QB][D / 32];  // dQ^T: lane holds query qw0 + 32 qb + col
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) dqT[qb][db] = (f32x16){};

  // LDS byte offsets of this lane's operands inside a stage: K and V
  // rows (row col, chunk 2 kc + grp; the 2 kc part applied per read as an
  // XOR of 32 kc) and the transposed K^T reads (rows 4 grp + (lane % 16) / 4
  // and that + 8 of each 16-key chunk, bytes 64 db + 32 ((lane / 16) % 2) +
  // 8 (lane % 4); the 64 db part applied per read as an XOR)
  const int trow = 4 * grp + ((lane & 15) >> 2);
  const int tx = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const uint32_t r_off = col * D * 2 + 16 * (grp ^ row_swz<D>(col));
  const uint32_t t_off0 = trow * D * 2 + 16 * (tx ^ row_swz<D>(trow)) + 8 * (lane & 1);
  const uint32_t t_off1 = (trow + 8) * D * 2 + 16 * (tx ^ row_swz<D>(trow + 8)) + 8 * (lane & 1);

  // tile 0 went out before Q; tile 1 now; everything (Q, dO, lse, D
  // included) waited for here, once, as in the forward
  if (n_kv > 1) dma_tile(kBT, 1);
  __builtin_amdgcn_s_waitcnt(kVmcntWait<0>);

  for (int t = 0; t < n_kv; ++t) {
    const int k0 = t * kBT;
    const bool more = t + 1 < n_kv;
    // this thread's loads of tile t landed once at most tile t + 1's are
    // in flight; the barrier makes every thread's share visible and says
    // that tile t - 1 (whose stage tile t + 2 overwrites) is done
    if (more)
      __builtin_amdgcn_s_waitcnt(kVmcntWait<2 * kDmaPer>);
    else
      __builtin_amdgcn_s_waitcnt(kVmcntWait<0>);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (t + 2 < n_kv) dma_tile(k0 + 2 * kBT, (t + 2) % 3);
    const int buf = t % 3;

    if (k0 < wave_kv_end) {
      const uint32_t stage_b =
          (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)(lds + buf * 2 * kTileElems);
      const uint32_t kr_b = stage_b + r_off, vr_b = stage_b + kTileElems * 2 + r_off;
      const uint32_t kt0_b = stage_b + t_off0, kt1_b = stage_b + t_off1;

      // S^T = K Q^T and dP^T (- D) = V dO^T (- D) for every block: lane
      // holds query qw0 + 32 qb + col, keys k0 + 8 (r/4) + 4 grp + r%4.  Each
      // K or V operand read from LDS feeds the products of all blocks.
      f32x16 s[QB], dp[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        s[qb] = (f32x16){};
        dp[qb] = QB == 1 ? ndrow : (f32x16){};
      }
      {
        // the 2 D / 16 MFMA steps of S and dP as one sequence, each K or V
        // operand read from LDS two steps ahead of its use (as in the dK/dV
        // kernel) and fed to the products of every block
        constexpr int KC = D / 16;
        auto rd = [&](int op) {
          return *(const lds_u32x4*)(uintptr_t)((op < KC ? kr_b : vr_b) ^ (32u * (op % KC)));
        };
        u32x4 ra[2];
        ra[0] = rd(0);
        ra[1] = rd(1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int op = 0; op < 2 * KC; ++op) {
          const u32x4 a_ = ra[op % 2];
          if (op + 2 < 2 * KC) ra[op % 2] = rd(op + 2);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            if (op < KC)
              s[qb] = HH::mfma(a_, qf[qb][op % KC], s[qb]);
            else
              dp[qb] = HH::mfma(a_, gf[qb][op % KC], dp[qb]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // dS^T = P^T (dP^T - D).  The masked form runs only on diagonal and
      // ragged tiles, as its own wave-uniform branch.  Register r holds key
      // k0 + 8 (r/4) + 4 grp + r%4, so the key is masked (past the end, or
      // after the row's last visible key) when 8 (r/4) + r%4 exceeds one
      // per-lane limit.
      // The K^T operands of d blocks 0 and 1 (transpose reads in inline
      // assembly: the compiler would make its own transpose-load intrinsic
      // wait for every load into LDS in flight) are read while the weights
      // are formed, each later block's two blocks ahead of its MFMAs.
      auto tread = [&](int db, u32x2 (&r)[2][2]) {
        const uint32_t a0 = kt0_b ^ (64u * db), a1 = kt1_b ^ (64u * db);
        r[0][0] = lds_read_tr16_b64<0>(a0);
        r[0][1] = lds_read_tr16_b64<0>(a1);
        r[1][0] = lds_read_tr16_b64<16 * D * 2>(a0);
        r[1][1] = lds_read_tr16_b64<16 * D * 2>(a1);
      };
      u32x2 r0[2][2], r1[2][2], r2[2][2];
      tread(0, r0);
      tread(1, r1);
      __builtin_amdgcn_sched_barrier(0);
      uint32_t pd[QB][8];
      auto weights = [&](auto masked, int qb) {
        const int my_q = qw0 + 32 * qb + col;
        const int last = CAUSAL ? min(nk - 1, my_q + off) : nk - 1;
        const int lim = last - k0 - 4 * grp;
        float dsv[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(s[qb][r], c, -lse2[qb]));
          if constexpr (decltype(masked)::value) p = 8 * (r >> 2) + (r & 3) > lim ? 0.f : p;
          dsv[r] = QB == 1 ? p * dp[qb][r] : p * (dp[qb][r] - drow[qb]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) pd[qb][i] = HH::pack(dsv[2 * i], dsv[2 * i + 1]);
      };
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if (k0 + kBT > nk || (CAUSAL && k0 + kBT - 1 > qw0 + 32 * qb + off))
          weights(std::true_type{}, qb);
        else
          weights(std::false_type{}, qb);
      }

      // dQ^T += K^T dS^T over the two 16-key chunks; each K^T operand feeds
      // every block.
      auto tmma = [&](int db, const u32x2 (&r)[2][2]) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const u32x4 ka = {r[ch][0][0], r[ch][0][1], r[ch][1][0], r[ch][1][1]};
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) {
            const u32x4 bd = {pd[qb][4 * ch], pd[qb][4 * ch + 1], pd[qb][4 * ch + 2],
                              pd[qb][4 * ch + 3]};
            dqT[qb][db] = HH::mfma(ka, bd, dqT[qb][db]);
          }
        }
      };
      // (the scheduling barriers keep the MFMAs from sinking below later
      // waits)
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (D / 32 == 2) {
        lds_wait_keep4(r0[0][0], r0[0][1], r0[1][0], r0[1][1]);
        tmma(0, r0);
        __builtin_amdgcn_sched_barrier(0);
        lds_wait_all(r1[0][0], r1[0][1], r1[1][0], r1[1][1]);
        tmma(1, r1);
      } else {
        static_assert(D / 32 == 4, "two or four d blocks");
        lds_wait_keep4(r0[0][0], r0[0][1], r0[1][0], r0[1][1]);
        tread(2, r2);
        tmma(0, r0);
        __builtin_amdgcn_sched_barrier(0);
        lds_wait_keep4(r1[0][0], r1[0][1], r1[1][0], r1[1][1]);
        tread(3, r0);
        tmma(1, r1);
        __builtin_amdgcn_sched_barrier(0);
        lds_wait_keep4(r2[0][0], r2[0][1], r2[1][0], r2[1][1]);
        tmma(2, r2);
        __builtin_amdgcn_sched_barrier(0);
        lds_wait_all(r0[0][0], r0[0][1], r0[1][0], r0[1][1]);
        tmma(3, r0);
      }
    }
  }

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int my_q = qw0 + 32 * qb + col;
    if (my_q < nq) {
      uint16_t* g = (uint16_t*)a.dq + qhead + (int64_t)my_q * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d0 = db * 32 + 8 * j + 4 * grp;
          const u32x2 w = {
              HH::pack(dqT[qb][db][4 * j] * a.scale, dqT[qb][db][4 * j + 1] * a.scale),
              HH::pack(dqT[qb][db][4 * j + 2] * a.scale, dqT[qb][db][4 * j + 3] * a.scale)};
          *(u32x2*)(g + d0) = w;
        }
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV from the parts of split head groups: the sum over parts in part
// order (deterministic), dK times scale, rounded to the I/O type.
// ---------------------------------------------------------------------------
template <bool BF16>
__global__ __launch_bounds__(256) void bwd_part_sum_kernel(const float* __restrict__ dk_part,
                                                           const float* __restrict__ dv_part,
                                                           int parts, int64_t quads, float scale,
                                                           uint16_t* __restrict__ dk,
                                                           uint16_t* __restrict__ dv) {
  using HH = Half<BF16>;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 4-float group
  if (i >= quads) return;
  f32x4 sk = *(const f32x4*)(dk_part + i * 4);
  f32x4 sv = *(const f32x4*)(dv_part + i * 4);
  for (int p = 1; p < parts; ++p) {
    sk += *(const f32x4*)(dk_part + (p * quads + i) * 4);
    sv += *(const f32x4*)(dv_part + (p * quads + i) * 4);
  }
  *(u32x2*)(dk + i * 4) = (u32x2){HH::pack(sk[0] * scale, sk[1] * scale),
                                  HH::pack(sk[2] * scale, sk[3] * scale)};
  *(u32x2*)(dv + i * 4) = (u32x2){HH::pack(sv[0], sv[1]), HH::pack(sv[2], sv[3])};
}

template <bool BF16, bool CAUSAL, int D>
hipError_t launch_bwd(const BwdArgs& a, const void* o, float* delta, hipStream_t s) {
  BwdArgs args = a;
  hipError_t e;
  // D_i = dO_i . O_i for every query row
  const int64_t rows = (int64_t)a.bh * a.nq;
  if (rows > 0) {
    constexpr int kRowsPerBlock = 256 / (D / 8);
    const uint16_t* op = (const uint16_t*)o;
    const uint16_t* gp = (const uint16_t*)a.dout;
    int64_t rows_arg = rows;
    void* p0[] = {&op, &gp, &delta, &rows_arg};
    e = hipLaunchKernel((const void*)&bwd_delta_kernel<BF16, D>,
                        dim3((unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock)), dim3(256),
                        p0, 0, s);
    if (e != hipSuccess) return e;
  }
  // dK, dV over the K/V heads' key tiles and head parts (zero when there are
  // no queries), then the sum of the parts
  int n_kt = (a.nk + kBwdRows - 1) / kBwdRows;
  int total_kv = (int)((int64_t)n_kt * a.bkv * a.hsplit);
  if (total_kv > 0) {
    void* p1[] = {&args};
    e = hipLaunchKernel((const void*)&bwd_dkdv_kernel<BF16, CAUSAL, D>, dim3(total_kv),
                        dim3(kBwdThreads), p1, 0, s);
    if (e != hipSuccess) return e;
    if (a.hsplit > 1) {
      const float* kp = a.dk_part;
      const float* vp = a.dv_part;
      int parts = a.hsplit;
      int64_t quads = (int64_t)a.bkv * a.nk * (D / 4);
      float scale = a.scale;
      uint16_t* dkp = (uint16_t*)a.dk;
      uint16_t* dvp = (uint16_t*)a.dv;
      void* p3[] = {&kp, &vp, &parts, &quads, &scale, &dkp, &dvp};
      e = hipLaunchKernel((const void*)&bwd_part_sum_kernel<BF16>,
                          dim3((unsigned)((quads + 255) / 256)), dim3(256), p3, 0, s);
      if (e != hipSuccess) return e;
    }
  }
  // dQ over the query heads' row tiles (zero when there are no keys).  A
  // d = 64 grid of fewer than kDqShortGrid 256-row workgroups takes 128-row
  // ones (one block per wave), twice as many.
  int n_qt = (a.nq + kDqRows<D> - 1) / kDqRows<D>;
  const void* dq_fn = (const void*)&bwd_dq_kernel<BF16, CAUSAL, D>;
  if constexpr (D == 64 && kDqBlocks<D> == 2) {
    if ((int64_t)n_qt * a.bh < kDqShortGrid) {
      n_qt = (a.nq + 32 * kBwdWaves - 1) / (32 * kBwdWaves);
      dq_fn = (const void*)&bwd_dq_kernel<BF16, CAUSAL, D, 1>;
    }
  }
  int total_q = (int)((int64_t)n_qt * a.bh);
  if (total_q > 0) {
    void* p2[] = {&args, &n_qt, &total_q};
    e = hipLaunchKernel(dq_fn, dim3(total_q), dim3(kBwdThreads), p2, 0, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <bool BF16, int D>
hipError_t launch_d(bool causal, const BwdArgs& a, const void* o, float* delta, hipStream_t s) {
  return causal ? launch_bwd<BF16, true, D>(a, o, delta, s)
                : launch_bwd<BF16, false, D>(a, o, delta, s);
}

}  // namespace

hipError_t launch_bwd_h16(bool bf16, int d, bool causal, const BwdArgs& a, const void* o,
                          float* delta, hipStream_t s) {
  if (bf16)
    return d == 64 ? launch_d<true, 64>(causal, a, o, delta, s)
                   : launch_d<true, 128>(causal, a, o, delta, s);
  return d == 64 ? launch_d<false, 64>(causal, a, o, delta, s)
                 : launch_d<false, 128>(causal, a, o, delta, s);
}

int64_t bwd_grid_blocks(int64_t bh, int64_t bkv, int64_t nq, int64_t nk, int64_t hsplit) {
  const int64_t kv = (nk + kBwdRows - 1) / kBwdRows * bkv * hsplit;
  const int64_t q = (nq + kBwdRows - 1) / kBwdRows * bh;
  const int64_t sum = hsplit > 1 ? (bkv * nk * 32 + 255) / 256 : 0;  // part-sum grid, d <= 128
  const int64_t m = kv > q ? kv : q;
  return m > sum ? m : sum;
}

int64_t bwd_dkdv_blocks(int64_t bkv, int64_t nk) { return (nk + kBwdRows - 1) / kBwdRows * bkv; }

}  // namespace fa_impl
