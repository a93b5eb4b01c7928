// fa_fwd_h16.hip -- FlashAttention forward, bf16 / fp16 inputs, fp32 accumulate,
// for MI355X (gfx950).
//
// What runs (one workgroup per (problem, query tile[, key range]); NW
// wave64s, each owning 32*QB query rows; the instance table at the end picks
// NW, QB and the key tile BN per head size, and a one-wave instance for
// problems of at most 32 rows, i.e. decoding steps):
//   * The query tile stays in registers for the whole key loop, as the
//     B operand of S^T = K Q^T (course lesson "FlashAttention Inner Loop
//     Implementation", section "Implementing the Inner Loop": Q is loaded
//     once and reused for every key/value step).
//   * K/V tiles are loaded by every thread of the workgroup (16-byte loads;
//     GitHub README "CUDA Flash Attention...", "Performance Analysis": the
//     K/V load must use all warps) while the previous tile is computed.
//     d = 64: staged HBM -> registers -> LDS, double buffered; K rows
//     padded by 16 bytes ("Design decisions": padded shared rows), V stored
//     transposed ([d][key]) with the key order permuted inside each 16-key
//     chunk, so each lane's operand for the P.V product is one 16-byte LDS
//     read.  d = 128: loaded HBM -> LDS directly (buffer loads with the LDS
//     bit: no staging registers, no LDS stores, no transposing permutes),
//     three stages deep with tile t+2 in flight while tile t is computed;
//     K and V both row-major, unpadded, 16-byte chunks XOR-swizzled per
//     row so that the K reads and the transposed V reads (ds_read_b64_tr_b16)
//     are free of bank conflicts.  The loads of a single-buffered tile sat
//     exposed on the critical path: +5-7 % on the d = 128 causal shapes.
//     The K and V^T operands are read from LDS two MFMAs ahead of their use
//     (+3-4 % together on the same shapes).
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16}: each lane ends up with
//     32 scores of ONE query (16 per 32-key block), the other 32 scores of
//     that query sit in the lane 32 positions away.  Row statistics are thus
//     an in-lane reduction plus one permlane32 swap.
//   * Online softmax ("FlashAttention dissected", "Algorithmic core in
//     pseudocode"): running reference max m and sum l per query row, in
//     registers; the scores enter exp2 with the scale folded into one FMA,
//     p = exp2(s * scale*log2e - m * scale*log2e).  Most tiles take a fast
//     path with no row max at all: the lane's partial row sum bounds every
//     weight, and only when it exceeds 2^15 (or the row has no m yet) does
//     the tile take the exact max, rescale O and l by
//     exp2((m_old - m_new) * scale*log2e) and recompute P.  A row whose max
//     is still -inf (no visible key yet) uses a shift of 0, so
//     -inf - (-inf) never forms a NaN (GitHub README, "NaN guard").
//   * P is rounded to bf16/fp16 (nearest-even) and is, unchanged, the
//     B operand of O^T = V^T P^T.  The row sum l adds the same rounded pairs
//     with one v_dot2c per pair at d = 64, whose register budget leaves no
//     room for the unrounded weights, and the unrounded fp32 weights at
//     d = 128 (v_dot2c keeps the SIMD about four times as long as an fp32
//     add; measured 1-3 % faster at d = 128, slower at d = 64).
//   * Causal and ragged masking (-inf) is applied only on tiles that cross
//     the diagonal or the end of the sequence; tiles wholly above the
//     diagonal are never loaded.
//   * Epilogue ("FlashAttention dissected", pseudocode's final step): one
//     division of O by l, rounding to the I/O type, and LSE = scale*m + ln l.
//     A workgroup of a split launch covers one range of keys and writes its
//     O / l in fp32 and its LSE as a partial result instead; a second kernel
//     merges the ranges (fa_combine.hip).
//   * Grouped K/V heads and query/key lengths of their own come in through
//     FwdArgs (kv_head(), causal_off), see fa_device.hpp.
#include <type_traits>

#include "fa_h16.hpp"
#include "fa_lds_dma.hpp"

namespace fa_impl {
namespace {

// Largest lane partial row sum accepted without an exact max (see the softmax).
constexpr float kFastSumLimit = 32768.f;


// Tile configuration: NW wave64s per workgroup, each owning QB blocks of 32
// query rows; K/V tiles of BN keys.  The instance table below picks one
// configuration per (dtype, d, causal).
// Cache policy of the K/V loads of one-wave (decoding) workgroups: every
// K/V byte is read exactly once there, and the non-temporal hint (nt) keeps
// that stream from displacing cached lines: 96.5 -> 85.2 us per call on the
// one-row decoding step (8 x 32 query heads on 8 K/V heads of 16384 keys,
// d = 128).  The multi-wave kernels re-read K/V tiles across workgroups
// through L2 and the MALL and keep the default policy.
constexpr int kStreamAux = 2;  // buffer-load cache policy bit: nt
template <int D_, int QB_, int BN_, int NW_>
struct Cfg {
  static constexpr int D = D_, QB = QB_, BN = BN_, NW = NW_;
  // K/V loads carry the non-temporal hint: one-wave workgroups of a decoding
  // step, which read every K/V byte once
  static constexpr bool kStream = NW == 1;
  static constexpr int kThreads = NW * 64;
  static constexpr int kQPerWave = 32 * QB;
  static constexpr int kBM = NW * kQPerWave;        // queries per workgroup
  static constexpr int kKStride = D + 8;            // elements per K row in LDS (+16 B)
  static constexpr int kVStride = BN + 8;           // elements per transposed-V row (+16 B)
  static constexpr int kKStage = BN * kKStride;
  static constexpr int kVStage = D * kVStride;
  // A one-wave workgroup has nobody to overlap with inside the workgroup:
  // it keeps one LDS stage (the next tile waits in registers) so that twice
  // as many workgroups fit in a CU's LDS.
  static constexpr int kStagesReg = NW == 1 ? 1 : 2;
  // d = 128 multi-wave tiles go HBM -> LDS directly (16-byte buffer loads
  // with the LDS bit), three stages deep, unpadded rows with swizzled chunks
  static constexpr bool kDma = D == 128 && NW % 4 == 0;
  static constexpr int kTileElems = BN * D;            // one K or V tile, unpadded
  static constexpr int kStages = kDma ? 3 : kStagesReg;
  static constexpr int kLdsElems = kDma ? kStages * 2 * kTileElems : kStages * (kKStage + kVStage);
  static constexpr int kDmaPer = kTileElems * 2 / (kThreads * 16);  // loads per thread per tile
  static_assert(!kDma || kDmaPer * kThreads * 16 == kTileElems * 2, "DMA tile split");
  static constexpr int kKUnits = BN * D / 8;        // 16-byte K chunks per tile
  static constexpr int kVUnits = (BN / 2) * (D / 8);  // (key pair, 8 columns) per tile
  static constexpr int kKPer = (kKUnits + kThreads - 1) / kThreads;
  static constexpr int kVPer = (kVUnits + kThreads - 1) / kThreads;
  static_assert(BN % 32 == 0 && D % 32 == 0, "tile shape");
};

// The one-wave 32-row tile for short d = 64 grids, where each row block of a
// problem reads its K/V again and the default cache policy keeps them.
template <int D_, int BN_>
struct CfgShort : Cfg<D_, 1, BN_, 1> {
  static constexpr bool kStream = false;
};

template <bool BF16, bool CAUSAL, bool SPLIT, class C>
__global__ __launch_bounds__(C::kThreads) void fwd_h16_kernel(FwdArgs a, int n_qt, int total) {
  using HH = Half<BF16>;
  constexpr int D = C::D, QB = C::QB, BN = C::BN;
  // keys per compute step: a staged tile of BN keys is consumed in BN / SB
  // steps, so a larger tile costs LDS but no registers
  constexpr int SB = BN > 64 ? 64 : BN;
  // row sums of unrounded weights (fp32 adds) rather than of the rounded
  // pairs (v_dot2c): see exp_row
  constexpr bool kSumUnrounded = D == 128;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[C::kLdsElems];

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform across a wave: keep it (and every branch on
  // it) scalar instead of exec-masked
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, grp = lane >> 5;
  const int NQ = a.nq, NK = a.nk;

  // logical tile -> (problem, key range, query tile)
  const int L = xcd_remap(blockIdx.x, total);
  int pr_sp, qt;
  tile_of<CAUSAL>(L, total, n_qt, pr_sp, qt);
  const int split = SPLIT ? pr_sp % a.splits : 0;
  const int prob = SPLIT ? pr_sp / a.splits : pr_sp;

  const int64_t qhead = (int64_t)prob * NQ * D;
  const int64_t kvhead = (int64_t)kv_head(a, prob) * NK * D;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc((const uint16_t*)a.q + qhead, NQ * D * 2);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const uint16_t*)a.k + kvhead, NK * D * 2);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const uint16_t*)a.v + kvhead, NK * D * 2);

  const int q0 = qt * C::kBM;
  const int qw0 = q0 + wave * C::kQPerWave;  // first query of this wave
  const int off = a.causal_off;

  // Keys of this workgroup: its split's range, cut at the last key that the
  // tile's last row may see.  A wave stops at its own last visible key, and
  // a wave whose rows all lie past the end does no arithmetic at all.
  const int kbeg = SPLIT ? split * a.kv_chunk : 0;
  const int kend = SPLIT ? min(kbeg + a.kv_chunk, NK) : NK;  // keys >= kend are masked
  int kstop = kend;
  if (CAUSAL) kstop = min(kstop, q0 + C::kBM + off);
  const int n_kv = kstop > kbeg ? (kstop - kbeg + BN - 1) / BN : 0;
  int wave_kv_end = CAUSAL ? min(qw0 + C::kQPerWave + off, NK) : NK;
  if (qw0 >= NQ) wave_kv_end = kbeg;

  // Direct HBM -> LDS staging (kDma): wave w's load i fills tile rows
  // 4 (i NW + w) .. +3, lane l writing the 16 bytes at l * 16 of that block,
  // i.e. slot l % 16 of row 4 (i NW + w) + l / 16; it fetches the chunk
  // that the swizzle puts there.  The row within its 16-row group is the
  // same for every i (NW is a multiple of 4), so the offset is one value.
  const int dma_row = 4 * wave + (lane >> 4);
  const int dma_off = dma_row * D * 2 + 16 * ((lane & 15) ^ chunk_swz(dma_row));
  auto dma_tile = [&](int k0, int stage) {
    uint16_t* kt = lds + stage * 2 * C::kTileElems;
    uint16_t* vt = kt + C::kTileElems;
    const int g = k0 * D * 2 + dma_off;
#pragma unroll
    for (int i = 0; i < C::kDmaPer; ++i) {
      const int rows = 4 * (i * C::NW + wave);
      buf_load16_lds(kr, kt + rows * D, g + i * C::NW * 4 * D * 2);
      buf_load16_lds(vr, vt + rows * D, g + i * C::NW * 4 * D * 2);
    }
  };
  if constexpr (C::kDma) {
    if (n_kv > 0) dma_tile(kbeg, 0);
  }

  // Q fragments: block qb, lane (col, grp) holds Q[qw0 + 32qb + col][16kc + 8grp .. +8);
  // rows past the end read as zero.
  u32x4 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kc = 0; kc < D / 16; ++kc)
      qf[qb][kc] = buf_load16(qr, ((qw0 + 32 * qb + col) * D + kc * 16 + grp * 8) * 2);

  u32x4 kst[C::kKPer];
  u32x4 vst[C::kVPer][2];

  // HBM -> registers for the tile of keys [k0, k0 + BN).  Keys past the
  // end read as zeros through the buffer range check (their scores are
  // masked, and zero V rows keep 0 * V finite); nothing waits on these loads
  // until the tile is stored to LDS.
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < C::kKPer; ++i) {
      const int u = tid + i * C::kThreads;
      if (C::kKUnits % C::kThreads == 0 || u < C::kKUnits) {
        const int row = u / (D / 8), cc = u % (D / 8);
        kst[i] = buf_load16<C::kStream ? kStreamAux : 0>(kr, ((k0 + row) * D + cc * 8) * 2);
      }
    }
#pragma unroll
    for (int i = 0; i < C::kVPer; ++i) {
      const int u = tid + i * C::kThreads;
      if (C::kVUnits % C::kThreads == 0 || u < C::kVUnits) {
        const int pr = u % (BN / 2), cc = u / (BN / 2);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          vst[i][h] = buf_load16<C::kStream ? kStreamAux : 0>(vr, ((k0 + 2 * pr + h) * D + cc * 8) * 2);
      }
    }
  };

  // registers -> LDS buffer `buf`: K row-major (padded), V transposed with
  // keys interleaved in pairs: one 32-bit word holds (V[kk][c], V[kk+1][c]).
  auto store_tile = [&](int buf) {
    uint16_t* ks = lds + buf * C::kKStage;
    uint16_t* vs = lds + C::kStages * C::kKStage + buf * C::kVStage;
#pragma unroll
    for (int i = 0; i < C::kKPer; ++i) {
      const int u = tid + i * C::kThreads;
      if (C::kKUnits % C::kThreads == 0 || u < C::kKUnits) {
        const int row = u / (D / 8), cc = u % (D / 8);
        *(u32x4*)(ks + row * C::kKStride + cc * 8) = kst[i];
      }
    }
#pragma unroll
    for (int i = 0; i < C::kVPer; ++i) {
      const int u = tid + i * C::kThreads;
      if (C::kVUnits % C::kThreads == 0 || u < C::kVUnits) {
        const int pr = u % (BN / 2), cc = u / (BN / 2);
        const int kk = 2 * pr;
        const int pos = (kk & ~15) | swap23(kk & 15);
        const u32x4 x = vst[i][0], y = vst[i][1];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          // lo = (x.lo16, y.lo16), hi = (x.hi16, y.hi16)
          const uint32_t lo = __builtin_amdgcn_perm(y[j], x[j], 0x05040100u);
          const uint32_t hi = __builtin_amdgcn_perm(y[j], x[j], 0x07060302u);
          *(uint32_t*)(vs + (cc * 8 + 2 * j) * C::kVStride + pos) = lo;
          *(uint32_t*)(vs + (cc * 8 + 2 * j + 1) * C::kVStride + pos) = hi;
        }
      }
    }
  };

  // LDS byte offsets of this lane's operands inside a stage (DMA layout).
  // K: row col, chunk 2 kc + grp -> slot (2 kc) ^ (grp ^ swz(col)); the
  // 2 kc part is applied per read as an XOR of 32 kc.  V (transposed read,
  // rows 4 grp + (lane % 16) / 4 and that + 8 of each 16-key chunk, bytes
  // 64 db + 32 ((lane / 16) % 2) + 8 (lane % 4)): the 64 db part is applied
  // per read as an XOR.
  const int vrow = 4 * grp + ((lane & 15) >> 2);
  const int vx = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const uint32_t k_off = col * D * 2 + 16 * (grp ^ chunk_swz(col));
  const uint32_t v_off0 = vrow * D * 2 + 16 * (vx ^ chunk_swz(vrow)) + 8 * (lane & 1);
  const uint32_t v_off1 = (vrow + 8) * D * 2 + 16 * (vx ^ chunk_swz(vrow + 8)) + 8 * (lane & 1);

  const float c = a.scale_log2;
  float m_run[QB];  // running reference max of raw scores q.k, per query row
  float l_run[QB];  // this lane's share of the running sum of exp2 terms
  // exp2 shift of the fast path, -m c (+inf while the row has no reference
  // max: every weight is then inf and the tile takes the exact path)
  float nmc[QB];
  f32x16 oacc[QB][D / 32];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
    nmc[qb] = __builtin_inff();
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = (f32x16){};
  }

  if constexpr (C::kDma) {
    // Tile 0 went out before Q (kernel start), tile 1 goes out now; all of
    // them are waited for here, once.  The compiler's own wait counting
    // leaves out loads into LDS, so a partial wait would leave Q "pending"
    // to it and it would wait inside the loop, for the prefetched tiles as
    // well; the two tiles were issued back to back, so waiting for tile 1
    // costs little.
    if (n_kv > 1) dma_tile(kbeg + BN, 1);
    __builtin_amdgcn_s_waitcnt(kVmcntWait<0>);
  } else {
    load_tile(kbeg);
    store_tile(0);
    // Everything loaded so far (Q included) has landed: the loop below then
    // never waits on a prefetch before its own LDS store.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  for (int t = 0; t < n_kv; ++t) {
    const int k0 = kbeg + t * BN;
    const bool more = t + 1 < n_kv;
    int buf;
    if constexpr (C::kDma) {
      // This thread's loads of tile t have landed once at most those of
      // tile t + 1 are in flight; the barrier then makes every thread's
      // share visible and tells that everyone is done with tile t - 1,
      // whose stage the loads of tile t + 2 overwrite.  No fence: it would
      // wait for the prefetch as well.
      if (more)
        __builtin_amdgcn_s_waitcnt(kVmcntWait<2 * C::kDmaPer>);
      else
        __builtin_amdgcn_s_waitcnt(kVmcntWait<0>);
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (t + 2 < n_kv) dma_tile(k0 + 2 * BN, (t + 2) % 3);
      buf = t % 3;
    } else {
      if (more) load_tile(k0 + BN);
      buf = C::kStages == 2 ? (t & 1) : 0;
    }
#pragma unroll
    for (int hsub = 0; hsub < BN / SB; ++hsub)
    if (k0 + hsub * SB < wave_kv_end && k0 + hsub * SB < kend) {
      const int kh = k0 + hsub * SB;
      const uint16_t* ks = lds + buf * C::kKStage + hsub * SB * C::kKStride;
      const uint16_t* vs = lds + C::kStages * C::kKStage + buf * C::kVStage + hsub * SB;
      // DMA layout: byte addresses of this lane's operands in the stage
      const uint32_t stage_b =
          (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t*)(lds + buf * 2 * C::kTileElems) +
          hsub * SB * D * 2;
      const uint32_t ka_b = stage_b + k_off;
      const uint32_t va0_b = stage_b + C::kTileElems * 2 + v_off0;
      const uint32_t va1_b = stage_b + C::kTileElems * 2 + v_off1;
      const bool ragged = kh + SB > kend;
      const bool diag = CAUSAL && (kh + SB - 1 > qw0 + off);

      // S^T = K Q^T for row block qb: lane holds keys
      // k0 + 32*kb + 8*(r/4) + 4*grp + r%4 of query qw0 + 32*qb + col.
      auto qk = [&](int qb, f32x16 (&sv)[SB / 32]) {
        if constexpr (C::kDma) {
          // K fragments read two ahead of the MFMA that takes them; the
          // scheduling barriers on both sides of each MFMA keep the compiler
          // from pulling each read down to its MFMA or behind the one before
          // (+2 %, and 1-2 % more once the second barrier made it a true
          // two-ahead, on the d = 128 causal shapes)
          static_assert(SB == 32, "one 32-key block per compute step");
          constexpr int KP = 2;
          u32x4 kf[KP];
#pragma unroll
          for (int j = 0; j < KP; ++j) kf[j] = *(const lds_u32x4*)(uintptr_t)(ka_b ^ (32u * j));
          __builtin_amdgcn_sched_barrier(0);
          sv[0] = (f32x16){};
#pragma unroll
          for (int kc = 0; kc < D / 16; ++kc) {
            const u32x4 ka = kf[kc % KP];
            if (kc + KP < D / 16)
              kf[kc % KP] = *(const lds_u32x4*)(uintptr_t)(ka_b ^ (32u * (kc + KP)));
            __builtin_amdgcn_sched_barrier(0);
            sv[0] = HH::mfma(ka, qf[qb][kc], sv[0]);
            __builtin_amdgcn_sched_barrier(0);
          }
          return;
        }
#pragma unroll
        for (int kb = 0; kb < SB / 32; ++kb) {
          sv[kb] = (f32x16){};
#pragma unroll
          for (int kc = 0; kc < D / 16; ++kc) {
            const u32x4 ka =
                *(const u32x4*)(ks + (kb * 32 + col) * C::kKStride + kc * 16 + grp * 8);
            sv[kb] = HH::mfma(ka, qf[qb][kc], sv[kb]);
          }
        }
      };
      auto mask = [&](int qb, f32x16 (&sv)[SB / 32]) {
        if (ragged || diag) {
          // register r holds key base + 8 (r / 4) + r % 4; the key is
          // masked past the end (>= kend) or, causal, past the row's
          // diagonal: both are "offset > lim" for one per-lane limit, so
          // each score costs one compare against a constant (the key
          // indices themselves, once hoisted by the compiler, cost an add
          // per score on every tile)
#pragma unroll
          for (int kb = 0; kb < SB / 32; ++kb) {
            const int base = kh + kb * 32 + 4 * grp;
            int lim = kend - 1 - base;
            if (CAUSAL) lim = min(lim, qw0 + 32 * qb + col + off - base);
            // keep the compares below inside this branch: hoisted into the
            // QK MFMAs' shadow they ran on every tile
            asm volatile("" : "+v"(lim));
#pragma unroll
            for (int r = 0; r < 16; ++r)
              sv[kb][r] = 8 * (r >> 2) + (r & 3) > lim ? kNegInf : sv[kb][r];
          }
        }
      };

      // P = exp2(S c - m c), rounded for the P.V product.  The row sum adds
      // either the rounded pairs with v_dot2c (the d = 64 tiles: one
      // instruction per pair, and their register budget has no room for the
      // unrounded weights) or the unrounded fp32 weights (d = 128: cheaper to
      // issue than v_dot2c, which occupies the SIMD about four times as long
      // as an fp32 add, and l is then the sum of the exact weights).
      uint32_t pk[QB][SB / 32][8];
      auto exp_row = [&](int qb, const f32x16 (&sv)[SB / 32], float shift) {
        float ls[2];  // two independent sum chains, each started by its first pair
#pragma unroll
        for (int kb = 0; kb < SB / 32; ++kb)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float p0 = fast_exp2(fmaf(sv[kb][2 * j], c, shift));
            const float p1 = fast_exp2(fmaf(sv[kb][2 * j + 1], c, shift));
            pk[qb][kb][j] = HH::pack(p0, p1);
            const float prev = kb == 0 && j < 2 ? 0.f : ls[j & 1];
            ls[j & 1] = kSumUnrounded ? prev + (p0 + p1) : HH::dot2(pk[qb][kb][j], prev);
          }
        return ls[0] + ls[1];
      };
      // Fast path: no row max.  P is formed against the current reference
      // max m, and the lane's partial sum bounds every weight it added; a sum
      // <= 2^15 means no weight can overflow fp16/bf16.  Otherwise (a score
      // rose well above m, or the row has no m yet: the shift is +inf and
      // the sum inf/NaN) take the exact max over both half-waves, rescale O
      // and l by exp2((m_old - m_new) c) and recompute P.
      auto fast = [&](int qb, const f32x16 (&sv)[SB / 32]) { return exp_row(qb, sv, nmc[qb]); };
      auto settle = [&](int qb, const f32x16 (&sv)[SB / 32], float lt) {
        if (__any(!(lt <= kFastSumLimit))) {
          float mx = tree_max<SB / 32>(sv);
          mx = half_swap_max(mx);
          const float m_new = fmaxf(m_run[qb], mx);
          const float alpha = m_new > m_run[qb] ? fast_exp2((m_run[qb] - m_new) * c) : 1.f;
          l_run[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[qb][db] *= alpha;
          m_run[qb] = m_new;
          nmc[qb] = m_new == kNegInf ? __builtin_inff() : -m_new * c;
          lt = exp_row(qb, sv, m_new == kNegInf ? 0.f : -m_new * c);
        }
        l_run[qb] += lt;
      };
      // O^T += V^T P^T over 16-key chunks.
      auto pv = [&](int qb) {
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int pc = 0; pc < SB / 16; ++pc) {
            const u32x4 va =
                *(const u32x4*)(vs + (db * 32 + col) * C::kVStride + pc * 16 + grp * 8);
            const int kb = pc >> 1, h = (pc & 1) * 4;
            const u32x4 pb = {pk[qb][kb][h], pk[qb][kb][h + 1], pk[qb][kb][h + 2],
                              pk[qb][kb][h + 3]};
            oacc[qb][db] = HH::mfma(va, pb, oacc[qb][db]);
          }
      };

      // DMA layout: the V^T operands come from the row-major V tile through
      // the LDS transpose read, issued as inline assembly: the compiler
      // would otherwise make every such read wait for all loads into LDS
      // in flight, the prefetched tiles included.  The values are then
      // passed through the s_waitcnt that completes them, so nothing reads
      // them before they have landed.
      typedef u32x2 vpair[SB / 16][2];
      auto vread = [&](int db, vpair& r) {
        const uint32_t a0 = va0_b ^ (64u * db), a1 = va1_b ^ (64u * db);
#pragma unroll
        for (int pc = 0; pc < SB / 16; ++pc) {
          r[pc][0] = pc == 0 ? lds_read_tr16_b64<0>(a0) : lds_read_tr16_b64<16 * D * 2>(a0);
          r[pc][1] = pc == 0 ? lds_read_tr16_b64<0>(a1) : lds_read_tr16_b64<16 * D * 2>(a1);
        }
      };
      auto vwait = [&](vpair& r) {
        if constexpr (C::kDma) {
          static_assert(SB / 16 == 2, "four transposed reads per d block");
          lds_wait_all(r[0][0], r[0][1], r[1][0], r[1][1]);
        }
      };
      // r's reads done, the four issued after them (the next block's) may
      // still be in flight
      auto vwait_next = [&](vpair& r) {
        if constexpr (C::kDma) lds_wait_keep4(r[0][0], r[0][1], r[1][0], r[1][1]);
      };
      auto vmma = [&](int qb, int db, const vpair& r) {
#pragma unroll
        for (int pc = 0; pc < SB / 16; ++pc) {
          const u32x4 va = {r[pc][0][0], r[pc][0][1], r[pc][1][0], r[pc][1][1]};
          const int kb = pc >> 1, h = (pc & 1) * 4;
          const u32x4 pb = {pk[qb][kb][h], pk[qb][kb][h + 1], pk[qb][kb][h + 2], pk[qb][kb][h + 3]};
          oacc[qb][db] = HH::mfma(va, pb, oacc[qb][db]);
        }
      };

      if constexpr (C::kDma) {
        static_assert(QB == 1 && D == 128, "DMA tiles: one 32-row block per wave, d = 128");
        // d blocks 0 and 1's operands are read while the softmax runs; each
        // later block's read is issued two blocks ahead of its MFMAs.
        static_assert(D / 32 == 4, "four d blocks");
        f32x16 s0[SB / 32];
        qk(0, s0);
        mask(0, s0);
        // (The scheduling barriers keep the compiler from sinking the reads
        // below the softmax and the MFMAs below later waits.)
        vpair r0, r1, r2;
        vread(0, r0);
        vread(1, r1);
        __builtin_amdgcn_sched_barrier(0);
        const float lt0 = fast(0, s0);
        settle(0, s0, lt0);
        vwait_next(r0);
        vread(2, r2);
        vmma(0, 0, r0);
        __builtin_amdgcn_sched_barrier(0);
        vwait_next(r1);
        vread(3, r0);
        vmma(0, 1, r1);
        __builtin_amdgcn_sched_barrier(0);
        vwait_next(r2);
        vmma(0, 2, r2);
        __builtin_amdgcn_sched_barrier(0);
        vwait(r0);
        vmma(0, 3, r0);
      } else if constexpr (QB == 2) {
        // The two 32-row blocks are independent: issued in this order, the
        // QK MFMAs of block 1 run under the softmax of block 0 and the PV
        // MFMAs of block 0 under the softmax of block 1, so each wave keeps
        // its matrix pipe busy while its VALU works (+4 % on the d = 64
        // headline shape against QK, QK, softmax, softmax, PV, PV).
        f32x16 s0[SB / 32], s1[SB / 32];
        qk(0, s0);
        mask(0, s0);
        qk(1, s1);
        const float lt0 = fast(0, s0);
        settle(0, s0, lt0);
        mask(1, s1);
        pv(0);
        const float lt1 = fast(1, s1);
        settle(1, s1, lt1);
        pv(1);
      } else {
        static_assert(QB == 1, "row blocks per wave");
        f32x16 s0[SB / 32];
        qk(0, s0);
        mask(0, s0);
        const float lt0 = fast(0, s0);
        settle(0, s0, lt0);
        pv(0);
      }
    }

    if constexpr (!C::kDma) {
      if (C::kStages == 1) __syncthreads();  // tile t's LDS reads are done
      if (more) store_tile(C::kStages == 2 ? ((t + 1) & 1) : 0);
      __syncthreads();
    }
  }

  // Epilogue: l over both half-waves, O / l, LSE.  The lane's row and column
  // half are recomputed from the lane id (mbcnt) instead of being kept live
  // across the key loop, which would cost registers the loop needs.
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int col_e = lane_e & 31, grp_e = lane_e >> 5;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int q = qw0 + 32 * qb + col_e;
    const float l_tot = half_swap_sum(l_run[qb]);
    const float inv = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
    const float lse = l_tot > 0.f ? (m_run[qb] * c + fast_log2(l_tot)) * kLn2 : kNegInf;
    if (SPLIT) {
      // partial result of this key range, fp32, for the combine step
      if (q < NQ) {
        const int64_t row = ((int64_t)split * a.problems + prob) * NQ + q;
        float* og = (float*)a.o + row * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 w = {oacc[qb][db][4 * j] * inv, oacc[qb][db][4 * j + 1] * inv,
                             oacc[qb][db][4 * j + 2] * inv, oacc[qb][db][4 * j + 3] * inv};
            *(f32x4*)(og + db * 32 + 8 * j + 4 * grp_e) = w;
          }
        if (grp_e == 0) a.lse[row] = lse;
      }
      continue;
    }
    if (q < NQ) {
      uint16_t* og = (uint16_t*)a.o + qhead + (int64_t)q * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int d0 = db * 32 + 8 * j + 4 * grp_e;
          const u32x2 w = {HH::pack(oacc[qb][db][4 * j] * inv, oacc[qb][db][4 * j + 1] * inv),
                           HH::pack(oacc[qb][db][4 * j + 2] * inv, oacc[qb][db][4 * j + 3] * inv)};
          *(u32x2*)(og + d0) = w;
        }
      if (grp_e == 0 && a.lse) a.lse[(int64_t)prob * NQ + q] = lse;
    }
  }
}

template <bool BF16, bool CAUSAL, bool SPLIT, class C>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  int n_qt = (a.nq + C::kBM - 1) / C::kBM;
  int total = (int)((int64_t)n_qt * a.problems * (SPLIT ? a.splits : 1));
  FwdArgs args = a;
  void* params[] = {&args, &n_qt, &total};
  return hipLaunchKernel((const void*)&fwd_h16_kernel<BF16, CAUSAL, SPLIT, C>, dim3(total),
                         dim3(C::kThreads), params, 0, s);
}

// Instance table: one tile configuration per head size (measured on MI355X:
// d = 64 is VALU-heavy, so eight waves of 64 query rows each halve the LDS
// reads per MFMA, and 128-key tiles, computed as two 64-key steps, halve the
// workgroup barriers (the two waves that share a SIMD drift apart less
// often); d = 128 prefers four waves of 32 rows with 32-key tiles).
// Overridable at build time (FA_H16_D64_CFG / FA_H16_D128_CFG = QB, BN, NW).
// Problems with at most 32 query rows (decoding, grouped heads packed into
// rows) take a one-wave workgroup instead, so that the grid is made of key
// ranges rather than of idle query rows; so do d = 64 grids too short to
// fill the chip with the eight-wave tiles (see pick below).
#ifndef FA_H16_D64_CFG
#define FA_H16_D64_CFG 2, 128, 8
#endif
#ifndef FA_H16_D128_CFG
#define FA_H16_D128_CFG 1, 32, 4
#endif
using CfgD64 = Cfg<64, FA_H16_D64_CFG>;
using CfgD128 = Cfg<128, FA_H16_D128_CFG>;
using CfgD64Small = Cfg<64, 1, 64, 1>;
using CfgD128Small = Cfg<128, 1, 32, 1>;
// The same one-wave 32-row workgroups for short grids, where the K/V of a
// problem are read by each of its row blocks and stay cached.
using CfgD64Short = CfgShort<64, 64>;

// d = 64 grids of at most kShortBlocks eight-wave workgroups leave most of
// the 256 compute units idle: they take 32-row one-wave workgroups instead,
// 16x as many, with half of a wave's rows each, so each wave's chain over
// the keys is half as long (measured on MI355X: one 512-row head 25.0 ->
// 12.6 us, 8 heads of 2048 rows 67.6 -> 39.9 us, 2 causal heads of 8192
// rows 231 -> 141 us, 64 heads of 512 rows 26.1 -> 16.9 us; at 192
// workgroups the eight-wave tile is ahead: 24 heads of 4096 rows 148 against
// 251 us).  d = 128 keeps its tile there: its
// waves already hold 32 rows each, so one-wave workgroups would only spread
// the same waves thinner without its direct-to-LDS staging (one causal
// 2048-row head: 48.8 -> 63.0 us).
constexpr int64_t kShortBlocks = 64;  // at most

enum class Pick { kBig, kSmall, kShort };

Pick pick(int d, bool causal, int64_t nq, int64_t problems) {
  if (!causal && nq <= 32) return Pick::kSmall;
  if (d == 64 && (nq + CfgD64::kBM - 1) / CfgD64::kBM * problems <= kShortBlocks) return Pick::kShort;
  return Pick::kBig;
}

template <bool BF16, int D>
hipError_t launch_d(bool causal, bool split, const FwdArgs& a, hipStream_t s) {
  using Big = typename std::conditional<D == 64, CfgD64, CfgD128>::type;
  using Small = typename std::conditional<D == 64, CfgD64Small, CfgD128Small>::type;
  const Pick k = pick(D, causal, a.nq, a.problems);
  if (k == Pick::kSmall)
    return split ? launch<BF16, false, true, Small>(a, s) : launch<BF16, false, false, Small>(a, s);
  if constexpr (D == 64) {
    using Short = CfgD64Short;
    if (k == Pick::kShort) {
      if (causal)
        return split ? launch<BF16, true, true, Short>(a, s) : launch<BF16, true, false, Short>(a, s);
      return split ? launch<BF16, false, true, Short>(a, s) : launch<BF16, false, false, Short>(a, s);
    }
  }
  if (causal)
    return split ? launch<BF16, true, true, Big>(a, s) : launch<BF16, true, false, Big>(a, s);
  return split ? launch<BF16, false, true, Big>(a, s) : launch<BF16, false, false, Big>(a, s);
}

}  // namespace

hipError_t launch_fwd_h16(bool bf16, int d, bool causal, bool split, const FwdArgs& a,
                          hipStream_t s) {
  if (bf16)
    return d == 64 ? launch_d<true, 64>(causal, split, a, s)
                   : launch_d<true, 128>(causal, split, a, s);
  return d == 64 ? launch_d<false, 64>(causal, split, a, s)
                 : launch_d<false, 128>(causal, split, a, s);
}

int h16_rows_per_block(int d, bool causal, int64_t nq, int64_t problems) {
  if (pick(d, causal, nq, problems) != Pick::kBig) return 32;
  return d == 64 ? CfgD64::kBM : CfgD128::kBM;
}

}  // namespace fa_impl
