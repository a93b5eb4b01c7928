// fa_fwd_f32.hip -- FlashAttention forward, fp32 in / fp32 MFMA / fp32 out,
// for MI355X (gfx950).
//
// Same schedule as the bf16/fp16 kernel (one workgroup per (problem,
// 128-query tile[, key range]), four wave64s of 32 queries, K/V tiles of 64 keys double
// buffered in LDS, S^T = K Q^T so that each lane holds one query's scores,
// online softmax with exp2, one division by l at the end), with fp32 data:
//   * both products run on v_mfma_f32_32x32x2_f32 (2-deep contraction per
//     instruction);
//   * the contraction order is permuted so each lane's operands come from
//     16-byte reads: lane half g feeds columns 8j + 4g .. 8j + 4g + 3 of K
//     and Q to four consecutive instructions; for P.V the score register r
//     of the S^T accumulator is, unchanged, the B operand of instruction r;
//   * V is stored transposed in LDS ([d][key], four keys per 16-byte word
//     group), a register-level 4x4 transpose on the way in;
//   * P stays fp32 and l is a plain fp32 sum.
// Sources as for the bf16/fp16 kernel: "FlashAttention dissected",
// "Algorithmic core in pseudocode" (the recurrence and final division),
// the GitHub README "CUDA Flash Attention..." (padded shared rows, K/V loads
// by all warps, tile masking, NaN guard, size_t indexing) and the course
// lesson "FlashAttention Inner Loop Implementation" (Q held in registers).
#include "fa_device.hpp"

namespace fa_impl {
namespace {

constexpr int kThreads = 256;
constexpr int kQPerWave = 32;
constexpr int kBM = 128;
constexpr int kBN = 64;

template <int D>
struct Tile {
  static constexpr int kKStride = D + 4;    // floats per K row in LDS (+16 B)
  static constexpr int kVStride = kBN + 4;  // floats per transposed-V row (+16 B)
  static constexpr int kKStage = kBN * kKStride;
  static constexpr int kVStage = D * kVStride;
  static constexpr int kLdsFloats = 2 * (kKStage + kVStage);
  static constexpr int kKChunks = kBN * D / 4 / kThreads;         // float4 K chunks per thread
  static constexpr int kVUnits = (kBN / 4) * (D / 4) / kThreads;  // (4 keys, 4 columns) per thread
  static_assert(kKChunks * kThreads * 4 == kBN * D, "K tile split");
  static_assert(kVUnits * kThreads * 16 == kBN * D, "V tile split");
};

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kThreads) void fwd_f32_kernel(FwdArgs a, int n_qt, int total) {
  using T = Tile<D>;
  __shared__ __attribute__((aligned(16))) float lds[T::kLdsFloats];

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
  const __amdgpu_buffer_rsrc_t qr = make_rsrc((const float*)a.q + qhead, NQ * D * 4);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const float*)a.k + kvhead, NK * D * 4);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const float*)a.v + kvhead, NK * D * 4);

  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * kQPerWave;
  const int my_q = qw0 + col;
  const int off = a.causal_off;

  // Q fragment: lane (col, grp) holds Q[my_q][8j + 4grp + e], e = 0..3; rows
  // past the end read as zero.
  f32x4 qf[D / 8];
#pragma unroll
  for (int j = 0; j < D / 8; ++j)
    qf[j] = __builtin_bit_cast(f32x4, buf_load16(qr, (my_q * D + j * 8 + grp * 4) * 4));

  // Keys of this workgroup and of this wave, as in the bf16/fp16 kernel.
  const int kbeg = SPLIT ? split * a.kv_chunk : 0;
  const int kend = SPLIT ? min(kbeg + a.kv_chunk, NK) : NK;  // keys >= kend are masked
  int kstop = kend;
  if (CAUSAL) kstop = min(kstop, q0 + kBM + off);
  const int n_kv = kstop > kbeg ? (kstop - kbeg + kBN - 1) / kBN : 0;
  int wave_kv_end = CAUSAL ? min(qw0 + kQPerWave + off, NK) : NK;
  if (qw0 >= NQ) wave_kv_end = kbeg;

  f32x4 kst[T::kKChunks];
  f32x4 vst[T::kVUnits][4];

  // HBM -> registers for keys [k0, k0 + kBN); keys past the end read as
  // zeros (buffer range check).
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i) {
      const int u = tid + i * kThreads;
      const int row = u / (D / 4), cc = u % (D / 4);
      kst[i] = __builtin_bit_cast(f32x4, buf_load16(kr, ((k0 + row) * D + cc * 4) * 4));
    }
#pragma unroll
    for (int i = 0; i < T::kVUnits; ++i) {
      const int u = tid + i * kThreads;
      const int kq = u % (kBN / 4), cc = u / (kBN / 4);
#pragma unroll
      for (int h = 0; h < 4; ++h)
        vst[i][h] = __builtin_bit_cast(f32x4, buf_load16(vr, ((k0 + 4 * kq + h) * D + cc * 4) * 4));
    }
  };

  auto store_tile = [&](int buf) {
    float* ks = lds + buf * T::kKStage;
    float* vs = lds + 2 * T::kKStage + buf * T::kVStage;
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i) {
      const int u = tid + i * kThreads;
      const int row = u / (D / 4), cc = u % (D / 4);
      *(f32x4*)(ks + row * T::kKStride + cc * 4) = kst[i];
    }
#pragma unroll
    for (int i = 0; i < T::kVUnits; ++i) {
      const int u = tid + i * kThreads;
      const int kq = u % (kBN / 4), cc = u / (kBN / 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const f32x4 w = {vst[i][0][e], vst[i][1][e], vst[i][2][e], vst[i][3][e]};
        *(f32x4*)(vs + (cc * 4 + e) * T::kVStride + kq * 4) = w;
      }
    }
  };

  const float c = a.scale_log2;
  float m_run = kNegInf;
  float l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16){};

  load_tile(kbeg);
  store_tile(0);
  // Everything loaded so far (Q included) has landed: the loop below then
  // never waits on a prefetch before its own LDS store.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < n_kv; ++t) {
    const int k0 = kbeg + t * kBN;
    const bool more = t + 1 < n_kv;
    if (more) load_tile(k0 + kBN);

    if (k0 < wave_kv_end) {
      const float* ks = lds + (t & 1) * T::kKStage;
      const float* vs = lds + 2 * T::kKStage + (t & 1) * T::kVStage;

      f32x16 s[kBN / 32];
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) s[kb] = (f32x16){};
#pragma unroll
      for (int j = 0; j < D / 8; ++j)
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb) {
          const f32x4 ka = *(const f32x4*)(ks + (kb * 32 + col) * T::kKStride + j * 8 + grp * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kb] = mfma_f32(ka[e], qf[j][e], s[kb]);
        }

      const bool ragged = k0 + kBN > kend;
      const bool diag = CAUSAL && (k0 + kBN - 1 > qw0 + off);
      if (ragged || diag) {
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * grp + (r & 3);
            const bool masked = key >= kend || (CAUSAL && key > my_q + off);
            s[kb][r] = masked ? kNegInf : s[kb][r];
          }
      }

      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = half_swap_max(mx);

      // Lazy reference max, as in the bf16/fp16 kernel.
      const bool grow = (mx - m_run) * c > kRescaleLog2;
      if (__any(grow)) {
        const float alpha = grow ? fast_exp2((m_run - mx) * c) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        m_run = grow ? mx : m_run;
      }
      const float nmc = m_run == kNegInf ? 0.f : -m_run * c;

#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[kb][r], c, nmc));
          s[kb][r] = p;
          l_run += p;
        }

      // O^T += V^T P^T: instruction r of key block kb takes score register r.
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const f32x4 va =
                *(const f32x4*)(vs + (db * 32 + col) * T::kVStride + kb * 32 + g4 * 8 + grp * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[db] = mfma_f32(va[e], s[kb][g4 * 4 + e], oacc[db]);
          }
    }

    if (more) store_tile((t + 1) & 1);
    __syncthreads();
  }

  const float l_tot = half_swap_sum(l_run);
  const float inv = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
  const float lse = l_tot > 0.f ? (m_run * c + fast_log2(l_tot)) * kLn2 : kNegInf;
  if (my_q < NQ) {
    // a split writes its partial result (fp32, like the output) to the
    // workspace rows of its key range
    const int64_t row = SPLIT ? ((int64_t)split * a.problems + prob) * NQ + my_q
                              : (int64_t)prob * NQ + my_q;
    float* og = (float*)a.o + row * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 w = {oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv,
                         oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv};
        *(f32x4*)(og + db * 32 + 8 * j + 4 * grp) = w;
      }
    if (grp == 0 && a.lse) a.lse[row] = lse;
  }
}

template <int D, bool CAUSAL, bool SPLIT>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  int n_qt = (a.nq + kBM - 1) / kBM;
  int total = (int)((int64_t)n_qt * a.problems * (SPLIT ? a.splits : 1));
  FwdArgs args = a;
  void* params[] = {&args, &n_qt, &total};
  return hipLaunchKernel((const void*)&fwd_f32_kernel<D, CAUSAL, SPLIT>, dim3(total),
                         dim3(kThreads), params, 0, s);
}

// Grids of at most kShortGrid workgroups of 128 rows take the small-problem
// kernel below; causal grids of at most kShortGridCausal, whose 128-row
// workgroups also differ in length, so that a grid of one or two per compute
// unit ends with a long tail.  Measured on MI355X (median of 30 queued
// calls): 32 heads of 512 rows (128 workgroups) 44.0 -> 36.4 us, causal
// 43.4 -> 30.8; 24 causal heads of 1024 rows (192) 80.8 -> 59.6 us; while
// non-causal grids from about 192 workgroups and causal ones of 256 run
// faster on the 128-row kernel (48 heads of 512 rows: 45.8 against 51.9 us;
// 16 causal heads of 512 rows x 4: 45.7 against 55.6).  Causal d = 64
// problems of at least 2048 rows gain up to kShortGridLong workgroups (8
// heads of 4096 rows, 256 workgroups: 298 -> 204 us; 6 of 8192, 384: 808 ->
// 614 us; one d = 128 case of 384 lost 5 %, so d = 128 stays out).
constexpr int kShortGrid = 128;
constexpr int kShortGridCausal = 255;
constexpr int kShortGridLong = 511;

// ---------------------------------------------------------------------------
// Small fp32 problems (at most kShortGrid workgroups of 128 rows, e.g. one
// 512-row head).  There the time is set by the serial MFMA chain of each
// compute unit, not by the chip's throughput, so the work is cut finer:
//   * 16 query rows per workgroup on v_mfma_f32_16x16x4_f32 (half the rows
//     of a 32x32 tile, so twice as many compute units share a head);
//   * the eight waves of a workgroup take every eighth 16-key tile of the
//     keys, each with its own online-softmax state, and are merged through
//     LDS at the end with the same rescale rule ("FlashAttention dissected",
//     "The mathematical breakthrough": partial results over disjoint key
//     sets combine through their maxima and sums);
//   * no waves share K/V tiles, so each lane loads its MFMA operands from
//     global memory (L2) directly, 16 contiguous bytes at a time, one tile
//     ahead of the compute.
// Operand layouts (measured on gfx950 with an in-bounds probe): for
// 16x16x4, lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16], and
// holds D[4 (l / 16) + r][l % 16] in register r.
//   * S^T = K Q^T per 16-key tile: the contraction over d is split into D/4
//     instructions; instruction m takes, in lane group g = l / 16, column
//     g D/4 + m, so each lane reads D/4 consecutive floats of its key row
//     (A) and of its query row (B).  Lane (j, g) ends up with keys 4g + r of
//     query j (r = 0..3).
//   * O^T += V^T P^T: instruction r of a tile contracts keys {4g + r}, which
//     lane (j, g) holds as its score register r, so P^T needs no data
//     movement; output tile t holds columns d = TD i + t (TD = D / 16) in
//     row i, so each lane reads TD consecutive floats of a value row (A) and
//     ends up with D/4 consecutive output columns g D/4 .. of query j.
// ---------------------------------------------------------------------------
constexpr int kTinyThreads = 512;  // eight waves
constexpr int kTinyRows = 16;

__device__ __forceinline__ f32x4 mfma16(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16-byte buffer load written as inline assembly (offsets past the
// resource's range read as zeros).  The compiler places no wait for it: the
// kernel waits by hand with tiny_vm_wait before any use, and never lets the
// result die before that wait (a load still in flight would otherwise land
// in registers given to another value).
__device__ __forceinline__ u32x4 tiny_buf_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  u32x4 v;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(byte_off), "s"(r));
#else
  v = (u32x4){(uint32_t)byte_off, 0u, 0u, 0u};
#endif
  return v;
}
// Wait until at most N vector-memory operations are in flight, passing one
// register buffer's loads through the wait so that no use of them can be
// scheduled before it.
template <int N, int KL, int VL>
__device__ __forceinline__ void tiny_vm_wait(u32x4 (&k)[KL], u32x4 (&v)[4][VL]);
template <>
__device__ __forceinline__ void tiny_vm_wait<8, 4, 1>(u32x4 (&k)[4], u32x4 (&v)[4][1]) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(8)" : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]),
               "+v"(v[0][0]), "+v"(v[1][0]), "+v"(v[2][0]), "+v"(v[3][0]));
#endif
}
template <>
__device__ __forceinline__ void tiny_vm_wait<0, 4, 1>(u32x4 (&k)[4], u32x4 (&v)[4][1]) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]),
               "+v"(v[0][0]), "+v"(v[1][0]), "+v"(v[2][0]), "+v"(v[3][0]));
#endif
}
template <>
__device__ __forceinline__ void tiny_vm_wait<16, 8, 2>(u32x4 (&k)[8], u32x4 (&v)[4][2]) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(16)" : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]), "+v"(k[4]),
               "+v"(k[5]), "+v"(k[6]), "+v"(k[7]), "+v"(v[0][0]), "+v"(v[0][1]), "+v"(v[1][0]),
               "+v"(v[1][1]), "+v"(v[2][0]), "+v"(v[2][1]), "+v"(v[3][0]), "+v"(v[3][1]));
#endif
}
template <>
__device__ __forceinline__ void tiny_vm_wait<0, 8, 2>(u32x4 (&k)[8], u32x4 (&v)[4][2]) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(0)" : "+v"(k[0]), "+v"(k[1]), "+v"(k[2]), "+v"(k[3]), "+v"(k[4]),
               "+v"(k[5]), "+v"(k[6]), "+v"(k[7]), "+v"(v[0][0]), "+v"(v[0][1]), "+v"(v[1][0]),
               "+v"(v[1][1]), "+v"(v[2][0]), "+v"(v[2][1]), "+v"(v[3][0]), "+v"(v[3][1]));
#endif
}

template <int N, int QL>
__device__ __forceinline__ void tiny_vm_wait_q(u32x4 (&q)[QL]);
template <>
__device__ __forceinline__ void tiny_vm_wait_q<16, 4>(u32x4 (&q)[4]) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(16)" : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]));
#endif
}
template <>
__device__ __forceinline__ void tiny_vm_wait_q<32, 8>(u32x4 (&q)[8]) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt vmcnt(32)" : "+v"(q[0]), "+v"(q[1]), "+v"(q[2]), "+v"(q[3]), "+v"(q[4]),
               "+v"(q[5]), "+v"(q[6]), "+v"(q[7]));
#endif
}

// max / sum over the four lane groups (lanes j, j + 16, j + 32, j + 48)
__device__ __forceinline__ float quad_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  return half_swap_max(x);
}

// TU: output tiles of 16 columns per workgroup.  With TU < TD the D / 16
// tiles of a 16-row block are shared out among TD / TU workgroups, each of
// which computes the block's scores and weights in full (the same bits in
// every one of them) but only its own tiles of P.V, so that each compute
// unit's MFMA chain is QK plus TU / TD of the P.V work when the blocks alone
// would leave most units idle.  They write disjoint columns of O; the first
// of them writes the LSE.
template <int D, bool CAUSAL, int TU>
__global__ __launch_bounds__(kTinyThreads) void fwd_f32_tiny_kernel(FwdArgs a, int n_qt, int total) {
  constexpr int DQ = D / 4;    // floats per lane of a K or Q row, and output columns per lane
  constexpr int TD = D / 16;   // output tiles of 16 columns
  constexpr int CG = TD / TU;  // workgroups per 16-row block
  static_assert(TU >= 1 && TD % TU == 0, "output tiles per workgroup");
  constexpr int NWV = kTinyThreads / 64;
  __shared__ __attribute__((aligned(16))) float lds[NWV * kTinyRows * D + 2 * NWV * kTinyRows];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 15, g = lane >> 4;
  const int NQ = a.nq, NK = a.nk;

  // logical index -> (16-row block, column group); the column groups of a
  // block are consecutive, so they run on one die and share its L2
  const int L = xcd_remap(blockIdx.x, total);
  const int cgi = CG == 1 ? 0 : L % CG;
  const int u0 = cgi * TU;  // first output tile of this workgroup
  int prob, qt;
  tile_of<CAUSAL>(CG == 1 ? L : L / CG, total / CG, n_qt, prob, qt);
  const int q0 = qt * kTinyRows;
  const int off = a.causal_off;

  const int64_t qhead = (int64_t)prob * NQ * D;
  const int64_t kvhead = (int64_t)kv_head(a, prob) * NK * D;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc((const float*)a.q + qhead, NQ * D * 4);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const float*)a.k + kvhead, NK * D * 4);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const float*)a.v + kvhead, NK * D * 4);

  // query row q0 + j, columns g DQ .. g DQ + DQ - 1 (rows past the end read
  // 0); loaded like the K/V tiles below (inline assembly, waited for by
  // hand), so that no load the compiler counts is in flight at the loop
  u32x4 qq[DQ / 4];
#pragma unroll
  for (int i = 0; i < DQ / 4; ++i) qq[i] = tiny_buf_load16(qr, ((q0 + j) * D + g * DQ + 4 * i) * 4);
  float qv[DQ];  // filled from qq once it has landed

  int kstop = NK;
  if (CAUSAL) kstop = max(0, min(kstop, q0 + kTinyRows + off));
  const int n_tiles = (kstop + 15) / 16;

  // this wave's tiles: wave, wave + NWV, ...; operands of tile t:
  // K row t*16 + j, columns g DQ ..; V rows t*16 + 4g + r, columns TD j ..
  // They rotate through two register buffers: the wave's next tile loads
  // while the current one is computed.  The loads are inline assembly with
  // the waits placed by hand (tiny_vm_wait): the compiler's own waits for
  // loads still in flight across the loop's back edge fell back to waiting
  // for all of them, the other buffer's prefetch included, so the loop ran
  // at one load latency per tile.  Every buffer is refilled on every pass
  // (tiles past the end read as zeros through the buffer range check and are
  // never computed), and every load is waited for before its registers die.
  constexpr int NB = 2;
  constexpr int KL = DQ / 4, VL = TD / 4;  // 16-byte loads per K row, per V row
  constexpr int kLoadsPerBuf = KL + 4 * VL;
  static_assert(kLoadsPerBuf <= 16, "buffer loads per wait");
  u32x4 kq[NB][KL], vq[NB][4][VL];
  auto load = [&](int buf, int t) {
    const int k0 = t * 16;
#pragma unroll
    for (int i = 0; i < KL; ++i)
      kq[buf][i] = tiny_buf_load16(kr, ((k0 + j) * D + g * DQ + 4 * i) * 4);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int i = 0; i < VL; ++i)
        vq[buf][r][i] = tiny_buf_load16(vr, ((k0 + 4 * g + r) * D + TD * j + 4 * i) * 4);
  };
  // buffer buf has landed once at most the other buffer's loads, issued
  // after it, are in flight
  auto wait_buf = [&](int buf) { tiny_vm_wait<(NB - 1) * kLoadsPerBuf, KL, VL>(kq[buf], vq[buf]); };
  auto kf = [&](int buf, int m) { return __uint_as_float(kq[buf][m >> 2][m & 3]); };
  // value of this workgroup's output tile u0 + uu from the V row loaded for
  // key 4g + r (the loads bring every tile's column; u0 is uniform)
  auto vf = [&](int buf, int r, int uu) {
    float x = __uint_as_float(vq[buf][r][uu >> 2][uu & 3]);
#pragma unroll
    for (int c = 1; c < CG; ++c) {
      const int u = c * TU + uu;
      x = cgi == c ? __uint_as_float(vq[buf][r][u >> 2][u & 3]) : x;
    }
    return x;
  };

  const float c = a.scale_log2;
  float m_run = kNegInf, l_run = 0.f;
  f32x4 oacc[TU];
#pragma unroll
  for (int t = 0; t < TU; ++t) oacc[t] = (f32x4){0.f, 0.f, 0.f, 0.f};

  const int my_q = q0 + j;
  // one tile of this wave from buffer buf (a constant at each call site, so
  // the buffers stay in registers); the buffer is then refilled with the
  // tile NB steps ahead
  auto step = [&](int buf, int t) {
    const int k0 = t * 16;
    f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < DQ; ++m) s = mfma16(kf(buf, m), qv[m], s);
    // lane (j, g) register r: key k0 + 4g + r of query my_q
    if (k0 + 16 > NK || (CAUSAL && k0 + 15 > q0 + off)) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * g + r;
        const bool masked = key >= NK || (CAUSAL && key > my_q + off);
        s[r] = masked ? kNegInf : s[r];
      }
    }
    float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
    mx = quad_max(mx);
    // lazy rescale: the reference maximum moves only when a score exceeds it
    // by more than kRescaleLog2 in exp2 units
    const bool grow = (mx - m_run) * c > kRescaleLog2;
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2((m_run - mx) * c) : 1.f;
      l_run *= alpha;
#pragma unroll
      for (int u = 0; u < TU; ++u) oacc[u] *= alpha;
      m_run = grow ? mx : m_run;
    }
    const float nmc = m_run == kNegInf ? 0.f : -m_run * c;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = fast_exp2(fmaf(s[r], c, nmc));
      l_run += p[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int u = 0; u < TU; ++u) oacc[u] = mfma16(vf(buf, r, u), p[r], oacc[u]);
  };
#pragma unroll
  for (int b = 0; b < NB; ++b) load(b, wave + b * NWV);
  tiny_vm_wait_q<NB * kLoadsPerBuf>(qq);  // Q has landed (issued before both buffers)
#pragma unroll
  for (int m = 0; m < DQ; ++m) qv[m] = __uint_as_float(qq[m >> 2][m & 3]);
  for (int t = wave; t < n_tiles; t += NB * NWV) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      wait_buf(b);
      if (t + b * NWV < n_tiles) step(b, t + b * NWV);
      load(b, t + b * NWV + NB * NWV);
    }
  }
  // the last refills (past the end) must land before their registers die
#pragma unroll
  for (int b = 0; b < NB; ++b) tiny_vm_wait<0, KL, VL>(kq[b], vq[b]);

  // Merge the waves: O_w (unnormalised, this lane's columns g DQ .. of row
  // j), l_w (the lane sum over the four lane groups) and m_w.
  float l_w = l_run;
  {
    const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(l_w), __float_as_uint(l_w),
                                                    false, false);
    l_w = __uint_as_float(x[0]) + __uint_as_float(x[1]);
  }
  l_w = half_swap_sum(l_w);
  float* om = lds;                                // [wave][row][D]
  float* st = lds + NWV * kTinyRows * D;          // [wave][row]: m, then l
  // output column of oacc[u][r]: g DQ + TD r + u0 + u
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    float* dst = om + (wave * kTinyRows + j) * D + g * DQ + TD * r + u0;
    if constexpr (TU % 4 == 0) {
#pragma unroll
      for (int u = 0; u < TU; u += 4) {
        const f32x4 w = {oacc[u][r], oacc[u + 1][r], oacc[u + 2][r], oacc[u + 3][r]};
        *(f32x4*)(dst + u) = w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < TU; ++u) dst[u] = oacc[u][r];
    }
  }
  if (g == 0) {
    st[wave * kTinyRows + j] = m_run;
    st[NWV * kTinyRows + wave * kTinyRows + j] = l_w;
  }
  __syncthreads();

  if constexpr (CG > 1) {
    // thread -> (row, one of this workgroup's 16 TU columns): the sum below,
    // column by column
    constexpr int kCols = 16 * TU;
    for (int u = tid; u < kTinyRows * kCols; u += kTinyThreads) {
      const int row = u / kCols, lc = u % kCols;
      const int col = (lc / (4 * TU)) * DQ + TD * ((lc / TU) % 4) + u0 + lc % TU;
      float m = kNegInf;
#pragma unroll
      for (int w = 0; w < NWV; ++w) m = fmaxf(m, st[w * kTinyRows + row]);
      float ltot = 0.f, o = 0.f;
#pragma unroll
      for (int w = 0; w < NWV; ++w) {
        const float mw = st[w * kTinyRows + row];
        const float wt = mw == kNegInf ? 0.f : fast_exp2((mw - m) * c);
        ltot += wt * st[NWV * kTinyRows + w * kTinyRows + row];
        o += wt * om[(w * kTinyRows + row) * D + col];
      }
      const int q = q0 + row;
      if (q < NQ) {
        const float inv = ltot > 0.f ? __builtin_amdgcn_rcpf(ltot) : 0.f;
        ((float*)a.o)[((int64_t)prob * NQ + q) * D + col] = o * inv;
        if (cgi == 0 && lc == 0 && a.lse)
          a.lse[(int64_t)prob * NQ + q] = ltot > 0.f ? (m * c + fast_log2(ltot)) * kLn2 : kNegInf;
      }
    }
    return;
  }
  // thread -> (row, 4-column group)
  constexpr int kGroups = D / 4;
  for (int u = tid; u < kTinyRows * kGroups; u += kTinyThreads) {
    const int row = u / kGroups, cg = u % kGroups;
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < NWV; ++w) m = fmaxf(m, st[w * kTinyRows + row]);
    float ltot = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NWV; ++w) {
      const float mw = st[w * kTinyRows + row];
      const float wt = mw == kNegInf ? 0.f : fast_exp2((mw - m) * c);
      ltot += wt * st[NWV * kTinyRows + w * kTinyRows + row];
      o += wt * *(const f32x4*)(om + (w * kTinyRows + row) * D + cg * 4);
    }
    const int q = q0 + row;
    if (q < NQ) {
      const float inv = ltot > 0.f ? __builtin_amdgcn_rcpf(ltot) : 0.f;
      *(f32x4*)((float*)a.o + ((int64_t)prob * NQ + q) * D + cg * 4) = o * inv;
      if (cg == 0 && a.lse)
        a.lse[(int64_t)prob * NQ + q] = ltot > 0.f ? (m * c + fast_log2(ltot)) * kLn2 : kNegInf;
    }
  }
}

// Column groups of the small-problem kernel: when its 16-row blocks number
// at most a quarter of kTinyFill, each block's output tiles are shared out
// among four workgroups.
constexpr int kTinyFill = 256;

template <int D, bool CAUSAL, int TU>
hipError_t launch_tiny_tu(const FwdArgs& a, hipStream_t s) {
  int n_qt = (a.nq + kTinyRows - 1) / kTinyRows;
  int total = (int)((int64_t)n_qt * a.problems * (D / 16 / TU));
  FwdArgs args = a;
  void* params[] = {&args, &n_qt, &total};
  return hipLaunchKernel((const void*)&fwd_f32_tiny_kernel<D, CAUSAL, TU>, dim3(total),
                         dim3(kTinyThreads), params, 0, s);
}

template <int D, bool CAUSAL>
hipError_t launch_tiny(const FwdArgs& a, hipStream_t s) {
  const int64_t blocks = (a.nq + kTinyRows - 1) / kTinyRows * (int64_t)a.problems;
  if (blocks * 4 <= kTinyFill) return launch_tiny_tu<D, CAUSAL, D / 64>(a, s);
  return launch_tiny_tu<D, CAUSAL, D / 16>(a, s);
}

template <int D>
hipError_t launch_d(bool causal, bool split, const FwdArgs& a, hipStream_t s) {
  if (!split && f32_small_kernel(a.nq, a.problems, causal, D))
    return causal ? launch_tiny<D, true>(a, s) : launch_tiny<D, false>(a, s);
  if (causal) return split ? launch<D, true, true>(a, s) : launch<D, true, false>(a, s);
  return split ? launch<D, false, true>(a, s) : launch<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_f32(int d, bool causal, bool split, const FwdArgs& a, hipStream_t s) {
  return d == 64 ? launch_d<64>(causal, split, a, s) : launch_d<128>(causal, split, a, s);
}

int f32_rows_per_block() { return kBM; }

bool f32_small_kernel(int64_t nq, int64_t problems, bool causal, int d) {
  const int64_t blocks = (nq + kBM - 1) / kBM * problems;
  if (!causal) return blocks <= kShortGrid;
  return blocks <= (d == 64 && nq >= 2048 ? kShortGridLong : kShortGridCausal);
}

}  // namespace fa_impl
