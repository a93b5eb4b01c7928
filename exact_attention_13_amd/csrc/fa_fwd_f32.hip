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

// ---------------------------------------------------------------------------
// Short grids (fewer workgroups than kShortGrid): each workgroup owns only 32
// query rows and its four waves split the keys instead of the rows.  A step
// stages KS = 4 KW keys in LDS (cooperatively, single-buffered); wave w runs
// the online softmax over keys [k0 + w KW, k0 + (w+1) KW) of every step, and
// at the end the four partial results (m_w, l_w, O_w) are merged through LDS
// with the rescaling of the online softmax ("FlashAttention dissected",
// "Tiling and Online Softmax"): O = sum_w e^(m_w - m) O_w / sum_w e^(m_w - m) l_w.
// The serial chain of a row is then a quarter as long, which is what bounds a
// latency-bound problem such as one 512-row head.
// ---------------------------------------------------------------------------
constexpr int kShortGrid = 128;

template <int D>
struct Short {
  static constexpr int KW = D == 64 ? 64 : 32;  // keys per wave per step
  static constexpr int KS = 4 * KW;             // keys per step
  static constexpr int kKStride = D + 4;
  static constexpr int kVStride = KS + 4;
  static constexpr int kKFloats = KS * kKStride;
  static constexpr int kVFloats = D * kVStride;
  static constexpr int kLdsFloats = kKFloats + kVFloats;
  static constexpr int kKChunks = KS * D / 4 / kThreads;         // float4 K chunks per thread
  static constexpr int kVUnits = (KS / 4) * (D / 4) / kThreads;  // (4 keys, 4 columns) per thread
  static_assert(kKChunks * kThreads * 4 == KS * D, "K tile split");
  static_assert(kVUnits * kThreads * 16 == KS * D, "V tile split");
  static_assert(4 * 32 * D + 2 * 4 * 32 <= kLdsFloats, "merge area");
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_f32_short_kernel(FwdArgs a, int n_qt, int total) {
  using T = Short<D>;
  constexpr int KW = T::KW, KS = T::KS;
  __shared__ __attribute__((aligned(16))) float lds[T::kLdsFloats];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, grp = lane >> 5;
  const int NQ = a.nq, NK = a.nk;

  const int L = xcd_remap(blockIdx.x, total);
  int prob, qt;
  tile_of<CAUSAL>(L, total, n_qt, prob, qt);
  const int q0 = qt * 32;
  const int my_q = q0 + col;
  const int off = a.causal_off;

  const int64_t qhead = (int64_t)prob * NQ * D;
  const int64_t kvhead = (int64_t)kv_head(a, prob) * NK * D;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc((const float*)a.q + qhead, NQ * D * 4);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const float*)a.k + kvhead, NK * D * 4);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const float*)a.v + kvhead, NK * D * 4);

  f32x4 qf[D / 8];
#pragma unroll
  for (int j = 0; j < D / 8; ++j)
    qf[j] = __builtin_bit_cast(f32x4, buf_load16(qr, (my_q * D + j * 8 + grp * 4) * 4));

  // keys the workgroup's last row may see, and the keys of this wave's rows
  int kstop = NK;
  if (CAUSAL) kstop = max(0, min(kstop, q0 + 32 + off));
  const int n_kv = (kstop + KS - 1) / KS;

  const float c = a.scale_log2;
  float m_run = kNegInf, l_run = 0.f;
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16){};

  float* ks = lds;
  float* vs = lds + T::kKFloats;
  for (int t = 0; t < n_kv; ++t) {
    const int k0 = t * KS;
    {
      f32x4 kst[T::kKChunks];
      f32x4 vst[T::kVUnits][4];
#pragma unroll
      for (int i = 0; i < T::kKChunks; ++i) {
        const int u = tid + i * kThreads;
        const int row = u / (D / 4), cc = u % (D / 4);
        kst[i] = __builtin_bit_cast(f32x4, buf_load16(kr, ((k0 + row) * D + cc * 4) * 4));
      }
#pragma unroll
      for (int i = 0; i < T::kVUnits; ++i) {
        const int u = tid + i * kThreads;
        const int kq = u % (KS / 4), cc = u / (KS / 4);
#pragma unroll
        for (int h = 0; h < 4; ++h)
          vst[i][h] =
              __builtin_bit_cast(f32x4, buf_load16(vr, ((k0 + 4 * kq + h) * D + cc * 4) * 4));
      }
      if (t > 0) __syncthreads();  // the previous step's LDS reads are done
#pragma unroll
      for (int i = 0; i < T::kKChunks; ++i) {
        const int u = tid + i * kThreads;
        const int row = u / (D / 4), cc = u % (D / 4);
        *(f32x4*)(ks + row * T::kKStride + cc * 4) = kst[i];
      }
#pragma unroll
      for (int i = 0; i < T::kVUnits; ++i) {
        const int u = tid + i * kThreads;
        const int kq = u % (KS / 4), cc = u / (KS / 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f32x4 w = {vst[i][0][e], vst[i][1][e], vst[i][2][e], vst[i][3][e]};
          *(f32x4*)(vs + (cc * 4 + e) * T::kVStride + kq * 4) = w;
        }
      }
      __syncthreads();
    }

    const int kw = k0 + wave * KW;  // this wave's first key of the step
    if (kw < kstop && (!CAUSAL || kw <= q0 + 31 + off)) {
      f32x16 s[KW / 32];
#pragma unroll
      for (int kb = 0; kb < KW / 32; ++kb) s[kb] = (f32x16){};
#pragma unroll
      for (int j = 0; j < D / 8; ++j)
#pragma unroll
        for (int kb = 0; kb < KW / 32; ++kb) {
          const f32x4 ka =
              *(const f32x4*)(ks + (wave * KW + kb * 32 + col) * T::kKStride + j * 8 + grp * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) s[kb] = mfma_f32(ka[e], qf[j][e], s[kb]);
        }

      if (kw + KW > NK || (CAUSAL && kw + KW - 1 > q0 + off)) {
#pragma unroll
        for (int kb = 0; kb < KW / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = kw + kb * 32 + 8 * (r >> 2) + 4 * grp + (r & 3);
            const bool masked = key >= NK || (CAUSAL && key > my_q + off);
            s[kb][r] = masked ? kNegInf : s[kb][r];
          }
      }

      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KW / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = half_swap_max(mx);
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
      for (int kb = 0; kb < KW / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(s[kb][r], c, nmc));
          s[kb][r] = p;
          l_run += p;
        }
#pragma unroll
      for (int kb = 0; kb < KW / 32; ++kb)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) {
            const f32x4 va = *(const f32x4*)(vs + (db * 32 + col) * T::kVStride + wave * KW +
                                             kb * 32 + g4 * 8 + grp * 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) oacc[db] = mfma_f32(va[e], s[kb][g4 * 4 + e], oacc[db]);
          }
    }
  }

  // Merge the four waves' partial results: O_w (unnormalised), l_w, m_w.
  const float l_w = half_swap_sum(l_run);
  __syncthreads();  // every wave is done with the K/V tiles
  float* om = lds;                   // [wave][row][D]
  float* st = lds + 4 * 32 * D;      // [wave][row]: m, then l
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int jr = 0; jr < 4; ++jr)
      *(f32x4*)(om + (wave * 32 + col) * D + db * 32 + 8 * jr + 4 * grp) =
          (f32x4){oacc[db][4 * jr], oacc[db][4 * jr + 1], oacc[db][4 * jr + 2],
                  oacc[db][4 * jr + 3]};
  if (grp == 0) {
    st[wave * 32 + col] = m_run;
    st[4 * 32 + wave * 32 + col] = l_w;
  }
  __syncthreads();

  // thread -> (row, 4-column group): D/4 groups per row, 32 rows
  constexpr int kGroups = D / 4;
#pragma unroll
  for (int it = 0; it < 32 * kGroups / kThreads; ++it) {
    const int u = tid + it * kThreads;
    const int row = u / kGroups, cg = u % kGroups;
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) m = fmaxf(m, st[w * 32 + row]);
    float ltot = 0.f;
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float mw = st[w * 32 + row];
      const float wt = mw == kNegInf ? 0.f : fast_exp2((mw - m) * c);
      ltot += wt * st[4 * 32 + w * 32 + row];
      o += wt * *(const f32x4*)(om + (w * 32 + row) * D + cg * 4);
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

template <int D, bool CAUSAL>
hipError_t launch_short(const FwdArgs& a, hipStream_t s) {
  int n_qt = (a.nq + 31) / 32;
  int total = (int)((int64_t)n_qt * a.problems);
  FwdArgs args = a;
  void* params[] = {&args, &n_qt, &total};
  return hipLaunchKernel((const void*)&fwd_f32_short_kernel<D, CAUSAL>, dim3(total),
                         dim3(kThreads), params, 0, s);
}

template <int D>
hipError_t launch_d(bool causal, bool split, const FwdArgs& a, hipStream_t s) {
  if (!split && (int64_t)((a.nq + kBM - 1) / kBM) * a.problems < kShortGrid)
    return causal ? launch_short<D, true>(a, s) : launch_short<D, false>(a, s);
  if (causal) return split ? launch<D, true, true>(a, s) : launch<D, true, false>(a, s);
  return split ? launch<D, false, true>(a, s) : launch<D, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_f32(int d, bool causal, bool split, const FwdArgs& a, hipStream_t s) {
  return d == 64 ? launch_d<64>(causal, split, a, s) : launch_d<128>(causal, split, a, s);
}

int f32_rows_per_block() { return kBM; }

}  // namespace fa_impl
