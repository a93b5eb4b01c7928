// fa_fwd_h16.hip -- FlashAttention forward, bf16 / fp16 inputs, fp32 accumulate,
// for MI355X (gfx950).
//
// What runs (one workgroup per (batch*head, 128-query tile); four wave64s,
// each owning 32 query rows):
//   * The query tile stays in registers for the whole key loop, as the
//     B operand of S^T = K Q^T (course lesson "FlashAttention Inner Loop
//     Implementation", section "Implementing the Inner Loop": Q is loaded
//     once and reused for every key/value step).
//   * K/V tiles of 64 keys are staged HBM -> registers -> LDS, double
//     buffered: tile t+1 is fetched by every thread (all four waves, 16-byte
//     loads) while tile t is computed, then written to the other LDS buffer
//     (GitHub README "CUDA Flash Attention...", "Performance Analysis": the
//     K/V load must use all warps; "Design decisions": padded shared rows).
//     K rows are padded by 16 bytes; V is stored transposed ([d][key]) with
//     the key order permuted inside each 16-key chunk, so each lane's
//     operand for the P.V product is one 16-byte LDS read.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16}: each lane ends up with
//     32 scores of ONE query (16 per 32-key block), the other 32 scores of
//     that query sit in the lane 32 positions away.  Row statistics are thus
//     an in-lane reduction plus one permlane32 swap.
//   * Online softmax ("FlashAttention dissected", "Algorithmic core in
//     pseudocode"): running max m and sum l per query row, in registers; the
//     scores enter exp2 with the scale folded into one FMA,
//     p = exp2(s * scale*log2e - m * scale*log2e); when the max grows, O and
//     l are rescaled by exp2((m_old - m_new) * scale*log2e).  The reference
//     max only moves when a score beats it by more than 2^8 in exp2 units,
//     so the rescale is skipped, wave-uniformly, on almost every tile.
//     A row whose max is still -inf (no visible key yet) uses a shift of 0,
//     so -inf - (-inf) never forms a NaN (GitHub README, "NaN guard").
//   * P is rounded to bf16/fp16 (nearest-even) and is, unchanged, the
//     B operand of O^T = V^T P^T; the row sum l adds the same rounded values
//     (v_dot2 with (1, 1)), so the weights that multiply V sum to one.
//   * Causal and ragged masking (-inf) is applied only on tiles that cross
//     the diagonal or the end of the sequence; tiles wholly above the
//     diagonal are never loaded.
//   * Epilogue ("FlashAttention dissected", pseudocode's final step): one
//     division of O by l, rounding to the I/O type, and LSE = scale*m + ln l.
#include "fa_device.hpp"

namespace fa_impl {
namespace {

constexpr int kThreads = 256;    // four wave64s
constexpr int kQPerWave = 32;    // one 32-wide MFMA column block per wave
constexpr int kBM = 128;         // queries per workgroup
constexpr int kBN = 64;          // keys per K/V tile

template <bool BF16>
struct Half;

template <>
struct Half<true> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    const bf16x2 t = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, t);
  }
  // acc + lo(p) + hi(p), fp32 accumulate
  static __device__ __forceinline__ float add_pair(uint32_t p, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
  }
};

template <>
struct Half<false> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float x, float y) {
    const f16x2 t = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, t);
  }
  static __device__ __forceinline__ float add_pair(uint32_t p, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), one, acc, false);
  }
};

template <int D>
struct Tile {
  static constexpr int kKStride = D + 8;    // elements per K row in LDS (+16 B)
  static constexpr int kVStride = kBN + 8;  // elements per transposed-V row (+16 B)
  static constexpr int kKStage = kBN * kKStride;
  static constexpr int kVStage = D * kVStride;
  static constexpr int kLdsElems = 2 * (kKStage + kVStage);
  static constexpr int kKChunks = kBN * D / 8 / kThreads;          // 16 B K chunks per thread
  static constexpr int kVUnits = (kBN / 2) * (D / 8) / kThreads;   // (key pair, 8 columns) per thread
  static_assert(kKChunks * kThreads * 8 == kBN * D, "K tile split");
  static_assert(kVUnits * kThreads * 16 == kBN * D, "V tile split");
};

template <bool BF16, int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void fwd_h16_kernel(FwdArgs a, int n_qt, int total) {
  using T = Tile<D>;
  using HH = Half<BF16>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[T::kLdsElems];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, grp = lane >> 5;
  const int N = a.n;

  const int L = xcd_remap(blockIdx.x, total);
  const int bh = L / n_qt;
  int qt = L - bh * n_qt;
  if (CAUSAL) qt = n_qt - 1 - qt;  // longest rows first

  const int64_t head = (int64_t)bh * N * D;
  const int head_bytes = N * D * 2;
  const __amdgpu_buffer_rsrc_t qr = make_rsrc((const uint16_t*)a.q + head, head_bytes);
  const __amdgpu_buffer_rsrc_t kr = make_rsrc((const uint16_t*)a.k + head, head_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc((const uint16_t*)a.v + head, head_bytes);

  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * kQPerWave;
  const int my_q = qw0 + col;

  // Q fragment: lane (col, grp) holds Q[my_q][16*kc + 8*grp .. +8); rows past
  // the end read as zero.
  u32x4 qf[D / 16];
#pragma unroll
  for (int kc = 0; kc < D / 16; ++kc) qf[kc] = buf_load16(qr, (my_q * D + kc * 16 + grp * 8) * 2);

  const int kv_end = CAUSAL ? min(q0 + kBM, N) : N;
  const int n_kv = (kv_end + kBN - 1) / kBN;
  const int wave_kv_end = CAUSAL ? min(qw0 + kQPerWave, N) : N;

  u32x4 kst[T::kKChunks];
  u32x4 vst[T::kVUnits][2];

  // HBM -> registers for tile t.  Keys >= N read as zeros through the
  // buffer range check (their scores are masked, and zero V rows keep 0 * V
  // finite); nothing waits on these loads until the tile is stored to LDS.
  auto load_tile = [&](int t) {
    const int k0 = t * kBN;
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i) {
      const int u = tid + i * kThreads;
      const int row = u / (D / 8), cc = u % (D / 8);
      kst[i] = buf_load16(kr, ((k0 + row) * D + cc * 8) * 2);
    }
#pragma unroll
    for (int i = 0; i < T::kVUnits; ++i) {
      const int u = tid + i * kThreads;
      const int pr = u % (kBN / 2), cc = u / (kBN / 2);
#pragma unroll
      for (int h = 0; h < 2; ++h) vst[i][h] = buf_load16(vr, ((k0 + 2 * pr + h) * D + cc * 8) * 2);
    }
  };

  // registers -> LDS buffer `buf`: K row-major (padded), V transposed with
  // keys interleaved in pairs: one 32-bit word holds (V[kk][c], V[kk+1][c]).
  auto store_tile = [&](int buf) {
    uint16_t* ks = lds + buf * T::kKStage;
    uint16_t* vs = lds + 2 * T::kKStage + buf * T::kVStage;
#pragma unroll
    for (int i = 0; i < T::kKChunks; ++i) {
      const int u = tid + i * kThreads;
      const int row = u / (D / 8), cc = u % (D / 8);
      *(u32x4*)(ks + row * T::kKStride + cc * 8) = kst[i];
    }
#pragma unroll
    for (int i = 0; i < T::kVUnits; ++i) {
      const int u = tid + i * kThreads;
      const int pr = u % (kBN / 2), cc = u / (kBN / 2);
      const int kk = 2 * pr;
      const int pos = (kk & ~15) | swap23(kk & 15);
      const u32x4 x = vst[i][0], y = vst[i][1];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // lo = (x.lo16, y.lo16), hi = (x.hi16, y.hi16)
        const uint32_t lo = __builtin_amdgcn_perm(y[j], x[j], 0x05040100u);
        const uint32_t hi = __builtin_amdgcn_perm(y[j], x[j], 0x07060302u);
        *(uint32_t*)(vs + (cc * 8 + 2 * j) * T::kVStride + pos) = lo;
        *(uint32_t*)(vs + (cc * 8 + 2 * j + 1) * T::kVStride + pos) = hi;
      }
    }
  };

  const float c = a.scale_log2;
  float m_run = kNegInf;  // running max of raw scores q.k for query my_q
  float l_run = 0.f;      // this lane's share of the running sum of exp2 terms
  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = (f32x16){};

  load_tile(0);
  store_tile(0);
  // Everything loaded so far (Q included) has landed: the loop below then
  // never waits on a prefetch before its own LDS store.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int t = 0; t < n_kv; ++t) {
    const int k0 = t * kBN;
    const bool more = t + 1 < n_kv;
    if (more) load_tile(t + 1);

    if (k0 < wave_kv_end) {
      const uint16_t* ks = lds + (t & 1) * T::kKStage;
      const uint16_t* vs = lds + 2 * T::kKStage + (t & 1) * T::kVStage;

      // S^T = K Q^T: lane holds keys k0 + 32*kb + 8*(r/4) + 4*grp + r%4.
      f32x16 s[kBN / 32];
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
        s[kb] = (f32x16){};
#pragma unroll
        for (int kc = 0; kc < D / 16; ++kc) {
          const u32x4 ka =
              *(const u32x4*)(ks + (kb * 32 + col) * T::kKStride + kc * 16 + grp * 8);
          s[kb] = HH::mfma(ka, qf[kc], s[kb]);
        }
      }

      const bool ragged = k0 + kBN > N;
      const bool diag = CAUSAL && (k0 + kBN - 1 > qw0);
      if (ragged || diag) {
#pragma unroll
        for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * grp + (r & 3);
            const bool masked = key >= N || (CAUSAL && key > my_q);
            s[kb][r] = masked ? kNegInf : s[kb][r];
          }
      }

      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = half_swap_max(mx);

      // Move the reference max only when the tile's max beats it by more
      // than 2^kRescaleLog2 (always on a row's first visible key, since
      // m_run = -inf there); a row still without a visible key keeps -inf.
      const bool grow = (mx - m_run) * c > kRescaleLog2;
      if (__any(grow)) {
        const float alpha = grow ? fast_exp2((m_run - mx) * c) : 1.f;
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
        m_run = grow ? mx : m_run;
      }
      const float nmc = m_run == kNegInf ? 0.f : -m_run * c;

      uint32_t pk[kBN / 32][8];
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p0 = fast_exp2(fmaf(s[kb][2 * j], c, nmc));
          const float p1 = fast_exp2(fmaf(s[kb][2 * j + 1], c, nmc));
          pk[kb][j] = HH::pack(p0, p1);
          l_run = HH::add_pair(pk[kb][j], l_run);
        }

      // O^T += V^T P^T over 16-key chunks.
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int pc = 0; pc < kBN / 16; ++pc) {
          const u32x4 va =
              *(const u32x4*)(vs + (db * 32 + col) * T::kVStride + pc * 16 + grp * 8);
          const int kb = pc >> 1, h = (pc & 1) * 4;
          const u32x4 pb = {pk[kb][h], pk[kb][h + 1], pk[kb][h + 2], pk[kb][h + 3]};
          oacc[db] = HH::mfma(va, pb, oacc[db]);
        }
    }

    if (more) store_tile((t + 1) & 1);
    __syncthreads();
  }

  // Epilogue: l over both half-waves, O / l, LSE.
  const float l_tot = half_swap_sum(l_run);
  const float inv = l_tot > 0.f ? __builtin_amdgcn_rcpf(l_tot) : 0.f;
  if (my_q < N) {
    uint16_t* og = (uint16_t*)a.o + head + (int64_t)my_q * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = db * 32 + 8 * j + 4 * grp;
        const u32x2 w = {HH::pack(oacc[db][4 * j] * inv, oacc[db][4 * j + 1] * inv),
                         HH::pack(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv)};
        *(u32x2*)(og + d0) = w;
      }
    if (grp == 0 && a.lse)
      a.lse[(int64_t)bh * N + my_q] =
          l_tot > 0.f ? (m_run * c + fast_log2(l_tot)) * kLn2 : kNegInf;
  }
}

template <bool BF16, int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t s) {
  int n_qt = (a.n + kBM - 1) / kBM;
  int total = (int)((int64_t)n_qt * a.bh);
  FwdArgs args = a;
  void* params[] = {&args, &n_qt, &total};
  return hipLaunchKernel((const void*)&fwd_h16_kernel<BF16, D, CAUSAL>, dim3(total),
                         dim3(kThreads), params, 0, s);
}

template <bool BF16, int D>
hipError_t launch_c(bool causal, const FwdArgs& a, hipStream_t s) {
  return causal ? launch<BF16, D, true>(a, s) : launch<BF16, D, false>(a, s);
}

}  // namespace

hipError_t launch_fwd_h16(bool bf16, int d, bool causal, const FwdArgs& a, hipStream_t s) {
  if (bf16) return d == 64 ? launch_c<true, 64>(causal, a, s) : launch_c<true, 128>(causal, a, s);
  return d == 64 ? launch_c<false, 64>(causal, a, s) : launch_c<false, 128>(causal, a, s);
}

int64_t h16_grid_blocks(int64_t bh, int64_t n) { return (n + kBM - 1) / kBM * bh; }

}  // namespace fa_impl
