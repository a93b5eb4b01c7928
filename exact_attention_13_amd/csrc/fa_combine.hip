// fa_combine.hip -- merges attention results computed over disjoint key
// ranges, for MI355X (gfx950).
//
// Each range s delivers, per query row, O_s (already divided by its own sum
// of exponentials) and LSE_s, the natural logarithm of that sum.  Because
// e^LSE_s is exactly the range's sum of exponentials, the merge is the
// online-softmax rescaling applied once more, at range granularity
// ("FlashAttention dissected", section "The mathematical breakthrough:
// Tiling and Online Softmax": partial sums are brought to a common maximum
// by exp(m_old - m_new) before they are added; the section "Interaction
// with the KV cache during inference" splits the keys of one query across
// compute units in exactly this way):
//     M   = max_s LSE_s
//     W   = sum_s exp(LSE_s - M)
//     O   = sum_s exp(LSE_s - M) O_s / W
//     LSE = M + ln W
// A range with no visible key has LSE_s = -inf and weight 0; a row with no
// visible key in any range gets O = 0 and LSE = -inf.
//
// The kernel is bound by HBM bandwidth (it reads splits * (d + 1) fp32 per
// row and writes one row): each row is handled by d/4 lanes with 16-byte
// loads, so one wave reads whole contiguous rows of every range.
#include "fa_device.hpp"

namespace fa_impl {
namespace {

// Small blocks: a decoding step has only a few hundred rows, and the blocks
// should spread over all compute units.
constexpr int kCombineThreads = 64;
constexpr float kLog2e = 1.44269504088896340736f;

template <int DT>  // 0: fp32, 1: bf16, 2: fp16 output
__device__ __forceinline__ void store4(void* o, int64_t idx, f32x4 x) {
  if (DT == 0) {
    *(f32x4*)((float*)o + idx) = x;
  } else if (DT == 1) {
    const bf16x2 a = {(__bf16)x[0], (__bf16)x[1]}, b = {(__bf16)x[2], (__bf16)x[3]};
    const u32x2 w = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
    *(u32x2*)((uint16_t*)o + idx) = w;
  } else {
    const f16x2 a = {(_Float16)x[0], (_Float16)x[1]}, b = {(_Float16)x[2], (_Float16)x[3]};
    const u32x2 w = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
    *(u32x2*)((uint16_t*)o + idx) = w;
  }
}

template <int D, int DT>
__global__ __launch_bounds__(kCombineThreads) void lse_combine_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, int splits,
    int64_t rows, void* __restrict__ o, float* __restrict__ lse) {
  constexpr int kLanesPerRow = D / 4;
  constexpr int kRowsPerBlock = kCombineThreads / kLanesPerRow;
  const int sub = threadIdx.x % kLanesPerRow;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  if (row >= rows) return;

  float m = kNegInf;
  for (int s = 0; s < splits; ++s) m = fmaxf(m, lse_part[(int64_t)s * rows + row]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float w_sum = 0.f;
  if (m != kNegInf) {
    const float mc = m * kLog2e;
#pragma unroll 8
    for (int s = 0; s < splits; ++s) {
      const int64_t r = (int64_t)s * rows + row;
      const float w = fast_exp2(fmaf(lse_part[r], kLog2e, -mc));  // 0 for an empty range
      const f32x4 x = *(const f32x4*)(o_part + r * D + sub * 4);
      acc += w * x;
      w_sum += w;
    }
  }
  const float inv = w_sum > 0.f ? 1.f / w_sum : 0.f;
  store4<DT>(o, row * D + sub * 4, acc * inv);
  if (sub == 0 && lse) lse[row] = w_sum > 0.f ? m + fast_log2(w_sum) * kLn2 : kNegInf;
}

template <int D, int DT>
hipError_t launch(const float* o_part, const float* lse_part, int splits, int64_t rows, void* o,
                  float* lse, hipStream_t s) {
  constexpr int kRowsPerBlock = kCombineThreads / (D / 4);
  const int64_t blocks = (rows + kRowsPerBlock - 1) / kRowsPerBlock;
  void* params[] = {&o_part, &lse_part, &splits, &rows, &o, &lse};
  return hipLaunchKernel((const void*)&lse_combine_kernel<D, DT>, dim3((unsigned)blocks),
                         dim3(kCombineThreads), params, 0, s);
}

template <int D>
hipError_t launch_d(const float* o_part, const float* lse_part, int splits, int64_t rows,
                    void* o, float* lse, int dtype, hipStream_t s) {
  if (dtype == 0) return launch<D, 0>(o_part, lse_part, splits, rows, o, lse, s);
  if (dtype == 1) return launch<D, 1>(o_part, lse_part, splits, rows, o, lse, s);
  return launch<D, 2>(o_part, lse_part, splits, rows, o, lse, s);
}

}  // namespace

hipError_t launch_lse_combine(const float* o_part, const float* lse_part, int splits,
                              int64_t rows, int d, void* o, float* lse, int dtype,
                              hipStream_t s) {
  return d == 64 ? launch_d<64>(o_part, lse_part, splits, rows, o, lse, dtype, s)
                 : launch_d<128>(o_part, lse_part, splits, rows, o, lse, dtype, s);
}

int64_t combine_grid_blocks(int64_t rows, int d) {
  const int64_t per = kCombineThreads / (d / 4);
  return (rows + per - 1) / per;
}

}  // namespace fa_impl
