// fa_h16.hpp -- helpers shared by the bf16/fp16 forward and backward kernels (gfx950).
#pragma once

#include "fa_device.hpp"

namespace fa_impl {

// MFMA, rounding of P and the element type of one 16-bit input family.
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
  // acc + lo(p) + hi(p): sums a pair of rounded weights in one instruction
  // (v_dot2c; it occupies the SIMD about as long as four fp32 adds)
  static __device__ __forceinline__ float dot2(uint32_t p, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p), one, acc, false);
  }
  // acc + x.lo * y.lo + x.hi * y.hi (products exact in fp32)
  static __device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x),
                                           __builtin_bit_cast(bf16x2, y), acc, false);
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
  static __device__ __forceinline__ float dot2(uint32_t p, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p), one, acc, false);
  }
  static __device__ __forceinline__ float dot2(uint32_t x, uint32_t y, float acc) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), __builtin_bit_cast(f16x2, y),
                                  acc, false);
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// A operand of a 32x32x16 MFMA that contracts over the rows of a row-major
// LDS tile (`stride` elements per row), read with gfx950's LDS transpose load
// (ds_read_b64_tr_b16): lane (col, grp) receives column c0 + col of rows
// r0 + 4 grp + 0..3 and r0 + 8 + 4 grp + 0..3, the row order in which a score
// tile's registers hold them (register r is row 8 (r/4) + 4 grp + r%4), so
// P or dS packed from those registers is the matching B operand.  Within each
// 16-lane group the instruction hands lane j element j % 4 of the 8-byte
// chunks supplied by lanes j/4, 4 + j/4, 8 + j/4 and 12 + j/4, so lane i
// supplies row i/4, columns 4 (i%4) .. +3 of the group's 4 x 16 block.
// Addresses must be 8-byte aligned (stride and c0 multiples of 4).
__device__ __forceinline__ u32x4 lds_tr_operand(const uint16_t* tile, int stride, int r0, int c0,
                                                int lane) {
  const int row = r0 + 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int colx = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const uint16_t* p = tile + row * stride + colx;
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * stride));
  const u32x2 a = __builtin_bit_cast(u32x2, lo), b = __builtin_bit_cast(u32x2, hi);
  return (u32x4){a[0], a[1], b[0], b[1]};
}

// Maximum of the KB x 16 scores held by a lane, as a tree of v_max3.
template <int KB>
__device__ __forceinline__ float tree_max(const f32x16 (&s)[KB]) {
  float m[KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb) {
    const float a = __builtin_fmaxf(__builtin_fmaxf(s[kb][0], s[kb][1]), s[kb][2]);
    const float b = __builtin_fmaxf(__builtin_fmaxf(s[kb][3], s[kb][4]), s[kb][5]);
    const float c = __builtin_fmaxf(__builtin_fmaxf(s[kb][6], s[kb][7]), s[kb][8]);
    const float d = __builtin_fmaxf(__builtin_fmaxf(s[kb][9], s[kb][10]), s[kb][11]);
    const float e = __builtin_fmaxf(__builtin_fmaxf(s[kb][12], s[kb][13]), s[kb][14]);
    const float f = __builtin_fmaxf(__builtin_fmaxf(a, b), c);
    const float g = __builtin_fmaxf(__builtin_fmaxf(d, e), s[kb][15]);
    m[kb] = __builtin_fmaxf(f, g);
  }
  float r = m[0];
#pragma unroll
  for (int kb = 1; kb < KB; ++kb) r = __builtin_fmaxf(r, m[kb]);
  return r;
}

}  // namespace fa_impl
