// fa_device.hpp -- device helpers shared by the libfa forward kernels (gfx950).
//
// Everything here is CDNA4-specific: wave64, 32x32 MFMA tiles, the
// permlane32 swap between the two halves of a wave, and the XCD layout of
// MI355X (eight accelerator dies, workgroups dealt round-robin across them).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa_impl {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;

// Lazy rescaling: the reference maximum of a row only moves when a new score
// exceeds it by more than kRescaleLog2 in exp2 units, so most tiles skip the
// rescale of O and l.  Every exp2 argument stays <= kRescaleLog2, i.e. each
// weight is <= 256: no overflow in fp32, bf16 or fp16.  Softmax does not
// depend on the shift, so the result is the same up to rounding.
constexpr float kRescaleLog2 = 8.0f;

// Arguments common to every forward kernel.
//
// The work is a set of independent attention problems.  Problem p has `nq`
// query rows at q + p*nq*d (o and lse likewise) and reads the K/V head
// kv(p) = (p / hp) * hkv + (p % hp) / grp, whose `nk` key rows start at
// k + kv(p)*nk*d (v likewise).  Plain multi-head attention is hp = hkv = H,
// grp = 1, nq = nk = N.  Grouped heads either map several query heads to one
// K/V head (grp = H / H_kv) or, when no mask depends on the row, are packed
// into the rows of one problem (nq = grp * N_q, grp = 1): the group's query
// heads are adjacent in memory, so the packed rows are contiguous.
//
// Causal masking hides key j from row i when j > i + causal_off.
//
// Split launches cut the keys into ranges of kv_chunk keys (a multiple of
// 64; kernels mask keys past the end of their range): workgroup (p, split)
// attends to keys
// [split*kv_chunk, min((split+1)*kv_chunk, nk)) only and writes its partial
// result in fp32, already divided by its own row sum, to
// o + ((split*problems + p)*nq + i)*d, and its partial logsumexp to
// lse[(split*problems + p)*nq + i].
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;      // may be null unless split
  int problems;    // independent (batch, head) problems
  int nq;          // query rows per problem
  int nk;          // key rows per K/V head
  int hp;          // problems per batch entry
  int hkv;         // K/V heads per batch entry
  int grp;         // consecutive problems that share one K/V head
  int causal_off;  // key j visible to row i iff j <= i + causal_off
  int splits;      // key ranges per problem (1: no split)
  int kv_chunk;    // keys per range when split
  float scale;     // multiplier of q.k
  float scale_log2;  // scale * log2(e): scores enter exp2 in this unit
};

// K/V head read by problem p.
__device__ __forceinline__ int kv_head(const FwdArgs& a, int p) {
  return (p / a.hp) * a.hkv + (p % a.hp) / a.grp;
}

// ---------------------------------------------------------------------------
// Workgroup -> tile mapping.
//
// The dispatcher deals workgroup w to XCD (w mod 8).  Re-indexing makes each
// XCD take one contiguous range of logical tiles, so the workgroups that a
// die runs at the same time mostly belong to one head and read the same K/V
// tiles through that die's L2.  The map is a bijection of [0, total).
// ---------------------------------------------------------------------------
constexpr int kXcdCount = 8;  // MI355X: eight dies (XCDs) of 32 CUs

__device__ __forceinline__ int xcd_remap(int w, int total) {
  constexpr int kXcds = kXcdCount;
  const int per = total / kXcds, extra = total % kXcds;
  const int x = w % kXcds, i = w / kXcds;
  const int base = x * per + (x < extra ? x : extra);
  return base + i;
}

// Logical tile L of a grid of `total` = units x n_qt tiles -> (unit, query
// tile).  Without a mask: unit-major, query tiles upward.  Under the causal
// mask a tile's work grows with its query tile, so the heaviest go first.
// When every die's range (xcd_remap) holds whole units, the range is taken
// in groups of kCausalGroup units, the heaviest query tiles of all units of
// a group first: the last tiles a die dispatches are then short ones rather
// than one unit's longest (measured: C3 / C5 / C4 made causal 4-5 % faster
// than unit by unit).  Groups never cross dies, which would hand one die all
// the heavy tiles.  Bijective on [0, total).
constexpr int kCausalGroup = 4;

template <bool CAUSAL>
__device__ __forceinline__ void tile_of(int L, int total, int n_qt, int& unit, int& qt) {
  if (!CAUSAL) {
    unit = L / n_qt;
    qt = L - unit * n_qt;
    return;
  }
  const int per = total / kXcdCount;
  const int upx = total % kXcdCount == 0 && per % n_qt == 0 ? per / n_qt : 0;
  if (upx == 0) {
    unit = L / n_qt;
    qt = n_qt - 1 - (L - unit * n_qt);
    return;
  }
  const int die = L / per, local = L - die * per;
  const int G = upx < kCausalGroup ? upx : kCausalGroup;
  const int g = local / (G * n_qt), r = local - g * (G * n_qt);
  const int gp = upx - g * G < G ? upx - g * G : G;
  const int level = r / gp;
  unit = die * upx + g * G + (r - level * gp);
  qt = n_qt - 1 - level;
}

// Buffer resource over `bytes` bytes from `base` (raw, no stride).  Loads
// whose offset lies past the end return zeros instead of touching memory:
// rows past the end of a sequence read as zero without a branch or a wait.
// 0x00020000 is the resource word 3 that gfx9-family parts expect.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// 16-byte buffer load; AUX is the cache-policy operand (0: default).
template <int AUX = 0>
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, AUX));
}

// Reduce a value with the lane that differs in bit 5 (the other half-wave).
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Key position inside a 16-key chunk of the transposed V tile: bits 2 and 3
// swapped.  The 32x32 score accumulator gives lane half g the keys
// {4g..4g+3, 8+4g..8+4g+3} of each 16-key chunk; storing key kk at
// swap23(kk) puts exactly those eight keys at positions 8g..8g+7, so one
// 16-byte LDS read yields a lane's whole A operand for the P.V product.
__host__ __device__ constexpr int swap23(int kk) {
  return (kk & ~0xC) | ((kk & 4) << 1) | ((kk & 8) >> 1);
}

// Host-side launchers (one per element-type family).  `split` selects the
// partial-output kernels (a.splits > 1).
hipError_t launch_fwd_h16(bool bf16, int d, bool causal, bool split, const FwdArgs& a,
                          hipStream_t s);
hipError_t launch_fwd_f32(int d, bool causal, bool split, const FwdArgs& a, hipStream_t s);


// Merge `splits` partial results (fp32 O divided by its own row sum, and its
// logsumexp) of `rows` rows of head size d into O of the I/O type and LSE.
// dtype: 0 fp32, 1 bf16, 2 fp16.
hipError_t launch_lse_combine(const float* o_part, const float* lse_part, int splits,
                              int64_t rows, int d, void* o, float* lse, int dtype,
                              hipStream_t s);

// Workgroups of a combine launch over `rows` rows of head size d.
int64_t combine_grid_blocks(int64_t rows, int d);

// Query rows per workgroup of the instance a launch would use (the host
// sizes grids and split counts with it).
int h16_rows_per_block(int d, bool causal, int64_t nq, int64_t problems);
int f32_rows_per_block();
// Whether an unsplit fp32 launch over `problems` problems of `nq` query rows
// takes the small-problem kernel (16-row blocks spread over the chip).
bool f32_small_kernel(int64_t nq, int64_t problems, bool causal, int d);

}  // namespace fa_impl
