// fa_lds_dma.hpp -- direct HBM -> LDS tile loads and the LDS reads that go
// with them (gfx950), shared by the bf16/fp16 forward and backward kernels.
//
// A tile of 32 rows x 128 bf16/fp16 columns sits in LDS unpadded, 256 bytes
// per row, with its 16-byte chunks XOR-swizzled per row; the 16-byte buffer
// loads that carry the LDS bit write it without passing through registers.
// The compiler leaves those loads out of the waits it places for ordinary
// loads, so the kernels wait for them by hand (kVmcntWait).  It does make
// its transpose-load intrinsic wait for every one in flight, and, in a
// kernel that declares more than one LDS array, every LDS read as well
// (the arrays' alias scopes mark the loads): so the kernels that use them
// declare one LDS array and read transposed operands through inline
// assembly (see below).
#pragma once

#include "fa_h16.hpp"

namespace fa_impl {

// Slot of a 16-byte chunk inside a 256-byte LDS row of a d = 128 tile:
// chunk c of tile row r sits at slot c ^ chunk_swz(r % 16).  The map is a
// bijection of the 16 rows of a 16-row group, so the row reads (16 rows, one
// chunk each: the K and V operands) and the transposed reads (4 rows x 64
// bytes per half-wave: V^T in the forward, K^T in the backward's dQ) each
// touch every bank once, with 64 banks and with 32 alike.
__device__ __forceinline__ int chunk_swz(int r) {
  return (((r >> 1) & 1) << 3) | ((r & 1) << 2) | ((((r >> 1) ^ (r >> 3)) & 1) << 1) |
         ((r >> 2) & 1);
}

typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

// 16-byte buffer load whose data goes straight to LDS: lane l of the wave
// writes bytes [16 l, 16 l + 16) from `dst` (wave-uniform).  Offsets past
// the resource's range read as zeros.  (A device function, not a lambda:
// lambdas inside kernels are host + device, and the host pass rejects the
// builtin there.)
__device__ __forceinline__ void buf_load16_lds(__amdgpu_buffer_rsrc_t r, uint16_t* dst,
                                               int byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           byte_off, 0, 0, 0);
}

// LDS transpose read (ds_read_b64_tr_b16) at byte address addr + OFF, as
// inline assembly, and a wait for every LDS read in flight that passes four
// such results through, so that no use of them can be scheduled before it.
// (The host pass of the compiler sees these bodies too; the asm exists only
// in the device pass.)
template <int OFF>
__device__ __forceinline__ u32x2 lds_read_tr16_b64(uint32_t addr) {
  u32x2 r;
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
#else
  r = (u32x2){addr, 0u};
#endif
  return r;
}
__device__ __forceinline__ void lds_wait_all(u32x2& a, u32x2& b, u32x2& c, u32x2& d) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
#endif
}
// The same, leaving the four most recent LDS operations in flight: enough
// for four reads that were followed by at least four more (LDS operations
// complete in order), such as the next operand block's reads.
__device__ __forceinline__ void lds_wait_keep4(u32x2& a, u32x2& b, u32x2& c, u32x2& d) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_waitcnt lgkmcnt(4)" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
#endif
}

// s_waitcnt operand that waits until at most N vector-memory operations are
// outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14, the other
// counters at their no-wait maxima)
template <int N>
constexpr int kVmcntWait = (N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14);

}  // namespace fa_impl
