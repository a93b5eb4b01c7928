// mfma_probe.hip -- the dense MFMA rate this GPU sustains, measured.
//
// Not part of libfa: a separate library (libfa_probe.so) that the benchmark
// loads to put an attention kernel's FLOP rate beside the rate of a plain
// MFMA loop on the same GPU, at the clock the chip holds under MFMA load
// (the published peaks assume 2.4 GHz).  The loop is what the attention
// kernels' MFMAs would achieve with no softmax, no memory traffic and no
// waits: every wave issues independent 32x32 MFMAs back to back, two waves
// per SIMD, every SIMD of the chip busy.  It also holds a delay kernel, which
// the benchmark queues its timed launches behind.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;             // four waves: one per SIMD
constexpr int kLdsBytes = 64 * 1024;      // two workgroups per CU fit in its LDS
constexpr int kAcc = 4;                   // independent accumulators per wave

template <int DT>
__global__ __launch_bounds__(kThreads) void mfma_loop(float* out, int iters) {
  extern __shared__ float lds[];
  const float t = (float)threadIdx.x * 1e-3f;
  f32x16 acc[kAcc] = {};
  bf16x8 ab, bb;
  f16x8 ah, bh;
  for (int i = 0; i < 8; ++i) {
    ab[i] = (__bf16)(t + i);
    bb[i] = (__bf16)(t - i);
    ah[i] = (_Float16)(t + i);
    bh[i] = (_Float16)(t - i);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kAcc; ++j) {
      if (DT == 1)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ab, bb, acc[j], 0, 0, 0);
      else if (DT == 2)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, acc[j], 0, 0, 0);
      else
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x2f32(t, t + 1.f, acc[j], 0, 0, 0);
    }
  }
  float r = 0.f;
  for (int j = 0; j < kAcc; ++j)
    for (int e = 0; e < 16; ++e) r += acc[j][e];
  lds[threadIdx.x] = r;  // the LDS allocation limits residency to two workgroups per CU
  out[blockIdx.x * kThreads + threadIdx.x] = r;
}

constexpr double kFlopsPerMfma[3] = {32.0 * 32 * 2 * 2, 32.0 * 32 * 16 * 2, 32.0 * 32 * 16 * 2};

// One wave that waits until `ticks` of the constant-rate real-time counter
// have passed since it started, then exits.
__global__ __launch_bounds__(64) void delay_kernel(uint64_t ticks) {
  const uint64_t t0 = wall_clock64();
  while (wall_clock64() - t0 < ticks) __builtin_amdgcn_s_sleep(8);
}

}  // namespace

extern "C" {

// Dense MFMA rate of the current device, in TFLOP/s, for dtype 0 (fp32,
// v_mfma_f32_32x32x2f32), 1 (bf16) or 2 (fp16, both v_mfma_f32_32x32x16):
// `launches` timed launches of `iters` loop iterations each, on `stream`
// (a hipStream_t; null = the default stream), after one untimed launch.
// *tflops receives the best launch's rate.  Returns 0, or a hipError_t code.
// The call allocates and frees its own device buffer and synchronises the
// stream.
int fa_probe_mfma_tflops(int dtype, int iters, int launches, void* stream, double* tflops) {
  if (dtype < 0 || dtype > 2 || iters <= 0 || launches <= 0 || !tflops) return (int)hipErrorInvalidValue;
  hipStream_t s = (hipStream_t)stream;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return (int)e;
  const int grid = 2 * cus;
  const void* fn = dtype == 1 ? (const void*)&mfma_loop<1>
                 : dtype == 2 ? (const void*)&mfma_loop<2> : (const void*)&mfma_loop<0>;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  if (e != hipSuccess) return (int)e;
  float* out = nullptr;
  e = hipMalloc((void**)&out, sizeof(float) * grid * kThreads);
  if (e != hipSuccess) return (int)e;
  hipEvent_t a = nullptr, b = nullptr;
  double best = 0.0;
  e = hipEventCreate(&a);
  if (e == hipSuccess) e = hipEventCreate(&b);
  for (int l = 0; e == hipSuccess && l <= launches; ++l) {
    void* params[] = {&out, &iters};
    e = hipEventRecord(a, s);
    if (e == hipSuccess) e = hipLaunchKernel(fn, dim3(grid), dim3(kThreads), params, kLdsBytes, s);
    if (e == hipSuccess) e = hipEventRecord(b, s);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, a, b);
    if (e == hipSuccess && l > 0 && ms > 0.f) {
      const double flops = kFlopsPerMfma[dtype] * kAcc * (double)iters * grid * (kThreads / 64);
      const double r = flops / (ms * 1e-3) / 1e12;
      if (r > best) best = r;
    }
  }
  if (a) (void)hipEventDestroy(a);
  if (b) (void)hipEventDestroy(b);
  (void)hipFree(out);
  if (e != hipSuccess) return (int)e;
  *tflops = best;
  return 0;
}

// Occupies `stream` (a hipStream_t; null = the default stream) for about
// `microseconds` (0 .. 1000000) with a one-wave kernel that waits on the
// GPU's real-time counter, so that launches the host makes next queue up
// behind it and then run back to back.  Asynchronous.  Returns 0, or a
// hipError_t code (hipErrorInvalidValue for an out-of-range time).
int fa_probe_delay(int microseconds, void* stream) {
  if (microseconds < 0 || microseconds > 1000000) return (int)hipErrorInvalidValue;
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return (int)e;
  if (khz <= 0) return (int)hipErrorInvalidValue;
  uint64_t ticks = (uint64_t)microseconds * (uint64_t)khz / 1000u;
  void* params[] = {&ticks};
  return (int)hipLaunchKernel((const void*)&delay_kernel, dim3(1), dim3(64), params, 0,
                              (hipStream_t)stream);
}

}  // extern "C"
