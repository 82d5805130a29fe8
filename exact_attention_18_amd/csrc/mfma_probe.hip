// Sustained bf16 matrix-core rate of the device, measured with the forward's
// own instruction (v_mfma_f32_32x32x16_bf16) and nothing else.
//
// The roofline analysis of "FlashAttention-4: Algorithm and Kernel Pipelining
// Co-Design for Asymmetric Hardware Scaling" (papercache summary), section
// 3.1.1, prices every unit of the attention tile in cycles of the matrix
// core; this kernel measures what that unit delivers on this device under a
// full grid, so the forward's rate can be set against it as well as against
// the published dense peak.  The published peak assumes the top shader
// clock; the chip lowers its clock under matrix-core load, by an amount that
// depends on the operand data, so the probe takes the operands from the
// caller (random data for the rate the forward can meet, zeros for the
// power-light bound) and reports the shader clock it ran at.
//
// Each wave holds four A and four B operands in VGPRs and issues 16 MFMAs per
// loop iteration into eight independent accumulators, every MFMA on a
// different (A, B) pair from the one before, so consecutive instructions change
// both operands.  The launch mirrors the forward's: one workgroup of 8 waves
// per CU, two waves per SIMD (the accumulators take enough registers that a
// second workgroup does not fit on a CU).  With more waves per SIMD the matrix
// core was measured to sustain less, not more.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn.h"
#include "cdna4.h"

namespace {

constexpr int kProbeWaves = 8;
constexpr int kProbeThreads = 64 * kProbeWaves;
constexpr int kProbeMfmaPerIter = 16;
constexpr int kProbeAcc = 8;

__global__ __launch_bounds__(kProbeThreads, 1) void mfma_probe_kernel(const bf16x8* __restrict__ ops,
                                                                       int iters,
                                                                       float* __restrict__ sink,
                                                                       uint64_t* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[i * 64 + lane];
    b[i] = ops[(4 + i) * 64 + lane];
  }
  f32x16 acc[kProbeAcc];
#pragma unroll
  for (int i = 0; i < kProbeAcc; ++i) acc[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    asm volatile("" : "+v"(a[i]), "+v"(b[i]));  // operands in place before the clock starts
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    // MFMA k: accumulator k % 8, A operand k % 4, B operand (k + k / 4) % 4
    static_for<0, kProbeMfmaPerIter>([&](auto I) __attribute__((always_inline)) {
      constexpr int k = decltype(I)::value;
      acc[k % kProbeAcc] = mfma32(a[k % 4], b[(k + k / 4) % 4], acc[k % kProbeAcc]);
    });
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kProbeAcc; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[i][e];
  sink[(long)blockIdx.x * kProbeThreads + threadIdx.x] = s;
  if (lane == 0) {
    const long w = (long)blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

}  // namespace

extern "C" int attn_probe_mfma(const void* operands, int iters, int workgroups, float* sink,
                               uint64_t* clocks, void* stream) {
  if (operands == nullptr || sink == nullptr || clocks == nullptr) return ATTN_ERR_NULL;
  if (iters < 1 || workgroups < 1) return ATTN_ERR_SIZE;
  if ((reinterpret_cast<uintptr_t>(operands) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(sink) & 3u) != 0 || (reinterpret_cast<uintptr_t>(clocks) & 7u) != 0)
    return ATTN_ERR_ALIGN;
  if (workgroups > (INT32_MAX / kProbeThreads)) return ATTN_ERR_TOO_LARGE;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), static_cast<const bf16x8*>(operands), iters,
                     sink, clocks);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    attn_detail::last_hip_error = static_cast<int>(err);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}
