// Sustained bf16 matrix-core rate of the device, measured with the forward's
// own instruction (v_mfma_f32_32x32x16_bf16), or the 16x16x32 shape, and
// nothing else.
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
// Each wave holds four A and four B operands in VGPRs and issues MFMAs into
// independent accumulators, every MFMA on a different (A, B) pair from the
// one before, so consecutive instructions change both operands.  Two shapes:
// the forward's 32x32x16 (16 MFMAs per loop iteration, 8 accumulators) and
// 16x16x32 (32 MFMAs of half the FLOPs, 16 accumulators), the same FLOPs per
// iteration.  The launch mirrors the forward's: one workgroup of 8 waves per
// CU, two waves per SIMD; each workgroup reserves more than half of the CU's
// LDS, so a second one never shares its CU whatever the register count.
// With more waves per SIMD the matrix core was measured to sustain less, not
// more.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn.h"
#include "cdna4.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kProbeWaves = 8;
constexpr int kProbeThreads = 64 * kProbeWaves;
constexpr int kProbeLdsFloats = 84 * 1024 / 4;  // 84 KB of the CU's 160 KB

template <int SHAPE>
__global__ __launch_bounds__(kProbeThreads, 1) void mfma_probe_kernel(const bf16x8* __restrict__ ops,
                                                                       int iters,
                                                                       float* __restrict__ sink,
                                                                       uint64_t* __restrict__ clocks) {
  __shared__ float reserve[kProbeLdsFloats];
  const int lane = threadIdx.x & 63;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[i * 64 + lane];
    b[i] = ops[(4 + i) * 64 + lane];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
    asm volatile("" : "+v"(a[i]), "+v"(b[i]));  // operands in place before the clock starts
  float s = 0.f;
  uint64_t t0, r0, t1, r1;
  if constexpr (SHAPE == 32) {
    f32x16 acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
      // MFMA k: accumulator k % 8, A operand k % 4, B operand (k + k / 4) % 4
      static_for<0, 16>([&](auto I) __attribute__((always_inline)) {
        constexpr int k = decltype(I)::value;
        acc[k % 8] = mfma32(a[k % 4], b[(k + k / 4) % 4], acc[k % 8]);
      });
    }
    t1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 16; ++e) s += acc[i][e];
  } else {
    f32x4 acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = f32x4{};
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
      // MFMA k: accumulator k % 16, A operand k % 4, B operand (k + k / 4) % 4
      static_for<0, 32>([&](auto I) __attribute__((always_inline)) {
        constexpr int k = decltype(I)::value;
        acc[k % 16] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[k % 4], b[(k + k / 4) % 4],
                                                              acc[k % 16], 0, 0, 0);
      });
    }
    t1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) s += acc[i][e];
  }
  // The sum passes through the reserved LDS so that the reservation stays.
  volatile float* res = reserve;
  res[threadIdx.x] = s;
  sink[(long)blockIdx.x * kProbeThreads + threadIdx.x] = res[threadIdx.x];
  if (lane == 0) {
    const long w = (long)blockIdx.x * kProbeWaves + (threadIdx.x >> 6);
    clocks[2 * w] = t1 - t0;
    clocks[2 * w + 1] = r1 - r0;
  }
}

// Where the dispatcher places workgroups: thread 0 of workgroup w records the
// XCD it runs on (hardware register XCC_ID, bits 3:0) and the HW_ID register
// (SE, CU, SIMD and wave slot of wave 0).  The forward's grid order deals its
// (batch, KV head) units to the XCDs on the premise that workgroup w runs on
// XCD w % 8; this records what the hardware does.  Workgroups of 512 threads
// with the LDS reservation of the probe above, as the forward's.
__global__ __launch_bounds__(kProbeThreads, 1) void xcd_probe_kernel(int32_t* __restrict__ ids) {
  __shared__ float reserve[kProbeLdsFloats];
  if (threadIdx.x == 0) {
    volatile float* res = reserve;
    res[0] = 0.f;  // keeps the reservation
    // s_getreg simm16: register id | offset << 6 | (size - 1) << 11
    const int xcc = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (3 << 11)) + (int)res[0];
    const int hw = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11));
    ids[2 * (long)blockIdx.x] = xcc;
    ids[2 * (long)blockIdx.x + 1] = hw;
  }
}

// ---------------------------------------------------------------------------
// Softmax issue probe: what the exponential costs beside the matrix core.
//
// FlashAttention-4 (papercache summary), section 3.1.3, evaluates part of
// each row's exp2 as a polynomial on the FMA units because on its hardware
// the exponential unit, not the FMA pipes, limits the softmax.  On CDNA4 the
// exponential issues from the same VALU as an FMA, so the question is what
// each form costs in VALU issue, with the other wave of the SIMD streaming
// MFMAs as in the forward's ping-pong.  Waves 0-3 stream
// v_mfma_f32_32x32x16_bf16 (or idle); waves 4-7, one per SIMD beside them, run a softmax-shaped loop:
// per lane and iteration 32 elements, each x = s * c - m (one FMA), e = exp2(x),
// a running sum, a running max (v_max3 over pairs) and packing pairs to bf16 --
// the forward's instruction mix.  The exponential is v_exp_f32 (kind 1), the
// polynomial exp2_poly (kind 2), or the polynomial on 8 of the 32 elements
// (kind 3, the share FlashAttention-4 emulates).  Every wave runs until a
// fixed real-time budget has passed (s_memrealtime always advances, so every
// wave ends) and records its iterations and shader-clock ticks.

// The polynomial is exp2_poly (cdna4.h), the one the forward can use.
template <int KIND>
__global__ __launch_bounds__(kProbeThreads, 1) void softmax_issue_probe_kernel(
    const bf16x8* __restrict__ ops, int mfma_on, uint64_t budget, float c, float dm,
    float* __restrict__ values, uint64_t* __restrict__ stats) {
  __shared__ float reserve[kProbeLdsFloats];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint64_t iters = 0, t0 = 0, t1 = 0, r0 = 0, r1 = 0;
  float chk = 0.f;
  __syncthreads();
  if (wave < 4) {
    if (mfma_on) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = ops[i * 64 + lane];
        b[i] = ops[(4 + i) * 64 + lane];
      }
      f32x16 acc[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = f32x16{};
      r0 = __builtin_amdgcn_s_memrealtime();
      t0 = __builtin_amdgcn_s_memtime();
      do {
        static_for<0, 16>([&](auto I) __attribute__((always_inline)) {
          constexpr int k = decltype(I)::value;
          acc[k % 8] = mfma32(a[k % 4], b[(k + k / 4) % 4], acc[k % 8]);
        });
        ++iters;
      } while (__builtin_amdgcn_s_memrealtime() - r0 < budget);
      t1 = __builtin_amdgcn_s_memtime();
      r1 = __builtin_amdgcn_s_memrealtime();
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) chk += acc[i][e];
    }
  } else if constexpr (KIND != 0) {
    float sc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) sc[i] = (lane + 64 * i) * (1.f / 256.f) - 8.f;  // x in [-8, 0)
    // element i of the loop: polynomial (kind 2, or kind 3 on 8 of the 32), else v_exp_f32
    auto ex = [](int i, float x) __attribute__((always_inline)) {
      return (KIND == 2 || (KIND == 3 && i % 8 < 2)) ? exp2_poly(x) : __builtin_amdgcn_exp2f(x);
    };
    if (blockIdx.x == 0 && wave == 4) {  // the loop's first exponentials, for an accuracy check
#pragma unroll
      for (int i = 0; i < 32; ++i) values[lane * 32 + i] = ex(i, fmaf(sc[i], c, -0.f));
    }
    float m = 0.f, l0 = 0.f, l1 = 0.f, mx = -INFINITY;
    uint32_t pk_x = 0;
    r0 = __builtin_amdgcn_s_memrealtime();
    t0 = __builtin_amdgcn_s_memtime();
    do {
#pragma unroll
      for (int i = 0; i < 32; i += 2) {
        const float e0 = ex(i, fmaf(sc[i], c, -m));
        const float e1 = ex(i + 1, fmaf(sc[i + 1], c, -m));
        l0 += e0;
        l1 += e1;
        mx = max3f(mx, e0, e1);
        const bf16x2 pk = {(__bf16)e0, (__bf16)e1};
        pk_x ^= __builtin_bit_cast(uint32_t, pk);
      }
      m += dm;
      ++iters;
    } while (__builtin_amdgcn_s_memrealtime() - r0 < budget);
    t1 = __builtin_amdgcn_s_memtime();
    r1 = __builtin_amdgcn_s_memrealtime();
    chk = l0 + l1 + mx + static_cast<float>(pk_x & 0xffu);
  }
  volatile float* res = reserve;  // keeps the LDS reservation
  res[threadIdx.x] = chk;
  if (lane == 0) {
    const long w = (long)blockIdx.x * kProbeWaves + wave;
    stats[4 * w] = iters;
    stats[4 * w + 1] = t1 - t0;
    stats[4 * w + 2] = r1 - r0;
    stats[4 * w + 3] = __float_as_uint(res[threadIdx.x]);
  }
}

}  // namespace

extern "C" int attn_probe_softmax_issue(const void* operands, int mfma_on, int exp_kind,
                                        int budget_us, int workgroups, float* values,
                                        uint64_t* stats, void* stream) {
  if (operands == nullptr || values == nullptr || stats == nullptr) return ATTN_ERR_NULL;
  if ((mfma_on != 0 && mfma_on != 1) || exp_kind < 0 || exp_kind > 3 || budget_us < 1 ||
      budget_us > 10000000 || workgroups < 1)
    return ATTN_ERR_SIZE;
  if ((reinterpret_cast<uintptr_t>(operands) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(values) & 3u) != 0 || (reinterpret_cast<uintptr_t>(stats) & 7u) != 0)
    return ATTN_ERR_ALIGN;
  if (workgroups > (INT32_MAX / kProbeThreads)) return ATTN_ERR_TOO_LARGE;
  (void)hipGetLastError();
  const auto* ops = static_cast<const bf16x8*>(operands);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const uint64_t budget = static_cast<uint64_t>(budget_us) * 100u;  // s_memrealtime runs at 100 MHz
  const float c = 1.f, dm = 1e-7f;
  switch (exp_kind) {
    case 0:
      hipLaunchKernelGGL(softmax_issue_probe_kernel<0>, dim3(workgroups), dim3(kProbeThreads), 0, st,
                         ops, mfma_on, budget, c, dm, values, stats);
      break;
    case 1:
      hipLaunchKernelGGL(softmax_issue_probe_kernel<1>, dim3(workgroups), dim3(kProbeThreads), 0, st,
                         ops, mfma_on, budget, c, dm, values, stats);
      break;
    case 2:
      hipLaunchKernelGGL(softmax_issue_probe_kernel<2>, dim3(workgroups), dim3(kProbeThreads), 0, st,
                         ops, mfma_on, budget, c, dm, values, stats);
      break;
    default:
      hipLaunchKernelGGL(softmax_issue_probe_kernel<3>, dim3(workgroups), dim3(kProbeThreads), 0, st,
                         ops, mfma_on, budget, c, dm, values, stats);
      break;
  }
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    attn_detail::last_hip_error = static_cast<int>(err);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

extern "C" int attn_probe_xcd(int workgroups, int32_t* ids, void* stream) {
  if (ids == nullptr) return ATTN_ERR_NULL;
  if (workgroups < 1) return ATTN_ERR_SIZE;
  if ((reinterpret_cast<uintptr_t>(ids) & 7u) != 0) return ATTN_ERR_ALIGN;
  if (workgroups > INT32_MAX / 2) return ATTN_ERR_TOO_LARGE;
  (void)hipGetLastError();
  hipLaunchKernelGGL(xcd_probe_kernel, dim3(workgroups), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), ids);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    attn_detail::last_hip_error = static_cast<int>(err);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

extern "C" int attn_probe_mfma(const void* operands, int shape, int iters, int workgroups,
                               float* sink, uint64_t* clocks, void* stream) {
  if (operands == nullptr || sink == nullptr || clocks == nullptr) return ATTN_ERR_NULL;
  if ((shape != 32 && shape != 16) || iters < 1 || workgroups < 1) return ATTN_ERR_SIZE;
  if ((reinterpret_cast<uintptr_t>(operands) & 15u) != 0 ||
      (reinterpret_cast<uintptr_t>(sink) & 3u) != 0 || (reinterpret_cast<uintptr_t>(clocks) & 7u) != 0)
    return ATTN_ERR_ALIGN;
  if (workgroups > (INT32_MAX / kProbeThreads)) return ATTN_ERR_TOO_LARGE;
  (void)hipGetLastError();  // clear a stale error so the check below is ours
  const auto* ops = static_cast<const bf16x8*>(operands);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (shape == 32)
    hipLaunchKernelGGL(mfma_probe_kernel<32>, dim3(workgroups), dim3(kProbeThreads), 0, st, ops,
                       iters, sink, clocks);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<16>, dim3(workgroups), dim3(kProbeThreads), 0, st, ops,
                       iters, sink, clocks);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) {
    attn_detail::last_hip_error = static_cast<int>(err);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}
