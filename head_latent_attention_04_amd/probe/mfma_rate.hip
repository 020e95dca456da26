// Measurement probe, not part of the attention path: the rate at which the chip sustains
// v_mfma_f32_32x32x16_bf16 work, and the shader clock it runs at while doing so, for a given operand
// content. The decode and prefill kernels multiply random bf16 data; their MFMA rate is set against
// this probe's rate on the same kind of data (and on constant data, which draws less power).
//
// Work-group = 4 waves (one per SIMD, the attention kernel's occupancy: one work-group per compute
// unit). Each wave holds 4 A and 4 B operand registers (16 bytes per lane each, read once from
// `operands`) and runs `iters` iterations of 16 MFMAs over 4 independent accumulators, the operand
// registers rotating from one MFMA to the next so consecutive instructions see different inputs.
// Lane 0 of each wave records the elapsed shader-clock counter (s_memtime) and 100 MHz real-time
// counter (s_memrealtime) around the loop; the accumulators are summed into `sink` so no MFMA is dead.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kMfmaPerIter = 16;
}  // namespace

__global__ void __launch_bounds__(kWaves * 64, 1) mfma_rate_kernel(const u32x4* __restrict__ operands, int iters,
                                                                  float* __restrict__ sink,
                                                                  uint64_t* __restrict__ stamps) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = __builtin_bit_cast(bf16x8, operands[i * 64 + lane]);
    b[i] = __builtin_bit_cast(bf16x8, operands[(4 + i) * 64 + lane]);
  }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = f32x16{};
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaPerIter / 4; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k)
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + k) & 3], b[(j + 3 * k) & 3], acc[k], 0, 0, 0);
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[k][e];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (lane == 0) {
    stamps[((int64_t)blockIdx.x * kWaves + wave) * 2] = t1 - t0;
    stamps[((int64_t)blockIdx.x * kWaves + wave) * 2 + 1] = r1 - r0;
  }
}

// operands: 8 x 64 x 16 bytes (device); sink: blocks x 256 floats; stamps: blocks x 4 x 2 uint64.
// Returns 0 or the HIP error code of the launch.
extern "C" int mla_probe_mfma_rate(const void* operands, int blocks, int iters, float* sink, uint64_t* stamps,
                                   hipStream_t stream) {
  if (!operands || !sink || !stamps || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_rate_kernel, dim3((unsigned)blocks), dim3(kWaves * 64), 0, stream,
                     static_cast<const u32x4*>(operands), iters, sink, stamps);
  return (int)hipGetLastError();
}

// FLOPs one launch performs: blocks x 4 waves x iters x 16 MFMAs x (2 x 32 x 32 x 16).
extern "C" double mla_probe_mfma_flops(int blocks, int iters) {
  return (double)blocks * kWaves * iters * kMfmaPerIter * 2.0 * 32 * 32 * 16;
}
