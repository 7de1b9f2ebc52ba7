// Throughput probes for the roofline's measured ceilings (gfx950): fp32
// fused multiply-adds on the vector ALUs, compiled like the scan kernels
// (packed-FP32 instruction selection off, so one v_fma_f32 per lane and
// instruction), and the bf16 MFMA with fp32 accumulation in its 16x16x32 and
// 32x32x16 shapes.  Each
// thread (wave) runs independent accumulation chains long enough to keep the
// pipes full; the results are written out so nothing is optimised away.  Not
// part of the scan's C ABI: a separate library that the benchmark loads.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kChains = 8;

__global__ void __launch_bounds__(kThreads) fma_probe(float* __restrict__ out, int iters) {
  float a[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) a[i] = 1e-3f * static_cast<float>(threadIdx.x + i);
  // x -> x m + c with m just below 1 stays bounded near c / (1 - m)
  const float m = 0.999f, c = 1e-3f;
#pragma unroll 4
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) a[i] = fmaf(a[i], m, c);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += a[i];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__global__ void __launch_bounds__(kThreads) mfma_probe(float* __restrict__ out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1e-3f * static_cast<float>((threadIdx.x + e) & 7));
    b[e] = static_cast<__bf16>(1e-3f * static_cast<float>((threadIdx.x * 3 + e) & 7));
  }
  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 2
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ void __launch_bounds__(kThreads) mfma32_probe(float* __restrict__ out, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(1e-3f * static_cast<float>((threadIdx.x + e) & 7));
    b[e] = static_cast<__bf16>(1e-3f * static_cast<float>((threadIdx.x * 3 + e) & 7));
  }
  f32x16 acc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
#pragma unroll 2
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < 2; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  out[blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

// flops of one launch: fma_probe 2 * kChains per thread and iteration;
// mfma_probe 4 products of 2 * 16 * 16 * 32 per wave and iteration.
extern "C" double ttt_peak_fp32_flops(int32_t blocks, int32_t iters) {
  return 2.0 * kChains * kThreads * static_cast<double>(blocks) * iters;
}
extern "C" double ttt_peak_bf16_mfma_flops(int32_t blocks, int32_t iters) {
  return 4.0 * 2 * 16 * 16 * 32 * (kThreads / 64) * static_cast<double>(blocks) * iters;
}
// mfma32_probe: 2 products of 2 * 32 * 32 * 16 per wave and iteration
extern "C" double ttt_peak_bf16_mfma32_flops(int32_t blocks, int32_t iters) {
  return 2.0 * 2 * 32 * 32 * 16 * (kThreads / 64) * static_cast<double>(blocks) * iters;
}

// Launch one probe on `stream`; `out` holds blocks * 256 floats.  Returns 0,
// or 1 on bad arguments, 2 on a launch error.
extern "C" int32_t ttt_peak_fp32(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(fma_probe, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
extern "C" int32_t ttt_peak_bf16_mfma(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma_probe, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
extern "C" int32_t ttt_peak_bf16_mfma32(float* out, int32_t blocks, int32_t iters, void* stream) {
  if (out == nullptr || blocks < 1 || iters < 1) return 1;
  hipLaunchKernelGGL(mfma32_probe, dim3(blocks), dim3(kThreads), 0,
                     static_cast<hipStream_t>(stream), out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
