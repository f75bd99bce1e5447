// MFMA throughput microbenchmark for the benchmark report: the dense matrix
// peak this part sustains under the same launch shape as the attention
// kernel (one workgroup of 4 wavefronts per CU, one wavefront per SIMD), with
// independent accumulator chains so that every MFMA issues back to back.
// Not part of the attention library's interface; bench.py loads it to put a
// measured peak next to the published one.
#include <hip/hip_runtime.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kChains = 8;  // enough independent accumulators to cover the MFMA latency

template <bool F8>
__global__ __launch_bounds__(256) void mfma_loop(int iters, float* out) {
  const int lane = threadIdx.x & 63;
  f32x16 c[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k) c[k] = f32x16{};
  if constexpr (F8) {
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = 0x38383838 ^ (lane & 1);
      b[e] = 0x30303030 ^ (e & 1);
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < kChains; ++k)
        c[k] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[k], 0, 0, 0, 127, 0, 127);
    }
  } else {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (__bf16)(0.001f * (lane + e));
      b[e] = (__bf16)(0.002f * (lane - e));
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int k = 0; k < kChains; ++k) c[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[k], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[k][e];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// Measured dense MFMA rate in TFLOP/s: fp8 != 0 for the e4m3 32x32x64 MFMA,
// else the bf16 32x32x16 one.  Runs on the current device and stream 0,
// synchronously (a warm-up launch, then `reps` timed ones); returns a
// negative value on a HIP error.
extern "C" double fp2_microbench_mfma_tflops(int fp8, int iters, int reps) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1.0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1.0;
  float* out = nullptr;
  if (hipMalloc(&out, (size_t)cus * 256 * sizeof(float)) != hipSuccess) return -1.0;
  hipEvent_t e0, e1;
  if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) return -1.0;
  auto launch = [&]() {
    if (fp8)
      hipLaunchKernelGGL(mfma_loop<true>, dim3(cus), dim3(256), 0, 0, iters, out);
    else
      hipLaunchKernelGGL(mfma_loop<false>, dim3(cus), dim3(256), 0, 0, iters, out);
  };
  launch();
  hipEventRecord(e0, 0);
  for (int r = 0; r < reps; ++r) launch();
  hipEventRecord(e1, 0);
  double res = -1.0;
  if (hipEventSynchronize(e1) == hipSuccess) {
    float ms = 0.f;
    hipEventElapsedTime(&ms, e0, e1);
    const double flop_per_mfma = fp8 ? 2.0 * 32 * 32 * 64 : 2.0 * 32 * 32 * 16;
    const double flops = (double)cus * 4 * kChains * (double)iters * reps * flop_per_mfma;
    res = flops / (ms * 1e-3) / 1e12;
  }
  hipEventDestroy(e0);
  hipEventDestroy(e1);
  hipFree(out);
  return hipGetLastError() == hipSuccess ? res : -1.0;
}
