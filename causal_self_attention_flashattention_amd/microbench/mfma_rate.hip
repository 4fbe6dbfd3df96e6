// Sustained rate of v_mfma_f32_32x32x16_bf16 on gfx950 with nothing else in the loop, at 1, 2 and 4
// waves per SIMD, with 1 or 4 independent accumulator chains per wave; then the same for
// v_mfma_f32_16x16x32_bf16 (half the flops per instruction), which the kernels use for the last
// 16 output columns of head dims 16 modulo 32.
//
// Each launch runs one 256-thread workgroup (one wave per SIMD) per CU and per wave-per-SIMD step
// (256 x w workgroups in all); each wave issues 8 x kIters products (2 x 32 x 32 x 16 flops each),
// then writes one float per thread.  Run it under `rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES
// SQ_BUSY_CYCLES GRBM_GUI_ACTIVE` to read the clock (GRBM_GUI_ACTIVE per XCD over the launch time)
// and the matrix-core busy share the rate corresponds to.
#include <hip/hip_runtime.h>

#include <cstdio>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kIters = 16384;

template <int CH>
__global__ __launch_bounds__(256) void chains(float* out) {
  const int l = threadIdx.x & 63;
  bf16x8 a, b;
  for (int s = 0; s < 8; ++s) {
    a[s] = (__bf16)(0.001f * (l + s));
    b[s] = (__bf16)(0.002f * (l - s));
  }
  f32x16 c[CH] = {};
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) c[r % CH] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[r % CH], 0, 0, 0);
  }
  float sum = 0.f;
  for (int k = 0; k < CH; ++k)
    for (int e = 0; e < 16; ++e) sum += c[k][e];
  out[blockIdx.x * 256 + threadIdx.x] = sum;
}

template <int CH>
__global__ __launch_bounds__(256) void chains16(float* out) {
  const int l = threadIdx.x & 63;
  bf16x8 a, b;
  for (int s = 0; s < 8; ++s) {
    a[s] = (__bf16)(0.001f * (l + s));
    b[s] = (__bf16)(0.002f * (l - s));
  }
  f32x4 c[CH] = {};
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) c[r % CH] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[r % CH], 0, 0, 0);
  }
  float sum = 0.f;
  for (int k = 0; k < CH; ++k)
    for (int e = 0; e < 4; ++e) sum += c[k][e];
  out[blockIdx.x * 256 + threadIdx.x] = sum;
}

template <int CH, bool S16 = false>
void run(float* out, int waves_per_simd) {
  const int grid = 256 * waves_per_simd;
  hipEvent_t e0, e1;
  hipEventCreate(&e0);
  hipEventCreate(&e1);
  auto kern = S16 ? chains16<CH> : chains<CH>;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, 0, out);  // warm-up
  hipEventRecord(e0);
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), 0, 0, out);
  hipEventRecord(e1);
  hipEventSynchronize(e1);
  float ms = 0.f;
  hipEventElapsedTime(&ms, e0, e1);
  const double flops = 8.0 * kIters * grid * 4 * (S16 ? 16384.0 : 32768.0);
  printf("%s waves/SIMD=%d chains/wave=%d  %8.3f ms  %7.1f TFLOP/s\n", S16 ? "16x16x32" : "32x32x16", waves_per_simd, CH,
         ms, flops / (ms * 1e-3) / 1e12);
  hipEventDestroy(e0);
  hipEventDestroy(e1);
}

}  // namespace

int main() {
  float* out = nullptr;
  if (hipMalloc(&out, 4 * 256 * 256 * sizeof(float)) != hipSuccess) return 1;
  for (int w : {1, 2, 4}) {
    run<1>(out, w);
    run<4>(out, w);
  }
  for (int w : {1, 2}) {
    run<1, true>(out, w);
    run<4, true>(out, w);
  }
  hipFree(out);
  printf("done\n");
  return 0;
}
