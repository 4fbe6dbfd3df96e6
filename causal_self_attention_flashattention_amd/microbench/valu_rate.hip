// Vector-ALU issue rates on gfx950, alone and beside v_mfma_f32_32x32x16_bf16, for the vector
// instructions of the attention kernels' softmax: v_fma_f32, v_exp_f32, v_max3_f32,
// v_cvt_pk_bf16_f32, v_dot2c_f32_bf16 and v_mul_f32.
//
// Alone: every wave runs kIters iterations of 8 independent chains of one instruction and reads the
// shader clock (s_memtime) before and after; the figure is clock cycles per instruction per wave.
// Beside the matrix core: every iteration issues 8 products (two accumulator chains) and, after
// each product, K instructions of one kind (kept in that order by sched_group_barrier); the figure is
// clock cycles per product per wave, 32 when the matrix core alone sets the pace.
//
// Launches hold one workgroup of 64 * W threads per CU (W waves, one per SIMD for W = 4, two for
// W = 8); every wave writes one float per lane.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <vector>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kIters = 2048;
constexpr int kCUs = 256;

enum Op { kFma = 0, kExp, kMax3, kCvtPk, kDot2, kMul, kOps };
const char* kNames[kOps] = {"v_fma_f32", "v_exp_f32", "v_max3_f32", "v_cvt_pk_bf16_f32", "v_dot2c_f32_bf16",
                            "v_mul_f32"};

// One instruction of kind OP on chain x (u: a per-lane operand).
template <int OP>
__device__ __forceinline__ float op(float x, float u) {
  if constexpr (OP == kFma) return __builtin_fmaf(x, u, 0.5f);
  if constexpr (OP == kExp) return __builtin_amdgcn_exp2f(-x);
  if constexpr (OP == kMax3) return fmaxf(fmaxf(x, u), -x);
  if constexpr (OP == kCvtPk) {
    // round two floats to a bf16 pair and reinterpret as a float: one v_cvt_pk_bf16_f32
    const bf16x2 p = {(__bf16)x, (__bf16)x};
    return __builtin_bit_cast(float, p);
  }
  if constexpr (OP == kDot2) {
    const bf16x2 a = __builtin_bit_cast(bf16x2, u);
    return __builtin_amdgcn_fdot2_f32_bf16(a, a, x, false);
  }
  if constexpr (OP == kMul) return x * u;
  return x;
}

__device__ __forceinline__ unsigned long long clk() { return __builtin_amdgcn_s_memtime(); }

template <int OP>
__global__ __launch_bounds__(512) void alone(float* out, unsigned long long* cyc) {
  const int l = threadIdx.x & 63;
  const float u = 0.75f + 0.001f * l;
  float x[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = 0.1f * (c + 1) + 0.0001f * l;
  __syncthreads();
  const unsigned long long t0 = clk();
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) x[c] = op<OP>(x[c], u);
  }
  const unsigned long long t1 = clk();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += x[c];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (l == 0) cyc[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
}

template <int OP, int K>
__global__ __launch_bounds__(512) void beside(float* out, unsigned long long* cyc) {
  const int l = threadIdx.x & 63;
  const float u = 0.75f + 0.001f * l;
  bf16x8 a, b;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    a[s] = (__bf16)(0.001f * (l + s));
    b[s] = (__bf16)(0.002f * (l - s));
  }
  f32x16 acc[2] = {};
  float x[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) x[c] = 0.1f * (c + 1) + 0.0001f * l;
  __syncthreads();
  const unsigned long long t0 = clk();
  for (int it = 0; it < kIters; ++it) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      acc[r & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[r & 1], 0, 0, 0);
#pragma unroll
      for (int k = 0; k < K; ++k) x[(r * K + k) & 7] = op<OP>(x[(r * K + k) & 7], u);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (K > 0) __builtin_amdgcn_sched_group_barrier(0x002, K, 0);
    }
  }
  const unsigned long long t1 = clk();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += x[c];
#pragma unroll
  for (int e = 0; e < 16; ++e) s += acc[0][e] + acc[1][e];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  if (l == 0) cyc[blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64] = t1 - t0;
}

float* g_out = nullptr;
unsigned long long* g_cyc = nullptr;

// Median over waves of the cycles each wave measured, divided by `per`.
template <class Kern>
double median_cycles(Kern kern, int waves, double per) {
  const int threads = 64 * waves;
  hipLaunchKernelGGL(kern, dim3(kCUs), dim3(threads), 0, 0, g_out, g_cyc);  // warm-up
  hipLaunchKernelGGL(kern, dim3(kCUs), dim3(threads), 0, 0, g_out, g_cyc);
  if (hipDeviceSynchronize() != hipSuccess) return -1.0;
  std::vector<unsigned long long> c(kCUs * waves);
  if (hipMemcpy(c.data(), g_cyc, c.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost) != hipSuccess)
    return -1.0;
  std::nth_element(c.begin(), c.begin() + c.size() / 2, c.end());
  return (double)c[c.size() / 2] / per;
}

template <int OP>
void run_op() {
  for (int w : {4, 8}) {
    const double a = median_cycles(alone<OP>, w, 8.0 * kIters);
    printf("%-18s alone        waves/SIMD=%d  %6.2f cycles per instruction per wave\n", kNames[OP], w / 4, a);
  }
  for (int w : {4, 8}) {
    const double per = 8.0 * kIters;
    printf("%-18s beside MFMA  waves/SIMD=%d  K=1,2,3,4,6,8: cycles per product per wave", kNames[OP], w / 4);
    printf(" %6.1f", median_cycles(beside<OP, 1>, w, per));
    printf(" %6.1f", median_cycles(beside<OP, 2>, w, per));
    printf(" %6.1f", median_cycles(beside<OP, 3>, w, per));
    printf(" %6.1f", median_cycles(beside<OP, 4>, w, per));
    printf(" %6.1f", median_cycles(beside<OP, 6>, w, per));
    printf(" %6.1f\n", median_cycles(beside<OP, 8>, w, per));
  }
}

}  // namespace

int main() {
  if (hipMalloc(&g_out, kCUs * 512 * sizeof(float)) != hipSuccess) return 1;
  if (hipMalloc(&g_cyc, kCUs * 8 * sizeof(unsigned long long)) != hipSuccess) return 1;
  for (int w : {4, 8})
    printf("v_mfma_f32_32x32x16_bf16 alone waves/SIMD=%d  %6.2f cycles per product per wave\n", w / 4,
           median_cycles(beside<kFma, 0>, w, 8.0 * kIters));
  run_op<kFma>();
  run_op<kExp>();
  run_op<kMax3>();
  run_op<kCvtPk>();
  run_op<kDot2>();
  run_op<kMul>();
  hipFree(g_out);
  hipFree(g_cyc);
  printf("done\n");
  return 0;
}
