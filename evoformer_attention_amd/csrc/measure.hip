// Instruction-throughput probes for the benchmark's ceiling estimate (not
// part of the attention path): each kernel keeps every wave issuing one kind
// of instruction from independent dependency chains, so that the elapsed time
// of a launch divided by the instructions each SIMD issued is that
// instruction's issue interval on this device.  The benchmark compares the
// transcendental and fused-multiply-add intervals with the matrix-core
// interval, whose rate at the published dense peak is known (one
// v_mfma_f32_16x16x32_bf16 per 16 clocks per SIMD), and derives from them
// the fraction of the matrix-core peak the softmax arithmetic leaves room
// for.
#include "evo_device.h"
#include "evo_kernels.h"

namespace evo {
namespace {

// kind 0: v_exp_f32, 8 independent chains x = exp2(-x) (stays in (0, 1]);
// kind 1: v_fma_f32, 8 chains x = x * 0.999 + 0.001;
// kind 2: v_mfma_f32_16x16x32_bf16, 8 independent accumulators.
template <int KIND>
__global__ void __launch_bounds__(256) probe_kernel(float* out, int iters) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = (threadIdx.x + i) * 1e-3f;
  f32x4 acc[8];
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i] = f32x4{x[i], 0.f, 0.f, 0.f};
    a[i] = (__bf16)(x[i] * 0.01f);
    b[i] = (__bf16)(x[7 - i] * 0.01f);
  }
#pragma clang loop unroll(disable)
  for (int it = 0; it < iters; ++it) {
    if constexpr (KIND == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = exp2_fast(-x[i]);
    } else if constexpr (KIND == 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = __builtin_fmaf(x[i], 0.999f, 0.001f);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = mma32(a, b, acc[i]);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) s += x[i] + acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  out[blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

hipError_t launch_probe(int kind, int waves_per_simd, int iters, float* out, hipStream_t s) {
  const dim3 grid(256 * waves_per_simd), block(256);
  if (kind == 0)
    hipLaunchKernelGGL(probe_kernel<0>, grid, block, 0, s, out, iters);
  else if (kind == 1)
    hipLaunchKernelGGL(probe_kernel<1>, grid, block, 0, s, out, iters);
  else
    hipLaunchKernelGGL(probe_kernel<2>, grid, block, 0, s, out, iters);
  return hipGetLastError();
}

}  // namespace evo
