// mfma_peak.hip -- measures the bf16 matrix-core rate this part sustains at
// the clock of the run: every wave issues back-to-back
// v_mfma_f32_32x32x16_bf16 on eight independent accumulators (no memory
// traffic in the loop).  Built into its own small library, separate from the
// attention library; the benchmark divides its attention FLOP rate by this.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kAcc = 8;   // independent accumulators per wave (8 x 32 cycles >> MFMA latency)

__global__ __launch_bounds__(256) void mfma_peak_kernel(float* out, int iters) {
  f32x16_t acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) acc[i] = f32x16_t{};
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)((threadIdx.x & 7) * 0.125f);
    b[i] = (__bf16)(i * 0.0625f);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kAcc; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// FLOPs one launch of pa_mfma_peak_run performs.
double pa_mfma_peak_flops(int blocks, int iters) {
  return (double)blocks * 4 /* waves */ * iters * kAcc * (2.0 * 32 * 32 * 16);
}

// Launches `blocks` work-groups of 4 waves, each wave running `iters`
// rounds of kAcc MFMAs; out: device buffer of blocks * 256 floats.  Returns
// the hipError_t of the launch.
int pa_mfma_peak_run(float* out, int blocks, int iters, hipStream_t stream) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(blocks), dim3(256), 0, stream, out, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
