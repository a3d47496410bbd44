// mfma_peak.hip -- measures the bf16 matrix-core rate this part sustains at
// the clock of the run: every wave issues back-to-back
// v_mfma_f32_32x32x16_bf16 on eight independent accumulators (no memory
// traffic in the loop).  Built into its own small library, separate from the
// attention library; the benchmark divides its attention FLOP rate by this.
//
// Two operand modes.  Constant operands (the same bf16 values in every lane
// and every MFMA) barely toggle the multipliers; random operands (four
// register sets of bf16 values hashed from the lane, the work-group and the
// set, cycled so consecutive MFMAs differ) draw the power that real data
// draws, and the part's power management then lowers the shader clock.  Each
// work-group records its shader clock: s_memtime (shader clock cycles) and
// s_memrealtime (a fixed 100 MHz counter) at its start and end.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kAcc = 8;   // independent accumulators per wave (8 x 32 cycles >> MFMA latency)
constexpr int kSets = 4;  // operand register sets

// 32-bit integer finaliser (xorshift-multiply rounds): operand bits only
__device__ __forceinline__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x21f0aaadu;
  x ^= x >> 15;
  x *= 0x735a2d97u;
  x ^= x >> 15;
  return x;
}

template <bool kRandom>
__global__ __launch_bounds__(256) void mfma_peak_kernel(float* out, uint64_t* clk, int iters) {
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  f32x16_t acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) acc[i] = f32x16_t{};
  bf16x8_t a[kSets], b[kSets];
#pragma unroll
  for (int j = 0; j < kSets; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (kRandom) {
        // values uniform in [-1, 1)
        const uint32_t h = hash32((threadIdx.x * 977u + blockIdx.x * 65537u) ^ (uint32_t)(j * 8 + i) * 0x9e3779b9u);
        a[j][i] = (__bf16)((float)(int)(h & 0xffffu) * (1.f / 32768.f) - 1.f);
        b[j][i] = (__bf16)((float)(int)(h >> 16) * (1.f / 32768.f) - 1.f);
      } else {
        a[j][i] = (__bf16)((threadIdx.x & 7) * 0.125f);
        b[j][i] = (__bf16)(i * 0.0625f);
      }
    }
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kAcc; ++i)
      acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i % kSets], b[(i / 2) % kSets], acc[i], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kAcc; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[i][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  const uint64_t c1 = __builtin_amdgcn_s_memtime();
  if (clk && threadIdx.x < 4)
    clk[4 * (int64_t)blockIdx.x + threadIdx.x] = threadIdx.x == 0 ? r0 : threadIdx.x == 1 ? r1 : threadIdx.x == 2 ? c0 : c1;
}

}  // namespace

extern "C" {

// FLOPs one launch of pa_mfma_peak_run performs.
double pa_mfma_peak_flops(int blocks, int iters) {
  return (double)blocks * 4 /* waves */ * iters * kAcc * (2.0 * 32 * 32 * 16);
}

// Launches `blocks` work-groups of 4 waves, each wave running `iters`
// rounds of kAcc MFMAs; random_operands: 0 constant operands, 1 random ones.
// out: device buffer of blocks * 256 floats; clk: null, or a device buffer
// of blocks * 4 uint64 that receives per work-group (s_memrealtime at start,
// at end, s_memtime at start, at end).  Returns the hipError_t of the
// launch.
int pa_mfma_peak_run(float* out, uint64_t* clk, int blocks, int iters, int random_operands, hipStream_t stream) {
  if (!out || blocks <= 0 || iters <= 0) return (int)hipErrorInvalidValue;
  if (random_operands)
    hipLaunchKernelGGL(mfma_peak_kernel<true>, dim3(blocks), dim3(256), 0, stream, out, clk, iters);
  else
    hipLaunchKernelGGL(mfma_peak_kernel<false>, dim3(blocks), dim3(256), 0, stream, out, clk, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
