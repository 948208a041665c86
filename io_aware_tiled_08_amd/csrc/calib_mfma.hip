// Calibration kernel for the roofline (not part of the attention library):
// independent chains of v_mfma_f32_32x32x16_f16 on register operands only, no
// memory traffic in the loop.  Its throughput, with the clock and power the
// card holds under it, is the matrix pipe's reachable ceiling on this machine.
#include <hip/hip_runtime.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// 8 waves per workgroup (two per SIMD), four independent accumulators per
// wave; operands are small values so the sums stay finite.
__global__ void __launch_bounds__(512) mfma_chain_kernel(float* out, int iters) {
  f32x16 acc[4] = {};
  f16x8 a, b;
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(((threadIdx.x * 7 + i * 13) % 31) * 0.001f - 0.015f);
    b[i] = (_Float16)(((threadIdx.x * 5 + i * 11) % 29) * 0.001f - 0.014f);
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 4; ++j)
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// out: device buffer of blocks * 512 floats.  FLOPs = blocks * 8 * 4 * iters * 32768.
extern "C" int fa_calib_mfma(float* out, int blocks, int iters, void* stream) {
  if (!out || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_chain_kernel, dim3(blocks), dim3(512), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}
