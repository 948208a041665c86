// Calibration kernels for the roofline (not part of the attention library):
// independent chains of f16 MFMAs on register operands only, no memory
// traffic in the loop.  Their throughput, with the clock and power the card
// holds under them, is the matrix pipe's reachable ceiling on this machine, per
// instruction shape and operand statistics:
//   shape 0: v_mfma_f32_32x32x16_f16, small operands (|x| < 0.02)
//   shape 1: v_mfma_f32_16x16x32_f16, small operands
//   shape 2: v_mfma_f32_32x32x16_f16, operands of about unit variance
//   shape 3: v_mfma_f32_16x16x32_f16, operands of about unit variance
// Every shape does 131072 FLOPs per wave per loop step (four 32x32x16 or
// eight 16x16x32 products).  Under a power limit the operands' bit activity
// moves the clock, hence the two operand kinds.
#include <hip/hip_runtime.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ inline _Float16 small_value(unsigned t, unsigned i, unsigned mul, unsigned add,
                                       unsigned mod) {
  return (_Float16)(((t * mul + i * add) % mod) * 0.001f - 0.015f);
}

// Integer hash to a sum of four uniform bytes, centred and scaled: roughly
// N(0, 1) values, so the multipliers see the bit activity of real data.
__device__ inline _Float16 unit_value(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  float f = (float)((x & 255) + ((x >> 8) & 255) + ((x >> 16) & 255) + (x >> 24)) - 510.f;
  return (_Float16)(f / 148.f);
}

// 8 waves per workgroup (two per SIMD).
template <bool kUnit>
__global__ void __launch_bounds__(512) chain_32x32x16(float* out, int iters) {
  f32x16 acc[4] = {};
  f16x8 a[4], b[4];
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 8; ++i) {
      unsigned t = threadIdx.x;
      a[j][i] = kUnit ? unit_value(t * 131 + j * 17 + i) : small_value(t, i + j, 7, 13, 31);
      b[j][i] = kUnit ? unit_value(t * 977 + j * 29 + i + 7777) : small_value(t, i + j, 5, 11, 29);
    }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[j], b[3 - j], acc[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 4; ++j)
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <bool kUnit>
__global__ void __launch_bounds__(512) chain_16x16x32(float* out, int iters) {
  f32x4 acc[8] = {};
  f16x8 a[4], b[4];
  for (int j = 0; j < 4; ++j)
    for (int i = 0; i < 8; ++i) {
      unsigned t = threadIdx.x;
      a[j][i] = kUnit ? unit_value(t * 131 + j * 17 + i) : small_value(t, i + j, 7, 13, 31);
      b[j][i] = kUnit ? unit_value(t * 977 + j * 29 + i + 7777) : small_value(t, i + j, 5, 11, 29);
    }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j & 3], b[(j >> 1) & 3], acc[j], 0, 0, 0);
  }
  float s = 0.f;
  for (int j = 0; j < 8; ++j)
    for (int r = 0; r < 4; ++r) s += acc[j][r];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

// out: device buffer of blocks * 512 floats; shape as listed above.
// FLOPs = blocks * 8 * iters * 131072.  Returns -1 on a bad argument, else the
// launch's hipError_t.
extern "C" int fa_calib_mfma(float* out, int blocks, int iters, int shape, void* stream) {
  if (!out || blocks <= 0 || iters <= 0 || shape < 0 || shape > 3) return -1;
  hipStream_t s = (hipStream_t)stream;
  switch (shape) {
    case 0: hipLaunchKernelGGL(chain_32x32x16<false>, dim3(blocks), dim3(512), 0, s, out, iters); break;
    case 1: hipLaunchKernelGGL(chain_16x16x32<false>, dim3(blocks), dim3(512), 0, s, out, iters); break;
    case 2: hipLaunchKernelGGL(chain_32x32x16<true>, dim3(blocks), dim3(512), 0, s, out, iters); break;
    default: hipLaunchKernelGGL(chain_16x16x32<true>, dim3(blocks), dim3(512), 0, s, out, iters); break;
  }
  return (int)hipGetLastError();
}
