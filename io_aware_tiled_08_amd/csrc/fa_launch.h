// Internal interface between the C ABI layer (fa_api.cpp) and the gfx950
// kernels (fa_fwd_f16.hip, fa_fwd_f32.hip).  Not installed, not part of the
// ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

enum class Dtype : int { F32 = 0, F16 = 1, BF16 = 2 };

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t BH;  // B * H
  int64_t N;
  int d;
  float scale;
  bool causal;
  Dtype dtype;
};

// Query rows owned by one workgroup (fixes the grid size).
constexpr int kRowsPerWorkgroupF16 = 256;
constexpr int kRowsPerWorkgroupF32 = 32;

inline int rows_per_workgroup(Dtype dtype) {
  return dtype == Dtype::F32 ? kRowsPerWorkgroupF32 : kRowsPerWorkgroupF16;
}

// Threads per workgroup of the forward kernel (the dispatch's total thread
// count, workgroups x this, must fit 32 bits).
inline int threads_per_workgroup(Dtype dtype, int d) {
  return dtype == Dtype::F32 ? (d == 64 ? 8 : 4) * 64 : 512;
}

// Enqueue the forward kernel on `stream`; arguments are already validated.
hipError_t launch_forward_f16(const FwdArgs& a, hipStream_t stream);  // FA_F16, FA_BF16
hipError_t launch_forward_f32(const FwdArgs& a, hipStream_t stream);

}  // namespace fa
