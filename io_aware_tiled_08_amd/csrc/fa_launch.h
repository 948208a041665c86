// Internal interface between the C ABI layer (fa_api.cpp) and the gfx950
// kernels (fa_fwd_kernel.hip).  Not installed, not part of the ABI.
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
  int64_t BH;      // B * H
  int64_t N;
  int d;
  float scale;
  bool causal;
  Dtype dtype;
};

// Rows of Q owned by one workgroup for a (dtype, d, causal) choice; the
// caller uses it for the grid-size overflow check.
int rows_per_workgroup(Dtype dtype, int d, bool causal);

// Enqueue the forward kernel on `stream`.  Arguments are already validated.
hipError_t launch_forward(const FwdArgs& a, hipStream_t stream);

}  // namespace fa
