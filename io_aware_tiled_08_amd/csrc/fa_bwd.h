// Internal interface between the C ABI layer (fa_api.cpp) and the backward
// kernels (fa_bwd.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  void* workspace;  // 2 * B * H * N floats: D = rowsum(dO * O), then LSE * log2(e)
  int64_t BH;
  int64_t N;
  int d;
  float scale;
  bool causal;
  Dtype dtype;
};

constexpr int kBwdRowsPerWorkgroup = 128;
constexpr int kBwdThreads = 512;

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream);  // FA_F16, FA_BF16

}  // namespace fa
