// Internal interface between the C ABI layer (fa_api.cpp) and the 8-bit
// forward kernel (fa_fwd_fp8.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace fa {

// Query rows owned by one workgroup of the 8-bit kernel.
constexpr int kRowsPerWorkgroupFp8 = 256;

struct Fp8Args {
  const void* q;  // e4m3 codes, [B, H, N, d]
  const void* k;
  const void* v;
  void* o;        // bf16 [B, H, N, d]
  float* lse;     // [B, H, N]
  int64_t BH;
  int64_t N;
  int d;
  float scale;
  bool causal;
  float q_descale;
  float k_descale;
  float v_descale;
};

hipError_t launch_forward_fp8(const Fp8Args& a, hipStream_t stream);

}  // namespace fa
