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
constexpr int kRowsPerWorkgroupF16KeySplit = 128;
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
// Persistent schedule: n_wg workgroups (1 <= n_wg <= B*H*ceil(N/256)) loop
// over the 256-row blocks (FA_F16, FA_BF16).
hipError_t launch_forward_f16_persistent(const FwdArgs& a, int n_wg, hipStream_t stream);
// Key-split schedule (d = 64 only): 128-row workgroups whose two wave groups
// take alternate key tiles; for causal problems with few 256-row blocks.
hipError_t launch_forward_f16_keysplit(const FwdArgs& a, hipStream_t stream);

// Whether an fp32 problem runs on the 4-row kernel (fwd_f32_q4_kernel):
// d = 64 and a small problem, where one workgroup per 32-row block would
// leave most CUs idle.  Every 4-row workgroup reads all of its head's K and V
// (N * 512 bytes), B*H*N/4 workgroups in all, so the limit on B*H*N^2 keeps
// that re-reading from L2 small (one head of 512 queries reads 32 MiB).
inline bool use_f32_q4(int d, int64_t BH, int64_t N) {
  return d == 64 && N <= 4096 && BH * N * N <= ((int64_t)1 << 20);
}

// Whether flash_attn_fwd uses the key-split schedule: causal, d = 64, and at
// most two 256-row blocks per CU of the MI355X (256 CUs), where the
// longest-first dispatch of 256-row blocks leaves CUs idle.
inline bool use_keysplit(Dtype dtype, int d, bool causal, int64_t BH, int64_t N) {
  return dtype != Dtype::F32 && d == 64 && causal &&
         BH * ((N + kRowsPerWorkgroupF16 - 1) / kRowsPerWorkgroupF16) <= 2 * 256;
}

// Whether flash_attn_fwd runs an unmasked fp16/bf16 problem on the persistent
// schedule (one workgroup per CU, each running its 256-row blocks as one tile
// stream): from two blocks per CU on, where the grid schedule pays every
// block's pipeline fill and drain, Q load and O store in series.
inline bool use_stream(Dtype dtype, bool causal, int64_t BH, int64_t N, int cus) {
  return dtype != Dtype::F32 && !causal && cus > 0 &&
         BH * ((N + kRowsPerWorkgroupF16 - 1) / kRowsPerWorkgroupF16) >= 2 * (int64_t)cus;
}

}  // namespace fa
