// Internal interface between the C ABI layer (fa_api.cpp) and the
// key/value-cache kernels (fa_fwd_kvcache.hip).  Not installed, not part of
// the ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {

constexpr int kKvRows = 32;        // query rows per workgroup
constexpr int kKvKeys = 32;        // keys per tile
constexpr int kKvMaxSplits = 256;  // most key ranges one call may use

struct KvArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  void* workspace;  // n_split * BH * Nq * (d + 1) floats when n_split > 1
  int64_t BH;       // B * H
  int64_t Nq;
  int64_t Nk;
  int d;
  float scale;
  bool causal;
  Dtype dtype;
  int n_split;          // key ranges, >= 1
  int tiles_per_split;  // 32-key tiles per range
};

// Waves per workgroup and LDS stages per wave of the cache kernel at head
// dimension d.  A stage is one 32-key K tile and one V tile (128*d bytes); a
// wave keeps kv_bufs - 1 tiles in flight while it computes on another.
// (Two stages at both head dimensions: 128 KiB of LDS per workgroup at d=128
// with 4 waves, and at d=64 with 8 waves.)
constexpr int kv_waves(int d) { return d == 128 ? 4 : 8; }
constexpr int kv_bufs(int) { return 2; }

// Enqueue the cache kernel (and, with n_split > 1, the merge kernel).
hipError_t launch_kvcache(const KvArgs& a, hipStream_t stream);  // FA_F16, FA_BF16

// Bytes of the library's own device scratch for the split partials of the
// allocation-free cache entry point (one array per GPU, held until the
// process ends).  Must equal FA_MI355X_KVCACHE_SCRATCH_BYTES in the header.
constexpr int64_t kKvScratchBytes = (int64_t)16 << 20;

// Device address of that scratch on the current device, looked up once per
// device (hipGetSymbolAddress) and kept.
hipError_t kvcache_scratch(void** ptr);

}  // namespace fa
