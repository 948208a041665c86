// Device-side pieces shared by the fp32 and the fp16/bf16 forward kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

struct KernelParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t N;
  int32_t n_qblk;   // query blocks per (b, h)
  float c;          // |scale| * log2(e): scores are kept in log2 units
  uint32_t q_sign;  // XOR mask on Q's bits: flips Q's sign when scale < 0
  int64_t n_items;  // B * H * n_qblk (the persistent schedule's item count)
};

template <typename To, typename From>
__device__ __forceinline__ To bits(From x) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, x);
}

// max / sum of x over lanes l and l^32 (the two halves of a 32x32 MFMA
// accumulator column).  v_permlane32_swap exchanges the upper half of its
// first operand with the lower half of its second; with both operands equal
// to x, the two results hold x[l % 32] and x[l % 32 + 32] in every lane.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(bits<uint32_t>(x), bits<uint32_t>(x), false, false);
  return fmaxf(bits<float>(r[0]), bits<float>(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(bits<uint32_t>(x), bits<uint32_t>(x), false, false);
  return bits<float>(r[0]) + bits<float>(r[1]);
}

// max / sum over lanes l, l^16, l^32, l^48 (the four lane groups of a 16x16
// MFMA result column): halves first, then v_permlane16_swap, which exchanges
// the odd 16-lane rows of its first operand with the even rows of its second,
// so with both operands x the results hold x of lanes l and l^16.
__device__ __forceinline__ float quad_max(float x) {
  x = halves_max(x);
  const auto r = __builtin_amdgcn_permlane16_swap(bits<uint32_t>(x), bits<uint32_t>(x), false, false);
  return fmaxf(bits<float>(r[0]), bits<float>(r[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  x = halves_sum(x);
  const auto r = __builtin_amdgcn_permlane16_swap(bits<uint32_t>(x), bits<uint32_t>(x), false, false);
  return bits<float>(r[0]) + bits<float>(r[1]);
}

// In the 32x32 MFMA accumulator, register r of a lane in wave half hh holds
// row 8*(r/4) + 4*hh + r%4.  The kernels feed K so that this row carries key
//   key_of_reg(r, hh) = 16*(r/8) + 8*hh + r%8
// of the 32-key block, i.e. the 8 keys a lane contributes to one 16-deep P V
// MFMA are 8 consecutive keys.  The A-operand lane of row m loads that key:
// bits 2 and 3 of m swapped.
__device__ __forceinline__ constexpr int key_of_reg(int r, int hh) {
  return 16 * (r >> 3) + 8 * hh + (r & 7);
}
__device__ __forceinline__ constexpr int k_row_of_lane(int l32) {
  return (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
}

// Workgroup -> (b*H + h, query block).  The dispatcher hands workgroup i to
// XCD i % 8; the remap gives each XCD a contiguous range of heads, so the
// query blocks of one head share that XCD's L2 copy of the head's K and V.
// Causal launches take the longest query blocks (highest index) first.  With
// at most four workgroups per CU (1024 in all) the order runs across the
// XCD's heads (block-major, when its range holds whole heads), so that each
// XCD starts all its longest blocks before any short one; longer launches
// keep one head at a time per XCD (head-major), which keeps that head's K
// and V hot in the XCD's L2.
struct WorkItem {
  int64_t bh;
  int qblk;
};
template <bool CAUSAL>
__device__ __forceinline__ WorkItem work_item(int n_qblk) {
  const int nblk = gridDim.x;
  const int wg = blockIdx.x;
  WorkItem w;
  if (CAUSAL && nblk <= 1024 && nblk % 8 == 0 && (nblk / 8) % n_qblk == 0) {
    const int heads = nblk / 8 / n_qblk;  // heads per XCD
    const int x = wg % 8, r = wg / 8;     // XCD, order within the XCD
    w.bh = (int64_t)x * heads + r % heads;
    w.qblk = n_qblk - 1 - r / heads;
    return w;
  }
  const int logical = (nblk % 8 == 0) ? (wg % 8) * (nblk / 8) + wg / 8 : wg;
  w.bh = logical / n_qblk;
  w.qblk = logical % n_qblk;
  if (CAUSAL) w.qblk = n_qblk - 1 - w.qblk;
  return w;
}

}  // namespace fa
