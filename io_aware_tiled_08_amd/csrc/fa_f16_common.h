// Device helpers shared by the 16-bit and 8-bit kernels (forward, key-split,
// key/value cache, backward): MFMA wrappers per input type, the LDS
// chunk permutation, transposing LDS reads, direct-to-LDS buffer loads,
// register fences and two forms of a maximum over many values.
#pragma once

#include <type_traits>

#include "fa_device.h"

namespace fa {
namespace {

// Largest excess (log2 units) of a score over the reference maximum before
// the accumulator is rescaled: weights stay <= 2^8 = 256, far inside the
// fp16/bf16 range and exact-ratio in fp32.
constexpr float kRescaleSlack = 8.0f;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Half;

template <>
struct Half<_Float16> {
  using Frag = f16x8;
  using Pair = f16x2;
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  // Round-to-nearest-even pair conversion (v_cvt_pk_f16_f32).
  static __device__ __forceinline__ Pair pack(float x, float y) {
    return __builtin_convertvector((f32x2){x, y}, Pair);
  }
  // acc + p.x + p.y in fp32 (v_dot2 with ones)
  static __device__ __forceinline__ float sum2(Pair p, float acc) {
    const Pair one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(p, one, acc, false);
  }
  // acc[r] + the sum of the four values in x, for every r: a 4x4x4 product
  // (16 blocks, one per four lanes) with an all-ones A operand, in which each
  // output column is one lane's own four B values.
  static __device__ __forceinline__ f32x4 sum4(u32x2 x, f32x4 acc) {
    const f16x4 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_mfma_f32_4x4x4f16(ones, bits<f16x4>(x), acc, 0, 0, 0);
  }
};

template <>
struct Half<__bf16> {
  using Frag = bf16x8;
  using Pair = bf16x2;
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // Round-to-nearest-even pair conversion (v_cvt_pk_bf16_f32).
  static __device__ __forceinline__ Pair pack(float x, float y) {
    return __builtin_convertvector((f32x2){x, y}, Pair);
  }
  static __device__ __forceinline__ float sum2(Pair p, float acc) {
    const Pair one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
  }
  static __device__ __forceinline__ f32x4 sum4(u32x2 x, f32x4 acc) {
    const i16x4 ones = {0x3f80, 0x3f80, 0x3f80, 0x3f80};  // bf16 1.0
    return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(ones, bits<i16x4>(x), acc, 0, 0, 0);
  }
};

// Position of 16-byte chunk c of row r inside the LDS row (rows are 2*D bytes,
// LDS banks repeat every 256 bytes = 16 chunks).  Each map is an XOR with a
// row-dependent mask, so it is its own inverse.
//   K is read as MFMA A rows: 16 lanes read one chunk of 16 different rows
//   (rows distinct mod 16), so those must land in 16 different bank groups.
//   V is read by transposing loads: 32 lanes read 4 chunks of 4 consecutive
//   rows (first row a multiple of 4); those 16 chunks must not collide.
template <int D>
struct Swizzle {
  static_assert(D == 64 || D == 128, "head dim");
  static __device__ __forceinline__ constexpr int k(int r, int c) {
    return D == 128 ? c ^ (r & 15) : c ^ ((r >> 1) & 7);
  }
  static __device__ __forceinline__ constexpr int v(int r, int c) {
    return D == 128 ? c ^ ((r & 3) << 2) : c ^ (((r >> 1) & 1) << 2);
  }
};

// Chunk swizzles for reads of 16x16x32 operands.  K: 16 lanes read one chunk
// of rows 8*(m/4) + m%4 (m = 0..15, plus a block offset in row bits 2, 5 and
// 6), so the 16 rows must land in 16 different bank groups (d = 128: 16-chunk
// rows; d = 64: 8-chunk rows, two rows per bank period, so 8 per half).  V:
// each 32-lane half of a transposing read covers 32 bytes (two chunks) of
// rows 8*g + 0..3, g = 0, 1, so the 8 chunk pairs must not collide.
template <int D>
struct Swizzle16 {
  static_assert(D == 64 || D == 128, "head dim");
  static __device__ __forceinline__ constexpr int k(int r, int c) {
    return D == 128 ? c ^ ((r & 3) | (((r >> 3) & 3) << 2))
                    : c ^ (((r >> 1) & 1) | (((r >> 3) & 3) << 1));
  }
  static __device__ __forceinline__ constexpr int v(int r, int c) {
    return D == 128 ? c ^ (2 * ((r & 3) | (((r >> 3) & 1) << 2)))
                    : c ^ (2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1)));
  }
};

// v_mfma_f32_16x16x32_{f16,bf16}: A lane l supplies row l%16 and k = 8*(l/16)
// .. +7, B lane l column l%16 with the same k, and the four result registers
// of lane l hold rows 4*(l/16) + r of column l%16.
template <typename T>
__device__ __forceinline__ f32x4 mma16(typename Half<T>::Frag a, typename Half<T>::Frag b, f32x4 c) {
  if constexpr (std::is_same_v<T, __bf16>)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

typedef short s16x4 __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;

// ds_read_b64_tr_b16: within each group of 16 lanes, output lane i, element
// e receives element i%4 of the 4 elements addressed by lane 4*e + i/4.  When
// lane j of the group addresses row r0 + j/4, columns c0 + 4*(j%4) .. +3 of a
// row-major 16-bit matrix, output lane i receives column c0 + i of rows
// r0 .. r0+3, i.e. a transposed 4 x 16 block.
__device__ __forceinline__ u32x2 lds_read_tr(const char* base, int byte_off) {
  lds_s16x4* ptr = (lds_s16x4*)((lds_char*)const_cast<char*>(base) + byte_off);
  return bits<u32x2>(__builtin_amdgcn_ds_read_tr16_b64_v4i16(ptr));
}

// Raw buffer resource over [base, base + bytes): buffer loads at offsets
// >= bytes return zeros.  Dword 3 is the gfx9 raw-buffer format word.
__device__ __forceinline__ u32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// buffer_load_dwordx4 ... lds: lane i copies the 16 bytes at buffer offset
// voff into LDS bytes lds + 16*i .. +15.  Issued from inline assembly so that
// the compiler's wait-count pass does not make every later LDS read wait for
// these loads (it cannot tell the double buffers apart); the kernel waits for
// them itself (vmcnt(0) + barrier) before the first read of the buffer.  M0
// holds the LDS base; nothing else in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma_load16(u32x4 rsrc, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_char*)const_cast<void*>(p);
}

// Issue priority of the calling wave (s_setprio).  In the kernels whose two
// wave groups alternate between a matrix-product phase and a softmax phase,
// the wave in its product phase runs at priority 1 and its SIMD partner at 0:
// when both have an instruction ready, the matrix product (which shares the
// SIMD's vector issue) goes first, and the softmax work fills the cycles in
// between.  The scheduling barriers keep the compiler from moving work across.
template <int P>
__device__ __forceinline__ void wave_priority() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_setprio(P);
  __builtin_amdgcn_sched_barrier(0);
}

// Register fences.  The compiler may move plain arithmetic across
// s_barrier (only memory effects are ordered by it); an empty volatile asm
// that reads and rewrites a value pins the computation of that value before
// the fence and every later use after it, which keeps each phase's work
// inside its slot.
template <typename V>
__device__ __forceinline__ void fence(V& x) {
  asm volatile("" : "+v"(x));
}

// Maximum of n values get(0..n-1) as a balanced tree of three-input maxima
// (v_max3_f32), so the dependency chain is log3(n) deep instead of n.
template <int n, typename Get>
__device__ __forceinline__ float tree_max(Get get) {
  if constexpr (n == 1) {
    return get(0);
  } else if constexpr (n == 2) {
    return fmaxf(get(0), get(1));
  } else {
    constexpr int a = (n + 2) / 3, b = (n - a + 1) / 2, c = n - a - b;
    const float x = tree_max<a>(get);
    const float y = tree_max<b>([&](int i) { return get(a + i); });
    const float z = tree_max<c>([&](int i) { return get(a + b + i); });
    return fmaxf(fmaxf(x, y), z);
  }
}

// Maximum of n values get(0..n-1) as four chains of three-input maxima
// (v_max3_f32): (n - 1) / 2 + 2 instructions, against about 0.65 n for a
// balanced tree; the chains are independent, so their latencies overlap.
template <int n, typename Get>
__device__ __forceinline__ float chain_max4(Get get) {
  static_assert(n % 4 == 0 && n >= 12, "four chains of at least three values");
  constexpr int L = n / 4;
  float m[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    float x = __builtin_fmaxf(__builtin_fmaxf(get(c * L), get(c * L + 1)), get(c * L + 2));
    int i = 3;
#pragma unroll
    for (; i + 1 < L; i += 2) x = __builtin_fmaxf(__builtin_fmaxf(x, get(c * L + i)), get(c * L + i + 1));
    if (i < L) x = __builtin_fmaxf(x, get(c * L + i));
    m[c] = x;
  }
  return __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(m[0], m[1]), m[2]), m[3]);
}

}  // namespace
}  // namespace fa
