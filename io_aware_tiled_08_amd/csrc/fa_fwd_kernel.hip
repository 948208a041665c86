// FlashAttention forward pass for gfx950 (CDNA4, MI355X).
//
// What is computed: exact attention O = softmax(scale * Q K^T) V and the
// natural-log log-sum-exp of each score row, for every (batch, head).
//
// How (the method of the FlashAttention explainer pages, mapped onto CDNA4):
//   * Tiling ("FlashAttention, Playable", EP 03; chapter 15 "The Tiling
//     Strategy"): each workgroup owns a block of query rows and walks the keys
//     one tile at a time.  K and V tiles are staged through LDS (double
//     buffered: the next tile's global loads are in flight while the current
//     tile is consumed); the block's Q stays in registers for the whole loop.
//   * Fusion ("FlashAttention: Tiled & Fused", section on speed and memory):
//     scores, softmax and the P V product happen in one kernel; scores and
//     probabilities live only in registers and O is written once at the end.
//   * Online softmax ("FlashAttention, Playable", EP 04): per query row a
//     running maximum m and running sum l; when a tile raises the maximum the
//     accumulator and l are multiplied by exp(m_old - m_new).
//
// CDNA4 mapping (not from the pages):
//   * Both products are 32x32 MFMA blocks with fp32 accumulation
//     (v_mfma_f32_32x32x16_{f16,bf16}; v_mfma_f32_32x32x2_f32 for fp32 input).
//   * Scores are produced transposed, S^T = K Q^T: in the 32x32 accumulator a
//     lane holds one column (one query) and 16 of the 32 rows (keys), the
//     other 16 sitting in lane l^32.  Row max and row sum are therefore mostly
//     in-lane with one exchange between the two wave halves, and the rescale
//     factor is a per-lane scalar.
//   * O is accumulated transposed too, O^T += V^T P^T: P^T is the B operand
//     straight from the score registers (converted to fp16/bf16), so P never
//     touches LDS.  The rows of K fed to the first product are permuted within
//     each 32-key block (bits 2 and 3 of the row index swapped) so that the 8
//     keys a lane contributes per MFMA are 8 consecutive keys; V is stored
//     transposed in LDS, so that operand is one 16-byte LDS read.
//   * exp is computed as exp2 with log2(e) folded into the scale; m is kept in
//     those log2 units.
//   * Workgroup ids are remapped so consecutive query blocks of one head land
//     on the same XCD (dispatch round-robins workgroups over the 8 XCDs) and
//     share its L2 copy of that head's K and V; causal launches start with the
//     longest query blocks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_launch.h"

namespace fa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

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
  int32_t n_qblk;    // query blocks per (b, h)
  float c;           // |scale| * log2(e)
  uint32_t q_sign;   // XOR mask applied to Q bits: flips Q's sign for scale < 0
};

// Per-element-type MFMA and packing helpers.
template <typename T>
struct Elem;

template <>
struct Elem<_Float16> {
  static constexpr int KG = 8;  // contraction elements a lane feeds per MFMA
  using Frag = f16x8;
  using Pair = f16x2;
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Pair pack(float x, float y) {
    Pair p;
    p[0] = (_Float16)x;
    p[1] = (_Float16)y;
    return p;
  }
  static __device__ __forceinline__ float sum2(Pair p, float acc) {
    const Pair one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(p, one, acc, false);
  }
};

template <>
struct Elem<__bf16> {
  static constexpr int KG = 8;
  using Frag = bf16x8;
  using Pair = bf16x2;
  static __device__ __forceinline__ f32x16 mma(Frag a, Frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ Pair pack(float x, float y) {
    Pair p;
    p[0] = (__bf16)x;
    p[1] = (__bf16)y;
    return p;
  }
  static __device__ __forceinline__ float sum2(Pair p, float acc) {
    const Pair one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
  }
};

template <>
struct Elem<float> {
  static constexpr int KG = 1;
  using Frag = float;
  static __device__ __forceinline__ f32x16 mma(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

template <typename To, typename From>
__device__ __forceinline__ To bits(From x) {
  static_assert(sizeof(To) == sizeof(From), "size mismatch");
  return __builtin_bit_cast(To, x);
}

// Value of x held by the lane in the other half of the wave (lane ^ 32).
__device__ __forceinline__ float other_half(float x) {
  return __shfl_xor(x, 32, 64);
}

// Key (within a 32-key block) carried by accumulator register r of a lane in
// wave half hh, given the permuted K rows described at the top of the file.
__device__ __forceinline__ constexpr int key_of_reg(int r, int hh) {
  return 16 * (r >> 3) + 8 * hh + (r & 7);
}

// K row (within a 32-key block) that lane l32 feeds as A-operand row l32:
// bits 2 and 3 swapped, so that S^T row m = 8a + 4b + c holds key
// 16(a>>1) + 8b + 4(a&1) + c.
__device__ __forceinline__ constexpr int k_row_of_lane(int l32) {
  return (l32 & ~12) | ((l32 & 4) << 1) | ((l32 & 8) >> 1);
}

// T: element type; D: head dim; NW: waves per workgroup; QB: 32-query blocks
// per wave; BC: keys per tile.
template <typename T, int D, bool CAUSAL, int NW, int QB, int BC>
__global__ void __launch_bounds__(NW * 64, 1) fwd_kernel(KernelParams p) {
  using E = Elem<T>;
  using Frag = typename E::Frag;
  constexpr bool kHalf = sizeof(T) == 2;
  constexpr int KG = E::KG;
  constexpr int KSTEP = 2 * KG;           // contraction depth of one MFMA
  constexpr int NT = NW * 64;             // threads per workgroup
  constexpr int BR = NW * QB * 32;        // query rows per workgroup
  constexpr int EPC = 16 / sizeof(T);     // elements per 16-byte chunk
  constexpr int CPR = D / EPC;            // 16-byte chunks per row of K or V
  constexpr int KS = D + EPC;             // LDS row stride of K (elements)
  constexpr int VS = BC + (kHalf ? 8 : 4);  // LDS row stride of V^T
  constexpr int NKB = BC / 32;            // 32-key blocks per tile
  constexpr int NKS = D / KSTEP;          // MFMAs per 32x32 score block
  constexpr int ND = D / 32;              // 32-row blocks of O^T
  constexpr int NJ = 32 / KSTEP;          // MFMAs per 32 keys in P V
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) T k_lds[2][BC * KS];
  __shared__ __attribute__((aligned(16))) T vt_lds[2][D * VS];

  // ---- work decomposition ---------------------------------------------------
  const int nblk = gridDim.x;
  const int wg = blockIdx.x;
  const int logical = (nblk % 8 == 0) ? (wg % 8) * (nblk / 8) + wg / 8 : wg;
  const int64_t bh = logical / p.n_qblk;
  int qblk = logical % p.n_qblk;
  if (CAUSAL) qblk = p.n_qblk - 1 - qblk;  // longest blocks first

  const int64_t N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t q0 = (int64_t)qblk * BR;
  const int64_t qw = q0 + (int64_t)wave * (QB * 32);

  const T* __restrict__ Qh = (const T*)p.q + bh * N * D;
  const T* __restrict__ Kh = (const T*)p.k + bh * N * D;
  const T* __restrict__ Vh = (const T*)p.v + bh * N * D;
  T* __restrict__ Oh = (T*)p.o + bh * N * D;
  float* __restrict__ Lh = p.lse + bh * N;

  // ---- Q block -> registers (B operand of S^T = K Q^T), loaded once --------
  Frag qf[QB][NKS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t qrow = qw + qb * 32 + l32;
    const bool ok = qrow < N;
    const T* src = Qh + (ok ? qrow : 0) * D + hh * KG;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      if constexpr (kHalf) {
        u32x4 raw = ok ? *(const u32x4*)(src + ks * KSTEP) : u32x4{0, 0, 0, 0};
        raw ^= p.q_sign;
        qf[qb][ks] = bits<Frag>(raw);
      } else {
        uint32_t raw = ok ? bits<uint32_t>(src[ks * KSTEP]) : 0u;
        qf[qb][ks] = bits<float>(raw ^ p.q_sign);
      }
    }
  }

  // ---- K/V staging: global -> registers -> LDS -----------------------------
  constexpr int K_CHUNKS = BC * CPR;
  constexpr int K_ITERS = (K_CHUNKS + NT - 1) / NT;
  // 16-bit V: a thread takes two consecutive keys of one 16-byte column chunk
  // and writes 8 dwords of (key, key+1) pairs into V^T.  fp32 V: one chunk,
  // 4 scalar writes.
  constexpr int V_ITEMS = kHalf ? (BC / 2) * CPR : BC * CPR;
  constexpr int V_ITERS = (V_ITEMS + NT - 1) / NT;
  constexpr int V_LOADS = kHalf ? 2 : 1;
  u32x4 kreg[K_ITERS];
  u32x4 vreg[V_ITERS][V_LOADS];

  // Rows past N read row N-1 (always in bounds) and are replaced by zeros, so
  // no address ever leaves the head and P = 0 never meets non-finite V.
  auto load_row = [&](const T* base, int64_t g, int cc) -> u32x4 {
    const u32x4 x = *(const u32x4*)(base + (g < N ? g : N - 1) * D + cc * EPC);
    return g < N ? x : u32x4{0, 0, 0, 0};
  };
  auto load_tile = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < K_ITERS; ++i) {
      const int c = tid + i * NT;
      if (K_ITERS * NT == K_CHUNKS || c < K_CHUNKS) {
        const int row = c / CPR, cc = c % CPR;
        kreg[i] = load_row(Kh, k0 + row, cc);
      }
    }
#pragma unroll
    for (int i = 0; i < V_ITERS; ++i) {
      const int it = tid + i * NT;
      if (V_ITERS * NT == V_ITEMS || it < V_ITEMS) {
        if constexpr (kHalf) {
          const int kp = it % (BC / 2), cc = it / (BC / 2);
          vreg[i][0] = load_row(Vh, k0 + 2 * kp, cc);
          vreg[i][1] = load_row(Vh, k0 + 2 * kp + 1, cc);
        } else {
          const int row = it % BC, cc = it / BC;
          vreg[i][0] = load_row(Vh, k0 + row, cc);
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    T* kl = &k_lds[buf][0];
    T* vl = &vt_lds[buf][0];
#pragma unroll
    for (int i = 0; i < K_ITERS; ++i) {
      const int c = tid + i * NT;
      if (K_ITERS * NT == K_CHUNKS || c < K_CHUNKS) {
        const int row = c / CPR, cc = c % CPR;
        *(u32x4*)(kl + row * KS + cc * EPC) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < V_ITERS; ++i) {
      const int it = tid + i * NT;
      if (V_ITERS * NT == V_ITEMS || it < V_ITEMS) {
        if constexpr (kHalf) {
          const int kp = it % (BC / 2), cc = it / (BC / 2);
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t a = vreg[i][0][w], b = vreg[i][1][w];
            const uint32_t even = (a & 0xffffu) | (b << 16);        // element 2w
            const uint32_t odd = (a >> 16) | (b & 0xffff0000u);     // element 2w+1
            *(uint32_t*)(vl + (cc * 8 + 2 * w) * VS + 2 * kp) = even;
            *(uint32_t*)(vl + (cc * 8 + 2 * w + 1) * VS + 2 * kp) = odd;
          }
        } else {
          const int row = it % BC, cc = it / BC;
#pragma unroll
          for (int e = 0; e < 4; ++e) vl[(cc * 4 + e) * VS + row] = bits<float>(vreg[i][0][e]);
        }
      }
    }
  };

  // ---- running state ---------------------------------------------------------
  f32x16 o[QB][ND];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = kNegInf;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < ND; ++db) o[qb][db] = f32x16{};
  }

  // Tiles the workgroup stages, and tiles this wave actually consumes (causal:
  // nothing past the wave's last query; rows past N: nothing at all).
  const int64_t kv_end = CAUSAL ? (q0 + BR < N ? q0 + BR : N) : N;
  const int n_tiles = (int)((kv_end + BC - 1) / BC);
  const int64_t wave_end = CAUSAL ? (qw + QB * 32 < N ? qw + QB * 32 : N) : N;
  const int wave_tiles = qw < N ? (int)((wave_end + BC - 1) / BC) : 0;
  const float c = p.c;
  const int krow = k_row_of_lane(l32);

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int64_t k0 = (int64_t)t * BC;
    if (t + 1 < n_tiles) load_tile(k0 + BC);

    if (t < wave_tiles) {
      const T* kl = &k_lds[buf][0];
      const T* vl = &vt_lds[buf][0];

      // S^T = K Q^T for this tile: s[kb][qb] is the 32 keys x 32 queries block.
      f32x16 s[NKB][QB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const T* src = kl + (kb * 32 + krow) * KS + ks * KSTEP + hh * KG;
          Frag a = *(const Frag*)src;
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kb][qb] = E::mma(a, qf[qb][ks], s[kb][qb]);
        }
      }

      // Keys past N, and (causal) keys after the query, are invisible.
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw);

      // Online softmax.
      float alpha[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int64_t qrow = qw + qb * 32 + l32;
        float mx = kNegInf;
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int64_t key = k0 + kb * 32 + key_of_reg(r, hh);
              const bool vis = key < N && (!CAUSAL || key <= qrow);
              if (!vis) s[kb][qb][r] = kNegInf;
              mx = fmaxf(mx, s[kb][qb][r]);
            }
        } else {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
        }
        mx = fmaxf(mx, other_half(mx));
        const float mxc = mx == kNegInf ? kNegInf : mx * c;
        const float m_new = fmaxf(m[qb], mxc);
        const float m_use = m_new == kNegInf ? 0.f : m_new;
        alpha[qb] = __builtin_amdgcn_exp2f(m[qb] - m_use);
        m[qb] = m_new;
        // p = 2^(c*s - m); invisible entries (s = -inf) give exactly 0.
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x = s[kb][qb][r];
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -m_use));
            s[kb][qb][r] = (need_mask && x == kNegInf) ? 0.f : e;
          }
      }

      // Rescale, row sums, and O^T += V^T P^T.
      if constexpr (kHalf) {
        using Pair = typename E::Pair;
        Frag pf[NKB][QB][NJ];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float rs = 0.f;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
              Frag f;
#pragma unroll
              for (int i = 0; i < KG; i += 2) {
                Pair pr = E::pack(s[kb][qb][j * KG + i], s[kb][qb][j * KG + i + 1]);
                rs = E::sum2(pr, rs);  // sum of the rounded weights P V uses
                f[i] = pr[0];
                f[i + 1] = pr[1];
              }
              pf[kb][qb][j] = f;
            }
          l[qb] = l[qb] * alpha[qb] + rs;
#pragma unroll
          for (int db = 0; db < ND; ++db) o[qb][db] *= alpha[qb];
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int db = 0; db < ND; ++db) {
              Frag a = *(const Frag*)(vl + (db * 32 + l32) * VS + kb * 32 + 16 * j + 8 * hh);
#pragma unroll
              for (int qb = 0; qb < QB; ++qb) o[qb][db] = E::mma(a, pf[kb][qb][j], o[qb][db]);
            }
      } else {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          float rs = 0.f;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) rs += s[kb][qb][r];
          l[qb] = l[qb] * alpha[qb] + rs;
#pragma unroll
          for (int db = 0; db < ND; ++db) o[qb][db] *= alpha[qb];
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int db = 0; db < ND; ++db) {
              const float a = vl[(db * 32 + l32) * VS + kb * 32 + key_of_reg(j, hh)];
#pragma unroll
              for (int qb = 0; qb < QB; ++qb) o[qb][db] = E::mma(a, s[kb][qb][j], o[qb][db]);
            }
      }
    }

    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O_acc / l written once; LSE = (m + log2 l) * ln 2 ------
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l[qb] + other_half(l[qb]);
    const int64_t qrow = qw + qb * 32 + l32;
    if (qrow < N) {
      const float inv = 1.0f / lt;
      if (hh == 0) Lh[qrow] = (m[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
      T* dst = Oh + qrow * D + hh * 4;
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& acc = o[qb][db];
          const float x0 = acc[4 * g] * inv, x1 = acc[4 * g + 1] * inv;
          const float x2 = acc[4 * g + 2] * inv, x3 = acc[4 * g + 3] * inv;
          T* out = dst + db * 32 + g * 8;
          if constexpr (kHalf) {
            typename E::Pair lo = E::pack(x0, x1), hi = E::pack(x2, x3);
            uint2 w;
            w.x = bits<uint32_t>(lo);
            w.y = bits<uint32_t>(hi);
            *(uint2*)out = w;
          } else {
            *(float4*)out = make_float4(x0, x1, x2, x3);
          }
        }
    }
  }
}

template <typename T, int D, bool CAUSAL, int NW, int QB, int BC>
hipError_t launch_one(const FwdArgs& a, hipStream_t stream) {
  constexpr int BR = NW * QB * 32;
  KernelParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.n_qblk = (int32_t)((a.N + BR - 1) / BR);
  p.c = __builtin_fabsf(a.scale) * kLog2e;
  const bool neg = a.scale < 0.f;
  p.q_sign = neg ? (sizeof(T) == 2 ? 0x80008000u : 0x80000000u) : 0u;
  const int64_t nblk = a.BH * p.n_qblk;
  hipLaunchKernelGGL((fwd_kernel<T, D, CAUSAL, NW, QB, BC>), dim3((unsigned)nblk),
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

// Tile configurations: 16-bit inputs use 4 waves x 64 queries (256 query rows
// per workgroup, 64-key tiles); fp32 uses 2 waves x 32 queries and 32-key
// tiles, which spreads the small fp32 problems over more workgroups.
template <typename T, int D, bool CAUSAL>
hipError_t dispatch_causal(const FwdArgs& a, hipStream_t s) {
  if constexpr (sizeof(T) == 2) return launch_one<T, D, CAUSAL, 4, 2, 64>(a, s);
  else return launch_one<T, D, CAUSAL, 2, 1, 32>(a, s);
}

template <typename T, int D>
hipError_t dispatch_d(const FwdArgs& a, hipStream_t s) {
  return a.causal ? dispatch_causal<T, D, true>(a, s) : dispatch_causal<T, D, false>(a, s);
}

template <typename T>
hipError_t dispatch_t(const FwdArgs& a, hipStream_t s) {
  return a.d == 64 ? dispatch_d<T, 64>(a, s) : dispatch_d<T, 128>(a, s);
}

}  // namespace

int rows_per_workgroup(Dtype dtype, int, bool) {
  return dtype == Dtype::F32 ? 2 * 1 * 32 : 4 * 2 * 32;
}

hipError_t launch_forward(const FwdArgs& a, hipStream_t stream) {
  switch (a.dtype) {
    case Dtype::F16: return dispatch_t<_Float16>(a, stream);
    case Dtype::BF16: return dispatch_t<__bf16>(a, stream);
    case Dtype::F32: return dispatch_t<float>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace fa
