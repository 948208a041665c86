// FlashAttention forward pass for fp16 and bf16 inputs on gfx950 (CDNA4).
//
// What is computed: exact attention O = softmax(scale * Q K^T) V and the
// natural-log log-sum-exp of each score row, for every (batch, head).
//
// The method (the FlashAttention explainer pages):
//   * Tiling ("FlashAttention, Playable", EP 03; chapter 15 "The Tiling
//     Strategy"): a workgroup owns a block of query rows and walks the keys
//     one tile at a time; K and V tiles are staged through on-chip memory.
//   * Fusion ("FlashAttention: Tiled & Fused"): scores, softmax and P V run in
//     one kernel; scores and probabilities never leave registers and O is
//     written once, at the end.
//   * Online softmax ("FlashAttention, Playable", EP 04): per query row a
//     running maximum m and running sum l; when a tile raises the maximum, what
//     was accumulated is multiplied by exp(m_old - m_new).
//
// CDNA4 mapping (our design, not the pages'):
//   * Workgroup = 8 waves x 32 query rows.  At <= 256 VGPRs per wave two waves
//     share a SIMD, so one wave's softmax (VALU) runs under the other wave's
//     matrix products (MFMA).
//   * K and V tiles (64 keys) are double buffered in LDS, row-major, with the
//     16-byte chunks of each row permuted (XOR swizzle) so that the reads below
//     hit all LDS banks; the next tile's global loads are in flight while the
//     current tile is consumed.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{f16,bf16}: a lane owns one query
//     (accumulator column) and 16 keys, the other 16 sit in lane l^32, so the
//     row max and sum are in-lane plus one v_permlane32_swap, and the rescale
//     factor is a per-lane scalar.  Q stays in registers for the whole loop.
//   * O^T += V^T P^T: P^T is the B operand taken straight from the score
//     registers (rounded to the input type), V^T comes from row-major V in
//     LDS through ds_read_b64_tr_b16 transposing loads.
//   * exp is exp2 with log2(e) folded into the scale.  The reference maximum
//     is only raised when a tile's maximum exceeds it by more than
//     kRescaleSlack (log2 units); until then the weights are exp2 of at most
//     kRescaleSlack, and in exact arithmetic the result is unchanged because
//     numerator and denominator share the reference.  This removes the
//     accumulator rescale from almost every tile.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

// Largest excess (log2 units) of a score over the reference maximum before
// the accumulator is rescaled: weights stay <= 2^8 = 256, far inside the
// fp16/bf16 range and exact-ratio in fp32.
constexpr float kRescaleSlack = 8.0f;

template <typename T>
struct Half;

template <>
struct Half<_Float16> {
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
  // acc + p.x + p.y in fp32 (v_dot2 with ones)
  static __device__ __forceinline__ float sum2(Pair p, float acc) {
    const Pair one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(p, one, acc, false);
  }
};

template <>
struct Half<__bf16> {
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

// Position of 16-byte chunk c of row r inside the LDS row (rows are 2*D bytes,
// LDS banks repeat every 256 bytes = 16 chunks).
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

typedef short s16x4 __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;

// ds_read_b64_tr_b16: within each group of 16 lanes, output lane i, element
// e receives element i%4 of the 4 elements addressed by lane 4*e + i/4.  When
// lane j of the group addresses row r0 + j/4, columns c0 + 4*(j%4) .. +3 of a
// row-major 16-bit matrix, output lane i receives column c0 + i of rows
// r0 .. r0+3, i.e. a transposed 4 x 16 block.
__device__ __forceinline__ u32x2 lds_read_tr(const char* base, int byte_off) {
  lds_s16x4* ptr = (lds_s16x4*)((lds_char*)const_cast<char*>(base) + byte_off);
  return bits<u32x2>(__builtin_amdgcn_ds_read_tr16_b64_v4i16(ptr));
}

template <typename T, int D, bool CAUSAL, int NW, int BC>
__global__ void __launch_bounds__(NW * 64, 1) fwd_f16_kernel(KernelParams p) {
  using H = Half<T>;
  using Frag = typename H::Frag;
  using Pair = typename H::Pair;
  using Sw = Swizzle<D>;
  constexpr int NT = NW * 64;        // threads per workgroup
  constexpr int BR = NW * 32;        // query rows per workgroup
  constexpr int RB = D * 2;          // bytes per row of K or V
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int TILE = BC * RB;      // bytes of one staged K (or V) tile
  constexpr int NKB = BC / 32;       // 32-key blocks per tile
  constexpr int NKS = D / 16;        // MFMAs per 32x32 score block
  constexpr int ND = D / 32;         // 32-row blocks of O^T
  constexpr int CHUNKS = BC * CPR;   // 16-byte chunks per staged tile
  constexpr int ITERS = CHUNKS / NT;
  static_assert(CHUNKS % NT == 0 && BC % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) char smem[2][2][TILE];  // [buffer][K, V]

  const WorkItem wi = work_item<CAUSAL>(p.n_qblk);
  const int64_t N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t q0 = (int64_t)wi.qblk * BR;
  const int64_t qw = q0 + (int64_t)wave * 32;
  const int64_t qrow = qw + l32;

  const T* __restrict__ Qh = (const T*)p.q + wi.bh * N * D;
  const T* __restrict__ Kh = (const T*)p.k + wi.bh * N * D;
  const T* __restrict__ Vh = (const T*)p.v + wi.bh * N * D;
  T* __restrict__ Oh = (T*)p.o + wi.bh * N * D;
  float* __restrict__ Lh = p.lse + wi.bh * N;

  // Q (B operand of S^T = K Q^T): lane holds Q[qrow][16*ks + 8*hh .. +7].
  Frag qf[NKS];
  {
    const bool ok = qrow < N;
    const T* src = Qh + (ok ? qrow : 0) * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 raw = ok ? *(const u32x4*)(src + ks * 16) : u32x4{0, 0, 0, 0};
      raw ^= p.q_sign;
      qf[ks] = bits<Frag>(raw);
    }
  }

  // ---- staging: global -> registers -> swizzled LDS -------------------------
  u32x4 kreg[ITERS], vreg[ITERS];
  // Rows past N read row N-1 (in bounds) and become zeros, so an invisible
  // key has finite V and a zero weight.
  auto load_row = [&](const T* base, int64_t g, int c) -> u32x4 {
    const u32x4 x = *(const u32x4*)(base + (g < N ? g : N - 1) * D + c * 8);
    return g < N ? x : u32x4{0, 0, 0, 0};
  };
  auto load_tile = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int ch = tid + i * NT;
      kreg[i] = load_row(Kh, k0 + ch / CPR, ch % CPR);
      vreg[i] = load_row(Vh, k0 + ch / CPR, ch % CPR);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int ch = tid + i * NT;
      const int r = ch / CPR, c = ch % CPR;
      *(u32x4*)(&smem[buf][0][r * RB + Sw::k(r, c) * 16]) = kreg[i];
      *(u32x4*)(&smem[buf][1][r * RB + Sw::v(r, c) * 16]) = vreg[i];
    }
  };

  // ---- lane-constant LDS offsets --------------------------------------------
  // K A operand for MFMA ks of key block kb: row kb*32 + krow, chunk 2*ks + hh
  // (the swizzle only sees the row modulo 16, so kb does not change it).
  const int krow = k_row_of_lane(l32);
  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = krow * RB + Sw::k(krow, 2 * ks + hh) * 16;
  // V^T A operand for O^T block db, keys kb*32 + 16*jj + 8*hh + 4*t + 0..3:
  // lane j of 16-lane group g addresses row (.. + j/4) at columns
  // db*32 + 16*(g%2) + 4*(j%4); the swizzle only sees the row modulo 4.
  int voff[ND];
  {
    const int g = lane >> 4, j16 = lane & 15;
    const int vrow = 8 * hh + (j16 >> 2);
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const int dcol = db * 32 + 16 * (g & 1) + 4 * (j16 & 3);
      voff[db] = vrow * RB + Sw::v(vrow, dcol >> 3) * 16 + (dcol & 7) * 2;
    }
  }

  // ---- running state ----------------------------------------------------------
  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) o[db] = f32x16{};
  float m = kNegInf;  // reference maximum of the row, log2 units
  float l = 0.f;      // this lane's share of the row sum (keys it holds)

  const int64_t kv_end = CAUSAL ? (q0 + BR < N ? q0 + BR : N) : N;
  const int n_tiles = (int)((kv_end + BC - 1) / BC);
  const int64_t wave_end = CAUSAL ? (qw + 32 < N ? qw + 32 : N) : N;
  const int wave_tiles = qw < N ? (int)((wave_end + BC - 1) / BC) : 0;
  const float c = p.c;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int64_t k0 = (int64_t)t * BC;
    if (t + 1 < n_tiles) load_tile(k0 + BC);

    if (t < wave_tiles) {
      const char* kl = &smem[buf][0][0];
      const char* vl = &smem[buf][1][0];

      // S^T = K Q^T: s[kb] is keys kb*32.. x this wave's 32 queries.
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const Frag a = bits<Frag>(*(const u32x4*)(kl + kb * 32 * RB + koff[ks]));
          s[kb] = H::mma(a, qf[ks], s[kb]);
        }

      // Invisible keys (past N, or after the query when causal) -> -inf.
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw);
      float mx = kNegInf;
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int64_t key = k0 + kb * 32 + key_of_reg(r, hh);
            if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = kNegInf;
            mx = fmaxf(mx, s[kb][r]);
          }
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      }
      mx = halves_max(mx);
      const float mxc = mx == kNegInf ? kNegInf : mx * c;

      // Online softmax: raise the reference maximum (and rescale l and O by
      // exp2(m_old - m_new)) only when this tile exceeds it by the slack.
      // m = -inf means no visible key yet: any visible key raises it.
      const bool grow = mxc > m + kRescaleSlack;
      if (__ballot(grow)) {
        const float alpha = grow ? __builtin_amdgcn_exp2f(m - mxc) : 1.0f;
        m = grow ? mxc : m;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < ND; ++db) o[db] *= alpha;
      }
      const float m_use = m == kNegInf ? 0.f : m;

      // P = exp2(c*s - m), rounded to T; l accumulates the rounded weights so
      // that O's normalisation matches the weights P V actually used.
      Frag pf[NKB][2];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          Frag f;
#pragma unroll
          for (int i = 0; i < 8; i += 2) {
            float e[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
              const float x = s[kb][8 * jj + i + u];
              e[u] = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -m_use));
              if (need_mask && x == kNegInf) e[u] = 0.f;
            }
            const Pair pr = H::pack(e[0], e[1]);
            rs = H::sum2(pr, rs);
            f[i] = pr[0];
            f[i + 1] = pr[1];
          }
          pf[kb][jj] = f;
        }
      l += rs;

      // O^T += V^T P^T.
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int db = 0; db < ND; ++db) {
            const int off = (kb * 32 + 16 * jj) * RB + voff[db];
            const u32x2 lo = lds_read_tr(vl, off);
            const u32x2 hi = lds_read_tr(vl, off + 4 * RB);
            const Frag a = bits<Frag>(u32x4{lo[0], lo[1], hi[0], hi[1]});
            o[db] = H::mma(a, pf[kb][jj], o[db]);
          }
    }

    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O_acc / l, written once; LSE = (m + log2 l) * ln 2 ----
  const float lt = halves_sum(l);
  if (qrow < N) {
    const float inv = 1.0f / lt;
    if (hh == 0) Lh[qrow] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
    T* dst = Oh + qrow * D + hh * 4;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const Pair lo = H::pack(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
        const Pair hi = H::pack(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
        *(u32x2*)(dst + db * 32 + g * 8) = u32x2{bits<uint32_t>(lo), bits<uint32_t>(hi)};
      }
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  constexpr int NW = 8, BC = 64, BR = NW * 32;
  static_assert(BR == kRowsPerWorkgroupF16, "rows per workgroup");
  KernelParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.n_qblk = (int32_t)((a.N + BR - 1) / BR);
  p.c = __builtin_fabsf(a.scale) * kLog2e;
  p.q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_f16_kernel<T, D, CAUSAL, NW, BC>), dim3((unsigned)(a.BH * p.n_qblk)),
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch<T, 64, true>(a, s) : launch<T, 64, false>(a, s);
  return a.causal ? launch<T, 128, true>(a, s) : launch<T, 128, false>(a, s);
}

}  // namespace

hipError_t launch_forward_f16(const FwdArgs& a, hipStream_t stream) {
  return a.dtype == Dtype::BF16 ? launch_t<__bf16>(a, stream) : launch_t<_Float16>(a, stream);
}

}  // namespace fa
