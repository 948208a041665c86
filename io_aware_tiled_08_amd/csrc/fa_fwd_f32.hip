// FlashAttention forward pass for fp32 inputs on gfx950.
//
// Same method as the fp16/bf16 kernel (tiles of K and V staged through LDS,
// online softmax with a running maximum and sum, O written once; see the
// FlashAttention explainer pages: chapter 15 "The Tiling Strategy",
// "FlashAttention, Playable" EP 03 and EP 04), with every step in fp32: both
// products use v_mfma_f32_32x32x2_f32 and the softmax weights stay fp32.
// Scores are produced transposed (S^T = K Q^T) so a lane owns one query row;
// V is written transposed into LDS so that the A operand of O^T += V^T P^T is
// one LDS word per lane.  The fp32 workloads are small, so the tile is small
// too (2 waves x 32 queries, 32-key tiles) to spread them over more CUs.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

template <int D, bool CAUSAL, int NW, int BC>
__global__ void __launch_bounds__(NW * 64, 1) fwd_f32_kernel(KernelParams p) {
  constexpr int NT = NW * 64;
  constexpr int BR = NW * 32;
  constexpr int CPR = D / 4;       // 16-byte chunks per row
  constexpr int KS = D + 4;        // LDS row stride of K (floats)
  constexpr int VS = BC + 4;       // LDS row stride of V^T (floats)
  constexpr int NKB = BC / 32;
  constexpr int ND = D / 32;
  static_assert(BC % 32 == 0 && D % 32 == 0, "tile shape");

  __shared__ __attribute__((aligned(16))) float k_lds[2][BC * KS];
  __shared__ __attribute__((aligned(16))) float vt_lds[2][D * VS];

  const WorkItem wi = work_item<CAUSAL>(p.n_qblk);
  const int64_t N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t q0 = (int64_t)wi.qblk * BR;
  const int64_t qw = q0 + (int64_t)wave * 32;

  const float* __restrict__ Qh = (const float*)p.q + wi.bh * N * D;
  const float* __restrict__ Kh = (const float*)p.k + wi.bh * N * D;
  const float* __restrict__ Vh = (const float*)p.v + wi.bh * N * D;
  float* __restrict__ Oh = (float*)p.o + wi.bh * N * D;
  float* __restrict__ Lh = p.lse + wi.bh * N;

  // Q (B operand of S^T = K Q^T): lane holds Q[query l32][2*ks + hh].
  float qf[D / 2];
  {
    const int64_t qrow = qw + l32;
    const bool ok = qrow < N;
    const float* src = Qh + (ok ? qrow : 0) * D + hh;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) {
      const uint32_t raw = ok ? bits<uint32_t>(src[2 * ks]) : 0u;
      qf[ks] = bits<float>(raw ^ p.q_sign);
    }
  }

  constexpr int CHUNKS = BC * CPR;
  constexpr int ITERS = (CHUNKS + NT - 1) / NT;
  u32x4 kreg[ITERS], vreg[ITERS];
  // Rows past N read row N-1 (in bounds) and are replaced by zeros.
  auto load_row = [&](const float* base, int64_t g, int cc) -> u32x4 {
    const u32x4 x = *(const u32x4*)(base + (g < N ? g : N - 1) * D + cc * 4);
    return g < N ? x : u32x4{0, 0, 0, 0};
  };
  auto load_tile = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int c = tid + i * NT;
      if (ITERS * NT == CHUNKS || c < CHUNKS) {
        kreg[i] = load_row(Kh, k0 + c / CPR, c % CPR);
        vreg[i] = load_row(Vh, k0 + c % BC, c / BC);
      }
    }
  };
  auto store_tile = [&](int buf) {
    float* kl = &k_lds[buf][0];
    float* vl = &vt_lds[buf][0];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int c = tid + i * NT;
      if (ITERS * NT == CHUNKS || c < CHUNKS) {
        *(u32x4*)(kl + (c / CPR) * KS + (c % CPR) * 4) = kreg[i];
        const int row = c % BC, cc = c / BC;
#pragma unroll
        for (int e = 0; e < 4; ++e) vl[(cc * 4 + e) * VS + row] = bits<float>(vreg[i][e]);
      }
    }
  };

  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) o[db] = f32x16{};
  float m = kNegInf, l = 0.f;

  const int64_t kv_end = CAUSAL ? (q0 + BR < N ? q0 + BR : N) : N;
  const int n_tiles = (int)((kv_end + BC - 1) / BC);
  const int64_t wave_end = CAUSAL ? (qw + 32 < N ? qw + 32 : N) : N;
  const int wave_tiles = qw < N ? (int)((wave_end + BC - 1) / BC) : 0;
  const float c = p.c;
  const int krow = k_row_of_lane(l32);
  const int64_t qrow = qw + l32;

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    const int64_t k0 = (int64_t)t * BC;
    if (t + 1 < n_tiles) load_tile(k0 + BC);

    if (t < wave_tiles) {
      const float* kl = &k_lds[buf][0];
      const float* vl = &vt_lds[buf][0];
      f32x16 s[NKB];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        s[kb] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < D / 2; ++ks)
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kl[(kb * 32 + krow) * KS + 2 * ks + hh],
                                                       qf[ks], s[kb], 0, 0, 0);
      }
      const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw);
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (need_mask) {
            const int64_t key = k0 + kb * 32 + key_of_reg(r, hh);
            if (key >= N || (CAUSAL && key > qrow)) s[kb][r] = kNegInf;
          }
          mx = fmaxf(mx, s[kb][r]);
        }
      mx = halves_max(mx);
      const float mxc = mx == kNegInf ? kNegInf : mx * c;
      const float m_new = fmaxf(m, mxc);
      const float m_use = m_new == kNegInf ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m - m_use);
      m = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float x = s[kb][r];
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -m_use));
          s[kb][r] = (need_mask && x == kNegInf) ? 0.f : e;
          rs += s[kb][r];
        }
      l = l * alpha + rs;
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] *= alpha;
      // O^T += V^T P^T: MFMA j takes P^T from accumulator register j.
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j)
#pragma unroll
          for (int db = 0; db < ND; ++db)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                vl[(db * 32 + l32) * VS + kb * 32 + key_of_reg(j, hh)], s[kb][j], o[db], 0, 0, 0);
    }

    if (t + 1 < n_tiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float lt = halves_sum(l);
  if (qrow < N) {
    const float inv = 1.0f / lt;
    if (hh == 0) Lh[qrow] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
    float* dst = Oh + qrow * D + hh * 4;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(dst + db * 32 + g * 8) =
            make_float4(o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv,
                        o[db][4 * g + 3] * inv);
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  constexpr int NW = 2, BC = 32, BR = NW * 32;
  static_assert(BR == kRowsPerWorkgroupF32, "rows per workgroup");
  KernelParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.n_qblk = (int32_t)((a.N + BR - 1) / BR);
  p.c = __builtin_fabsf(a.scale) * kLog2e;
  p.q_sign = a.scale < 0.f ? 0x80000000u : 0u;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, NW, BC>), dim3((unsigned)(a.BH * p.n_qblk)),
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
