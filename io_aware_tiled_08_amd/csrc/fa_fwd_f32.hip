// FlashAttention forward pass for fp32 inputs on gfx950.
//
// Same method as the fp16/bf16 kernel (K and V tiles, online softmax with a
// running maximum and sum, O written once; FlashAttention explainer pages:
// chapter 15 "The Tiling Strategy", "FlashAttention, Playable" EP 03 and
// EP 04), with every step in fp32: both products use v_mfma_f32_32x32x2_f32
// and the softmax weights stay fp32.
//
// The fp32 workloads are small (a single head of 512 queries is 16 blocks of
// 32 rows), so parallelism comes from the key axis: a workgroup owns 32
// query rows and its waves (8 at d=64; 4 at d=128, where a wave needs twice
// the registers) take every 8th (4th) 32-key tile each, each wave
// running its own online softmax (its own running max, sum and O).  The
// partial results are then merged through LDS, each scaled by 2^(m_w - M)
// where M is the largest of the waves' maxima -- the same rescaling rule the
// online softmax applies between tiles, applied once more between waves.
//
// Scores are produced transposed (S^T = K Q^T) so a lane owns one query row.
// Each wave reads its K and V tiles straight from global memory into
// registers (no tile is shared between waves); Q is staged once in LDS.
#include "fa_device.h"
#include "fa_launch.h"

namespace fa {
namespace {

constexpr int kRows = 32;   // query rows per workgroup
constexpr int kKeys = 32;   // keys per tile

template <int D>
struct F32Lds {
  static constexpr int kWaves = D == 64 ? 8 : 4;
  static constexpr int QS = D + 4;  // row stride (floats) of the staged Q block
  static constexpr int OS = D + 4;  // row stride of a wave's partial O
  static constexpr int kFloats = kWaves * kRows * OS + 2 * kWaves * kRows;
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(F32Lds<D>::kWaves * 64, 1) fwd_f32_kernel(KernelParams p) {
  constexpr int kWaves = F32Lds<D>::kWaves;
  constexpr int NT = kWaves * 64;
  constexpr int ND = D / 32;
  constexpr int QS = F32Lds<D>::QS;
  constexpr int OS = F32Lds<D>::OS;
  static_assert(kRows * QS <= kWaves * kRows * OS, "Q block fits the merge area");

  __shared__ __attribute__((aligned(16))) float lds[F32Lds<D>::kFloats];
  float* m_lds = lds + kWaves * kRows * OS;  // [wave][row] running max (log2 units)
  float* l_lds = m_lds + kWaves * kRows;     // [wave][row] running sum

  const WorkItem wi = work_item<CAUSAL>(p.n_qblk);
  const int64_t N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t q0 = (int64_t)wi.qblk * kRows;

  const float* __restrict__ Qh = (const float*)p.q + wi.bh * N * D;
  const float* __restrict__ Kh = (const float*)p.k + wi.bh * N * D;
  const float* __restrict__ Vh = (const float*)p.v + wi.bh * N * D;
  float* __restrict__ Oh = (float*)p.o + wi.bh * N * D;
  float* __restrict__ Lh = p.lse + wi.bh * N;

  // The d index of MFMA step ks for wave half hh is hh*D/2 + ks, so a lane's
  // K fragment is one contiguous half row.
  const float* q_lds = lds + l32 * QS + hh * (D / 2);
  const int krow = k_row_of_lane(l32);
  const int64_t qrow = q0 + l32;
  const float c = p.c;

  const int64_t kv_end = CAUSAL ? (q0 + kRows < N ? q0 + kRows : N) : N;
  const int n_tiles = (int)((kv_end + kKeys - 1) / kKeys);

  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) o[db] = f32x16{};
  float m = kNegInf, l = 0.f;

  // Tile loads go through raw buffer resources that end at row N: rows past
  // N read as zeros (their scores are masked; zero V rows add nothing).
  float kf[D / 2];
  float vf[ND][16];
  auto tile_rsrc = [&](const float* head, int64_t k0) {
    const int64_t rows = N - k0 < kKeys ? N - k0 : kKeys;
    return __builtin_amdgcn_make_buffer_rsrc((void*)(head + k0 * D), (short)0,
                                             (int)(rows * D * 4), 0x00020000);
  };
  auto load_k = [&](int t) {
    const auto rs = tile_rsrc(Kh, (int64_t)t * kKeys);
    const int off = (krow * D + hh * (D / 2)) * 4;
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rs, off + 16 * i, 0, 0);
      kf[4 * i] = bits<float>(x[0]);
      kf[4 * i + 1] = bits<float>(x[1]);
      kf[4 * i + 2] = bits<float>(x[2]);
      kf[4 * i + 3] = bits<float>(x[3]);
    }
  };
  auto load_v = [&](int t) {
    const auto rs = tile_rsrc(Vh, (int64_t)t * kKeys);
    const int off = (8 * hh * D + l32) * 4;
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int db = 0; db < ND; ++db)
        vf[db][j] = bits<float>(__builtin_amdgcn_raw_buffer_load_b32(
            rs, off + ((key_of_reg(j, 0) * D) + db * 32) * 4, 0, 0));
  };

  // The first tile's loads are in flight while the Q block is staged.
  if (wave < n_tiles) {
    load_k(wave);
    load_v(wave);
  }
  // Stage the Q block (sign-flipped when scale < 0; rows past N are zero).
  for (int ch = tid; ch < kRows * D / 4; ch += NT) {
    const int row = ch / (D / 4), c4 = ch % (D / 4);
    u32x4 x = {0, 0, 0, 0};
    if (q0 + row < N) x = *(const u32x4*)(Qh + (q0 + row) * D + c4 * 4);
    x ^= p.q_sign;
    *(u32x4*)(lds + row * QS + c4 * 4) = x;
  }
  __syncthreads();

  for (int t = wave; t < n_tiles; t += kWaves) {
    const int64_t k0 = (int64_t)t * kKeys;
    f32x16 s = f32x16{};
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const float4 qv = *(const float4*)(q_lds + 4 * i);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[4 * i], qv.x, s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[4 * i + 1], qv.y, s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[4 * i + 2], qv.z, s, 0, 0, 0);
      s = __builtin_amdgcn_mfma_f32_32x32x2f32(kf[4 * i + 3], qv.w, s, 0, 0, 0);
    }
    if (t + kWaves < n_tiles) load_k(t + kWaves);

    const bool need_mask = (k0 + kKeys > N) || (CAUSAL && k0 + kKeys - 1 > q0);
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (need_mask) {
        const int64_t key = k0 + key_of_reg(r, hh);
        if (key >= N || (CAUSAL && key > qrow)) s[r] = kNegInf;
      }
      mx = fmaxf(mx, s[r]);
    }
    mx = halves_max(mx);
    const float mxc = mx == kNegInf ? kNegInf : mx * c;
    const float m_new = fmaxf(m, mxc);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    m = m_new;
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float x = s[r];
      const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x, c, -m_use));
      s[r] = (need_mask && x == kNegInf) ? 0.f : e;
      rs += s[r];
    }
    l = l * alpha + rs;
#pragma unroll
    for (int db = 0; db < ND; ++db) o[db] *= alpha;
    // O^T += V^T P^T: MFMA j takes P^T from accumulator register j.
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
      for (int db = 0; db < ND; ++db)
        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vf[db][j], s[j], o[db], 0, 0, 0);
    if (t + kWaves < n_tiles) load_v(t + kWaves);
  }

  // Merge the waves' partial results.  The Q block's LDS is reused, so every
  // wave must be done with it first.
  const float lt = halves_sum(l);
  __syncthreads();
  {
    float* ow = lds + wave * kRows * OS + l32 * OS + 4 * hh;
    // Accumulator register r holds O^T row 8*(r/4) + 4*hh + r%4 of its
    // 32-column block: four consecutive d columns per group of four.
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(ow + db * 32 + 8 * g) =
            make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
    if (hh == 0) {
      m_lds[wave * kRows + l32] = m;
      l_lds[wave * kRows + l32] = lt;
    }
  }
  __syncthreads();

  for (int item = tid; item < kRows * D / 4; item += NT) {
    const int row = item / (D / 4), c4 = item % (D / 4);
    const int64_t qi = q0 + row;
    if (qi >= N) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, m_lds[w * kRows + row]);
    const float M_use = M == kNegInf ? 0.f : M;
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float wt = __builtin_amdgcn_exp2f(m_lds[w * kRows + row] - M_use);
      L += wt * l_lds[w * kRows + row];
      const float4 x = *(const float4*)(lds + w * kRows * OS + row * OS + 4 * c4);
      acc.x += wt * x.x;
      acc.y += wt * x.y;
      acc.z += wt * x.z;
      acc.w += wt * x.w;
    }
    const float inv = 1.0f / L;
    *(float4*)(Oh + qi * D + 4 * c4) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (c4 == 0) Lh[qi] = (M + __builtin_amdgcn_logf(L)) * kLn2;
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  static_assert(kRows == kRowsPerWorkgroupF32, "rows per workgroup");
  if (threads_per_workgroup(Dtype::F32, D) != F32Lds<D>::kWaves * 64) return hipErrorInvalidConfiguration;
  KernelParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.n_qblk = (int32_t)((a.N + kRows - 1) / kRows);
  p.c = __builtin_fabsf(a.scale) * kLog2e;
  p.q_sign = a.scale < 0.f ? 0x80000000u : 0u;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)(a.BH * p.n_qblk)),
                     dim3(F32Lds<D>::kWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
