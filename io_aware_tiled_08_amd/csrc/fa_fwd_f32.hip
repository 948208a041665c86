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
#include "fa_f16_common.h"
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

// ---------------------------------------------------------------------------
// Small fp32 problems at d = 64 (few 32-row blocks, e.g. one head of 512
// queries): a workgroup owns only 4 query rows, so the launch spreads over
// eight times as many CUs, and its 4 waves take every 4th chunk of 32 keys.
//
// v_mfma_f32_4x4x1_16b_f32 computes 16 independent 4x4 blocks; lane 4b + i
// supplies row i of block b's A column, lane 4b + j column j of its B row,
// and register r of lane 4b + j receives D[b][r][j].  Block b = 8h + bb:
// the two halves h of the wave work on the same 32 keys (bb = key block).
//   Scores:  lane (h, bb, i) supplies K[k0 + 4bb + i][32h + t] as A and
//            lane (h, bb, j) Q[q0 + j][32h + t] as B at step t < 32; register
//            r of lane (h, bb, j) then holds half h's share of the score of
//            key 4bb + r against query j, and one lane swap between the
//            halves adds the other share, so both halves hold the scores.
//   P V:     product (r, c), c < 8: B is register r of the weights (the
//            lane's own query j), A in lane (h, bb, i) is
//            V[k0 + 4bb + r][16 i + 8h + c].  Register i of lane (h, bb, j)
//            then sums V[.][16 i + 8h + c] P[j][.] over block bb's keys: a
//            partial O for query j, summed over the 8 blocks (and the waves)
//            at the end.
// The online softmax is the 32-row kernel's: running max (in log2 units)
// over the chunk, reduced across the lanes of a query, rescale by
// exp2(m_old - m_new); each lane keeps a partial sum of its own weights.
//
// Every workgroup streams its head's whole K and V through its CU, so the
// CU's load path (about 64 bytes a cycle) and the loads' latency set the
// time, not the products.  Chunks of 32 keys let each wave keep two of them
// in flight in LDS (16 KiB each), so that path has work from the start:
// each wave issues its first two chunks at once and chunk i+2 as soon as
// chunk i is in registers.  Q is staged once per workgroup (one 1 KiB load).
// At the end each wave's partial O (per lane and block) goes to LDS, and
// every thread sums one output over the 8 blocks and the 4 waves with
// weights 2^(m_w - M).
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kQ4Rows = 4;
constexpr int kQ4Keys = 32;
constexpr int kQ4Waves = 4;

// Maximum over the 16 lanes of one query (lanes congruent mod 4): row
// rotations by 4 and 8 within each 16-lane row, then the row pairs
// (permlane16 swap) and the halves (permlane32 swap).
template <typename Op>
__device__ __forceinline__ float query_reduce(float x, Op op) {
  x = op(x, bits<float>(__builtin_amdgcn_update_dpp(0, bits<int>(x), 0x124, 0xF, 0xF, false)));
  x = op(x, bits<float>(__builtin_amdgcn_update_dpp(0, bits<int>(x), 0x128, 0xF, 0xF, false)));
  const auto r16 = __builtin_amdgcn_permlane16_swap(bits<uint32_t>(x), bits<uint32_t>(x), false, false);
  x = op(bits<float>(r16[0]), bits<float>(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(bits<uint32_t>(x), bits<uint32_t>(x), false, false);
  return op(bits<float>(r32[0]), bits<float>(r32[1]));
}

// s_waitcnt immediate for vmcnt(n) alone (gfx9 layout: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima), n <= 63.
constexpr int vmcnt_imm(int n) { return (n & 0xF) | ((n >> 4) << 14) | 0x0F70; }

template <bool CAUSAL>
__global__ void __launch_bounds__(kQ4Waves * 64, 1) fwd_f32_q4_kernel(KernelParams p) {
  constexpr int D = 64;
  constexpr int RB = D * 4;              // bytes per K or V row
  constexpr int CH = kQ4Keys * RB;       // bytes of one chunk of K (or V)
  constexpr int PIECES = CH / 1024;      // 1 KiB loads per chunk of K (or V)
  // [wave][buffer][K, V]; after the loop the same LDS holds the waves'
  // partial O for the merge ([wave][lane][32 floats]).
  __shared__ __attribute__((aligned(1024))) char smem[kQ4Waves][2][2][CH];
  static_assert(sizeof(float) * kQ4Waves * 64 * 32 <= sizeof(smem), "merge area");
  float(*part)[64][32] = (float(*)[64][32])&smem[0][0][0][0];
  __shared__ __attribute__((aligned(16))) float q_lds[kQ4Rows][D];
  __shared__ float m_lds[kQ4Waves][kQ4Rows];
  __shared__ float l_lds[kQ4Waves][64];

  const int64_t N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 3;          // query of the lane (B column / output column) and A row
  const int bb = (lane >> 2) & 7;  // key block
  const int h = lane >> 5;         // half: d range 32h .. (scores), O columns 16 i + 8h .. (P V)
  const int64_t bh = blockIdx.x / p.n_qblk;
  int qblk = (int)(blockIdx.x % p.n_qblk);
  if (CAUSAL) qblk = p.n_qblk - 1 - qblk;  // longest blocks first
  const int64_t q0 = (int64_t)qblk * kQ4Rows;
  const int64_t qj = q0 + j;

  const float* __restrict__ Qh = (const float*)p.q + bh * N * D;
  const float* __restrict__ Kh = (const float*)p.k + bh * N * D;
  const float* __restrict__ Vh = (const float*)p.v + bh * N * D;

  const int64_t kv_end = CAUSAL ? (q0 + kQ4Rows < N ? q0 + kQ4Rows : N) : N;
  const int n_chunks = (int)((kv_end + kQ4Keys - 1) / kQ4Keys);
  // This wave's chunks: wave, wave + 4, ...
  const int n_mine = wave < n_chunks ? (n_chunks - wave + kQ4Waves - 1) / kQ4Waves : 0;
  const float c = p.c;

  // Chunk i of this wave goes to its buffer i % 2 by direct-to-LDS loads, read
  // coalesced (piece pc covers rows 4 pc .. 4 pc + 3; lane i fills LDS chunk
  // slot i % 16 of row 4 pc + i / 16).  Each row's 16-byte chunks are stored
  // permuted so the operand reads below spread evenly over the banks (four
  // lanes per 16-byte bank group, the least 64 lanes of 16 bytes allow):
  // chunk s of K row r at slot s ^ (r & 15), chunk s of V row r at slot
  // s ^ ((r >> 2) & 3).  The permutation is applied on the global side; rows
  // past N read as zeros (the buffer resources end there).
  const int prow = lane >> 4, slot = lane & 15;  // row within a piece, LDS slot
  auto issue = [&](int i) {
    const int64_t k0 = (int64_t)(wave + kQ4Waves * i) * kQ4Keys;
    const int64_t rows = N - k0 < kQ4Keys ? N - k0 : kQ4Keys;
    const u32x4 rk = buffer_rsrc(Kh + k0 * D, (uint32_t)(rows * RB));
    const u32x4 rv = buffer_rsrc(Vh + k0 * D, (uint32_t)(rows * RB));
    const uint32_t lk = lds_addr(&smem[wave][i & 1][0][0]);
    const uint32_t lv = lds_addr(&smem[wave][i & 1][1][0]);
#pragma unroll
    for (int pc = 0; pc < PIECES; ++pc) {
      const int r = 4 * pc + prow;
      dma_load16(rk, lk + pc * 1024, r * RB + (slot ^ (r & 15)) * 16);
      dma_load16(rv, lv + pc * 1024, r * RB + (slot ^ ((r >> 2) & 3)) * 16);
    }
  };
  // The lane's operands of chunk i: K row 4bb + j, d = 32h .. 32h + 31 (the
  // A row index of the score product is the lane's j), and V rows 4bb + r,
  // columns 16 i' + 8h .. +7 for i' = j (the A row index of the P V product).
  auto read_chunk = [&](int i, float* kf, float* vf) {
    const char* kl = &smem[wave][i & 1][0][0];
    const char* vl = &smem[wave][i & 1][1][0];
    const int kr = 4 * bb + j;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const float4 x = *(const float4*)(kl + kr * RB + ((8 * h + s) ^ (kr & 15)) * 16);
      kf[4 * s] = x.x;
      kf[4 * s + 1] = x.y;
      kf[4 * s + 2] = x.z;
      kf[4 * s + 3] = x.w;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int row = 4 * bb + r;
        const float4 x = *(const float4*)(vl + row * RB + ((4 * j + 2 * h + k) ^ ((row >> 2) & 3)) * 16);
        vf[8 * r + 4 * k] = x.x;
        vf[8 * r + 4 * k + 1] = x.y;
        vf[8 * r + 4 * k + 2] = x.z;
        vf[8 * r + 4 * k + 3] = x.w;
      }
  };

  // Q: one 1 KiB load by wave 0 into LDS (lane i: row i / 16, 16 bytes at
  // chunk i % 16), issued before the chunks; rows past N read as zeros.
  if (wave == 0) {
    const int64_t rows = N - q0 < kQ4Rows ? N - q0 : kQ4Rows;
    const u32x4 rq = buffer_rsrc(Qh + q0 * D, (uint32_t)(rows * RB));
    dma_load16(rq, lds_addr(&q_lds[0][0]), lane * 16);
  }
  if (n_mine > 0) issue(0);
  if (n_mine > 1) issue(1);
  // Q, issued first, has landed when at most the chunk loads issued after it
  // are outstanding (vmcnt counts a wave's loads in order).
  if (wave == 0) {
    if (n_mine > 1)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(4 * PIECES));
    else if (n_mine > 0)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PIECES));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  }
  __syncthreads();
  float qf[32];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const u32x4 x = *(const u32x4*)&q_lds[j][32 * h + 4 * s] ^ p.q_sign;
    qf[4 * s] = bits<float>(x[0]);
    qf[4 * s + 1] = bits<float>(x[1]);
    qf[4 * s + 2] = bits<float>(x[2]);
    qf[4 * s + 3] = bits<float>(x[3]);
  }

  f32x4 acc[8];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) acc[cc] = f32x4{};
  float m = kNegInf, lpart = 0.f;

  auto compute = [&](const float* kf, const float* vf, int i) {
    const int64_t k0 = (int64_t)(wave + kQ4Waves * i) * kQ4Keys;
    // Four independent accumulators (t mod 4), summed at the end; then the
    // other half's share.
    f32x4 sp[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
#pragma unroll
    for (int t = 0; t < 32; ++t)
      sp[t & 3] = __builtin_amdgcn_mfma_f32_4x4x1f32(kf[t], qf[t], sp[t & 3], 0, 0, 0);
    f32x4 s = (sp[0] + sp[1]) + (sp[2] + sp[3]);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const auto x = __builtin_amdgcn_permlane32_swap(bits<uint32_t>(s[r]), bits<uint32_t>(s[r]), false, false);
      s[r] = bits<float>(x[0]) + bits<float>(x[1]);
    }
    // Key 4bb + r of the chunk against query qj; past N or after the query
    // (causal) it is invisible.
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t key = k0 + 4 * bb + r;
      if (key >= N || (CAUSAL && key > qj)) s[r] = kNegInf;
      mx = fmaxf(mx, s[r]);
    }
    mx = query_reduce(mx, [](float x, float y) { return fmaxf(x, y); });
    const float mxc = mx == kNegInf ? kNegInf : mx * c;
    const float m_new = fmaxf(m, mxc);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m - m_use);
    m = m_new;
    float pw[4];
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pw[r] = s[r] == kNegInf ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -m_use));
      rs += pw[r];
    }
    lpart = lpart * alpha + rs;
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) acc[cc] *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int cc = 0; cc < 8; ++cc)
        acc[cc] = __builtin_amdgcn_mfma_f32_4x4x1f32(vf[8 * r + cc], pw[r], acc[cc], 0, 0, 0);
  };

  for (int i = 0; i < n_mine; ++i) {
    float kf[32], vf[32];
    // Chunk i has landed when at most chunk i + 1's loads are outstanding.
    if (i + 1 < n_mine)
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PIECES));
    else
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    read_chunk(i, kf, vf);
    if (i + 2 < n_mine) {
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the buffer's reads are done
      issue(i + 2);
    }
    compute(kf, vf, i);
  }
  __syncthreads();  // every wave is done with its LDS buffers

  // Merge: each lane's partial O (its query j, its half and block) and
  // partial sum go to LDS; thread t then forms output (q, d) = (t / 64,
  // t % 64) over the 8 blocks and the 4 waves.  Both halves hold the same
  // weights, so the sums come from half 0.
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) *(f32x4*)&part[wave][lane][4 * cc] = acc[cc];
  l_lds[wave][lane] = lpart;
  if (lane < kQ4Rows) m_lds[wave][lane] = m;
  __syncthreads();
  {
    const int q = tid >> 6, d = tid & 63;
    const int64_t qi = q0 + q;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kQ4Waves; ++w) M = fmaxf(M, m_lds[w][q]);
    const float M_use = M == kNegInf ? 0.f : M;
    // Column d = 16 i + 8 h + c of O is register i of accumulator c in the
    // lanes of half h.
    const int hd = (d >> 3) & 1, e = (d & 7) * 4 + (d >> 4);
    float L = 0.f, o = 0.f;
#pragma unroll
    for (int w = 0; w < kQ4Waves; ++w) {
      const float wt = __builtin_amdgcn_exp2f(m_lds[w][q] - M_use);
      float lw = 0.f, aw = 0.f;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        lw += l_lds[w][4 * kb + q];
        aw += part[w][32 * hd + 4 * kb + q][e];
      }
      L += wt * lw;
      o += wt * aw;
    }
    if (qi < N) {
      ((float*)p.o)[(bh * N + qi) * D + d] = o / L;
      if (d == 0) p.lse[bh * N + qi] = (M + __builtin_amdgcn_logf(L)) * kLn2;
    }
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

template <bool CAUSAL>
hipError_t launch_q4(const FwdArgs& a, hipStream_t stream) {
  KernelParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.n_qblk = (int32_t)((a.N + kQ4Rows - 1) / kQ4Rows);
  p.c = __builtin_fabsf(a.scale) * kLog2e;
  p.q_sign = a.scale < 0.f ? 0x80000000u : 0u;
  hipLaunchKernelGGL((fwd_f32_q4_kernel<CAUSAL>), dim3((unsigned)(a.BH * p.n_qblk)),
                     dim3(kQ4Waves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_f32(const FwdArgs& a, hipStream_t stream) {
  if (use_f32_q4(a.d, a.BH, a.N))
    return a.causal ? launch_q4<true>(a, stream) : launch_q4<false>(a, stream);
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
