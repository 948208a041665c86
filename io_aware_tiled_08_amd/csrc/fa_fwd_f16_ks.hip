// FlashAttention forward pass for fp16 and bf16, key-split schedule for small
// causal problems with d = 64, on gfx950.
//
// Same computation, tiles and online softmax as fa_fwd_f16.hip (see there for
// the method and the CDNA4 mapping).  What differs is how the eight waves
// share the work: a workgroup owns 128 query rows instead of 256; waves w and
// w+4 hold the same 32 rows, and the two wave groups take alternate 128-key
// tiles (group A the even ones, group B the odd ones), each group keeping its
// own running maximum, sum and output.  The groups still alternate matrix and
// softmax phases half a tile apart.  At the end group B hands its (m, l, O)
// to group A through LDS, and A merges them with weights 2^(m_g - M), the
// rescale rule of the online softmax ("FlashAttention, Playable", EP 04)
// applied once across the two halves of the keys.
//
// Why: under a causal mask the 256-row blocks of a short sequence differ in
// length by up to the number of blocks (2..16 tiles at N = 2048), and with
// about one block per CU the longest block sets the time.  Blocks of 128 rows
// double the workgroup count and halve each one's length, so the dispatcher's
// longest-first order packs the CUs evenly.  The price is twice the K/V tile
// traffic per row (each tile serves 128 rows), and four LDS buffers per
// tensor (the groups read different tiles at once): 128 KiB at d = 64, which is
// why the schedule is used for d = 64 only.  Each workgroup runs two blocks of
// one head back to back, block n_qblk - 1 - i and then block i: their lengths
// add up to the same tile count for every pair, so one workgroup per pair
// balances by construction and a CU does not wait for a second dispatch.
#include "fa_device.h"
#include "fa_f16_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

// One 128-row block (work item wi), from its Q load to its O and LSE stores.
template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void ks_block(const KernelParams& p, const WorkItem wi) {
  using H = Half<T>;
  using Frag = typename H::Frag;
  using Pair = typename H::Pair;
  using Sw = Swizzle<D>;
  constexpr int NW = 8;              // waves per workgroup
  constexpr int BR = NW / 2 * 32;    // query rows per workgroup (two waves per row group)
  constexpr int BC = 128;            // keys per tile
  constexpr int RB = D * 2;          // bytes per row of K or V
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int TILE = BC * RB;      // bytes of one staged K (or V) tile
  constexpr int NKB = BC / 32;       // 32-key blocks per tile
  constexpr int NKS = D / 16;        // MFMAs per 32x32 score block
  constexpr int ND = D / 32;         // 32-row blocks of O^T
  constexpr int RPL = 1024 / RB;     // rows one wave-wide 1 KiB load covers
  constexpr int LPW = TILE / 1024 / 4;  // 1 KiB loads per loading wave per tensor
  static_assert(LPW >= 1 && TILE % 4096 == 0, "tile shape");
  static_assert(D == 64, "four buffers per tensor fit LDS at d = 64 only");

  __shared__ __attribute__((aligned(1024))) char smem[2][4][TILE];  // [K, V][buffer]

  const int64_t N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_b = wave >= 4;
  const int gw = wave & 3;  // wave index inside its group
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t q0 = (int64_t)wi.qblk * BR;
  const int gsel = group_b ? 1 : 0;  // this group takes the tiles t with t % 2 == gsel
  const int64_t qw = q0 + (int64_t)gw * 32;
  const int64_t qrow = qw + l32;

  const T* __restrict__ Qh = (const T*)p.q + wi.bh * N * D;
  const T* __restrict__ Kh = (const T*)p.k + wi.bh * N * D;
  const T* __restrict__ Vh = (const T*)p.v + wi.bh * N * D;
  T* __restrict__ Oh = (T*)p.o + wi.bh * N * D;
  float* __restrict__ Lh = p.lse + wi.bh * N;

  const int64_t kv_end = CAUSAL ? (q0 + BR < N ? q0 + BR : N) : N;
  const int n_tiles = (int)((kv_end + BC - 1) / BC);
  const int64_t wave_end = CAUSAL ? (qw + 32 < N ? qw + 32 : N) : N;
  const int wave_tiles = qw < N ? (int)((wave_end + BC - 1) / BC) : 0;

  // ---- tile loads: global -> LDS, 16 bytes per lane -------------------------
  // Group B (four waves) loads every tile.  Load j of group-wave gw
  // covers rows (gw*LPW + j)*RPL .. +RPL of the tile; lane i fills LDS chunk
  // slot i%CPR of row .. + i/CPR, which holds global chunk slot ^ mask(row).
  int kvoff[LPW], vvoff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = (gw * LPW + j) * RPL + lane / CPR;
    const int slot = lane % CPR;
    kvoff[j] = r * RB + Sw::k(r, slot) * 16;
    vvoff[j] = r * RB + Sw::v(r, slot) * 16;
  }
  const uint32_t lds_k = lds_addr(&smem[0][0][0]) + gw * LPW * 1024;
  const uint32_t lds_v = lds_addr(&smem[1][0][0]) + gw * LPW * 1024;
  auto issue_k = [&](int t) {
    if (t >= n_tiles) return;
    const int64_t k0 = (int64_t)t * BC;
    const uint32_t rows = (uint32_t)(N - k0 < BC ? N - k0 : BC);
    const u32x4 rs = buffer_rsrc(Kh + k0 * D, rows * RB);
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma_load16(rs, lds_k + (t & 3) * TILE + j * 1024, kvoff[j]);
  };
  auto issue_v = [&](int t) {
    if (t >= n_tiles) return;
    const int64_t k0 = (int64_t)t * BC;
    const uint32_t rows = (uint32_t)(N - k0 < BC ? N - k0 : BC);
    const u32x4 rs = buffer_rsrc(Vh + k0 * D, rows * RB);
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma_load16(rs, lds_v + (t & 3) * TILE + j * 1024, vvoff[j]);
  };
  auto barrier = [] {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto wait_loads = [] {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads have landed in LDS
    __builtin_amdgcn_sched_barrier(0);
  };

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
  if (group_b) {
    issue_k(0);
    issue_k(1);
  }

  // ---- lane-constant LDS read offsets ----------------------------------------
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
  f32x16 s[NKB];
  Frag pf[NKB][2];
  float m = kNegInf;  // reference maximum of the row, log2 units
  // This lane's share of the row sum (the keys it holds), accumulated on the
  // matrix pipe next to the P V products of the same weights; element 0 is
  // used (the product writes the same value to all four).
  f32x4 lacc = f32x4{};
  const float c = p.c;

  // M phase of tile t: O += P(t-1) V(t-1), then S(t) = K(t) Q^T: NPV + NS
  // matrix products whose A operands come from LDS.  In the steady state
  // (m_pv_s) the operand reads run kPipe products ahead of the products, so
  // LDS latency hides under the matrix pipe; the sched_group_barrier pairs
  // pin that order.  A wave's first tile has no P V product and its last
  // (t = wave_tiles) no score product (m_s, m_pv).
  constexpr int NPV = NKB * 2 * ND;  // O^T += V^T P^T products
  constexpr int NS = NKS * NKB;      // S^T = K Q^T products
  constexpr int kPipe = 4;
  auto fetch = [&](const char* vl, const char* kl, int i) -> Frag {
    if (i < NPV) {
      const int kb = i / (2 * ND), jj = (i / ND) % 2, db = i % ND;
      const int off = (kb * 32 + 16 * jj) * RB + voff[db];
      const u32x2 lo = lds_read_tr(vl, off);
      const u32x2 hi = lds_read_tr(vl, off + 4 * RB);
      return bits<Frag>(u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
    const int j = i - NPV, ks = j / NKB, kb = j % NKB;
    return bits<Frag>(*(const u32x4*)(kl + kb * 32 * RB + koff[ks]));
  };
  auto apply = [&](int i, Frag a) {
    if (i < NPV) {
      const int kb = i / (2 * ND), jj = (i / ND) % 2, db = i % ND;
      o[db] = H::mma(a, pf[kb][jj], o[db]);
      if (db == ND - 1) {
        const u32x4 w = bits<u32x4>(pf[kb][jj]);
        lacc = H::sum4(u32x2{w[0], w[1]}, lacc);
        lacc = H::sum4(u32x2{w[2], w[3]}, lacc);
      }
    } else {
      const int j = i - NPV, ks = j / NKB, kb = j % NKB;
      s[kb] = H::mma(a, qf[ks], s[kb]);
    }
  };
  auto m_pv_s = [&](int j) {
    const char* vl = &smem[1][(2 * j - 2 + gsel) & 3][0];
    const char* kl = &smem[0][(2 * j + gsel) & 3][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    Frag ring[kPipe];
    constexpr int PRE = 2 * kPipe;  // the first kPipe products are P V products
    static_assert(kPipe <= NPV, "pipeline prologue");
#pragma unroll
    for (int i = 0; i < kPipe; ++i) ring[i] = fetch(vl, kl, i);
    __builtin_amdgcn_sched_group_barrier(0x100, PRE, 0);
#pragma unroll
    for (int i = 0; i < NPV + NS; ++i) {
      const Frag a = ring[i % kPipe];
      if (i + kPipe < NPV + NS) ring[i % kPipe] = fetch(vl, kl, i + kPipe);
      apply(i, a);
      if (i + kPipe < NPV + NS) {
        if (i + kPipe < NPV) {
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
      if (i < NPV && i % ND == ND - 1) {
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);  // with the two row-sum products
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      }
    }
  };
  auto m_pv = [&](int j) {
    const char* vl = &smem[1][(2 * j - 2 + gsel) & 3][0];
#pragma unroll
    for (int i = 0; i < NPV; ++i) apply(i, fetch(vl, vl, i));
  };
  auto m_s = [&](int j) {
    const char* kl = &smem[0][(2 * j + gsel) & 3][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int i = NPV; i < NPV + NS; ++i) apply(i, fetch(kl, kl, i));
  };

  // V phase of tile t: online softmax of S(t) into P(t).
  auto v_phase = [&](int j) {
    const int64_t k0 = (int64_t)(2 * j + gsel) * BC;
    // Keys k0 + i with i >= lim are invisible (past N, or after the query
    // when causal): their scores become -inf.  Register r of key block kb
    // holds key kb*32 + key_of_reg(r, hh) of the tile.
    int64_t lim64 = N - k0;
    if (CAUSAL && qrow + 1 - k0 < lim64) lim64 = qrow + 1 - k0;
    const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw);
    if (need_mask) {
      const int lim = (int)(lim64 < 0 ? 0 : (lim64 > BC ? BC : lim64)) - 8 * hh;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kb * 32 + key_of_reg(r, 0) >= lim) s[kb][r] = kNegInf;
    }
    // Row maximum as a tree (short dependency chains), then across halves.
    float mx = chain_max4<NKB * 16>([&](int i) { return s[i / 16][i % 16]; });
    mx = halves_max(mx);
    const float mxc = mx * c;  // c > 0, so -inf stays -inf

    // Online softmax: raise the reference maximum (and rescale l and O by
    // exp2(m_old - m_new)) only when this tile exceeds it by the slack.
    // m = -inf means no visible key yet: any visible key raises it.
    const bool grow = mxc > m + kRescaleSlack;
    if (__ballot(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - mxc) : 1.0f;
      m = grow ? mxc : m;
      lacc *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] *= alpha;
    }
    // A lane whose row has seen no visible key yet keeps m = -inf; its
    // weights are exp2(-inf) = 0 either way.
    const float m_use = m == kNegInf ? 0.f : m;

    // P = exp2(c*s - m), rounded to T (the row sum is formed from these
    // rounded weights in the next matrix phase, so O's normalisation matches
    // the weights P V actually uses).  Masked scores are -inf and c > 0, so
    // their weight is exp2(-inf) = 0.
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        u32x4 f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * jj + 2 * i], c, -m_use));
          const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * jj + 2 * i + 1], c, -m_use));
          f[i] = bits<uint32_t>(H::pack(e0, e1));
        }
        pf[kb][jj] = bits<Frag>(f);
      }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) fence(pf[kb][jj]);
    fence(lacc);
    fence(m);
  };

  // K(0) must be resident before slot 0; the Q loads above land with it.
  wait_loads();
  barrier();

  // Slots as in fa_fwd_f16.hip with local steps j: in slot 2j group A runs
  // M(j) on tile 2j while group B runs V(j-1) on tile 2j-1; in slot 2j+1 A
  // runs V(j) and B runs M(j) on tile 2j+1.  At the start of its V phase in
  // step j (slot 2j+2) group B issues K(2j+4), K(2j+5), V(2j+2), V(2j+3): their
  // buffers (tile % 4) were last read in slots 2j and 2j+1, and they are
  // awaited at the end of B's next M phase (slot 2j+3), before their first
  // reader (slot 2j+4).
  auto iteration = [&](int j, auto mwork, auto vwork) {
    wave_priority<1>();
    mwork();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) fence(s[kb]);
#pragma unroll
    for (int db = 0; db < ND; ++db) fence(o[db]);
    fence(lacc);
    wave_priority<0>();
    if (group_b) wait_loads();
    barrier();
    if (group_b) {
      issue_k(2 * j + 4);
      issue_k(2 * j + 5);
      issue_v(2 * j + 2);
      issue_v(2 * j + 3);
    }
    vwork();
    barrier();
  };
  // This wave's tiles t < wave_tiles with t % 2 == gsel, and the workgroup's
  // step count (every wave takes part in every barrier).
  const int W = (wave_tiles - gsel + 1) / 2;
  const int J = (n_tiles + 1) / 2;
  if (group_b) {
    issue_k(2);
    issue_k(3);
    issue_v(0);
    issue_v(1);
    barrier();
  }
  iteration(
      0, [&] { if (W >= 1) m_s(0); }, [&] { if (W >= 1) v_phase(0); });
  for (int j = 1; j < W; ++j) iteration(j, [&] { m_pv_s(j); }, [&] { v_phase(j); });
  if (W >= 1) iteration(W, [&] { m_pv(W); }, [] {});
  for (int j = W >= 1 ? W + 1 : 1; j <= J; ++j) iteration(j, [] {}, [] {});
  if (!group_b) barrier();

  // ---- merge the two key halves: B -> LDS -> A ------------------------------
  // Every tile read is done (the last barrier closed the last M phase).
  constexpr int OS = D + 4;  // row stride (floats) of a partial O
  float* mo = (float*)&smem[0][0][0];
  float* mstat = mo + 4 * 32 * OS;  // [row group][row]: m, then l
  const float lt_g = halves_sum(lacc[0]);
  if (group_b) {
    float* ow = mo + (gw * 32 + l32) * OS + 4 * hh;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(ow + db * 32 + 8 * g) =
            make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
    if (hh == 0) {
      mstat[gw * 32 + l32] = m;
      mstat[128 + gw * 32 + l32] = lt_g;
    }
  }
  barrier();
  if (!group_b && qrow < N) {
    const float mb = mstat[gw * 32 + l32];
    const float lb = mstat[128 + gw * 32 + l32];
    const float M = fmaxf(m, mb);
    const float M_use = M == kNegInf ? 0.f : M;
    const float wa = __builtin_amdgcn_exp2f(m - M_use);
    const float wb = __builtin_amdgcn_exp2f(mb - M_use);
    const float lt = wa * lt_g + wb * lb;
    const float inv = 1.0f / lt;
    if (hh == 0) Lh[qrow] = (M + __builtin_amdgcn_logf(lt)) * kLn2;
    const float* ob = mo + (gw * 32 + l32) * OS + 4 * hh;
    T* dst = Oh + qrow * D + hh * 4;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float4 x = *(const float4*)(ob + db * 32 + 8 * g);
        const Pair lo = H::pack((wa * o[db][4 * g] + wb * x.x) * inv, (wa * o[db][4 * g + 1] + wb * x.y) * inv);
        const Pair hi = H::pack((wa * o[db][4 * g + 2] + wb * x.z) * inv, (wa * o[db][4 * g + 3] + wb * x.w) * inv);
        *(u32x2*)(dst + db * 32 + g * 8) = u32x2{bits<uint32_t>(lo), bits<uint32_t>(hi)};
      }
  }
}

// Two blocks of one head per workgroup, run back to back: block i and block
// n_qblk - 1 - i (equal total length under the causal mask).
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) fwd_f16_ks_pair_kernel(KernelParams p) {
  const int pairs = (p.n_qblk + 1) / 2;  // per head
  const int nblk = gridDim.x, wg = blockIdx.x;
  const int logical = (nblk % 8 == 0) ? (wg % 8) * (nblk / 8) + wg / 8 : wg;
  WorkItem w;
  w.bh = logical / pairs;
  const int i = logical % pairs;
  w.qblk = p.n_qblk - 1 - i;  // the longer block first
  ks_block<T, D, CAUSAL>(p, w);
  if (i != p.n_qblk - 1 - i) {
    // The first block's merge reads LDS that the second block's first tile
    // loads overwrite.
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    w.qblk = i;
    ks_block<T, D, CAUSAL>(p, w);
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  constexpr int BR = 128;
  static_assert(BR == kRowsPerWorkgroupF16KeySplit, "rows per workgroup");
  KernelParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.n_qblk = (int32_t)((a.N + BR - 1) / BR);
  // |scale| * log2(e); a zero scale becomes the smallest normal float so
  // that masked (-inf) scores still map to -inf and every visible score to
  // exp2(0) = 1.
  p.c = __builtin_fmaxf(__builtin_fabsf(a.scale) * kLog2e, 1.17549435e-38f);
  p.q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  hipLaunchKernelGGL((fwd_f16_ks_pair_kernel<T, D, CAUSAL>),
                     dim3((unsigned)(a.BH * ((p.n_qblk + 1) / 2))), dim3(512), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_f16_keysplit(const FwdArgs& a, hipStream_t stream) {
  if (a.d != 64 || !a.causal) return hipErrorInvalidValue;
  return a.dtype == Dtype::BF16 ? launch<__bf16, 64, true>(a, stream)
                                : launch<_Float16, 64, true>(a, stream);
}

}  // namespace fa
