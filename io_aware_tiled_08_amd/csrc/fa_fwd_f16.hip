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
//   * Workgroup = 8 waves x 32 query rows, in two groups of four (waves 0-3
//     and 4-7; wave w and wave w+4 share a SIMD).  The groups run half a tile
//     apart ("ping-pong"): while one group issues the matrix products of its
//     tile (M phase) the other runs its softmax on the vector ALU (V phase),
//     and a workgroup barrier swaps the roles.  For tile t a wave's M phase is
//     O += P(t-1) V(t-1) followed by S(t) = K(t) Q^T, and its V phase turns
//     S(t) into P(t).  The softmax's vector instructions issue while the
//     partner wave's matrix products run (a wave64 fp32 VALU op occupies the
//     vector pipe 4 cycles, exp 8; a 16x16x32 MFMA the matrix pipe 16).  The
//     wave in its M phase runs at issue priority 1, its partner at 0.
//   * K and V tiles (128 keys) are double buffered in LDS and filled by
//     buffer_load ... lds (HBM/L2 straight into LDS, no register staging).
//     The CU's load path takes one 1 KiB piece per about 16 cycles and a wave
//     issues in order, so a wave that issues a tile's pieces is held until
//     they are accepted; the two tensors' loads are therefore split between
//     the groups: group B issues K two tiles ahead at the start of its V
//     phase, group A issues V for the tile it is about to turn into P (that
//     buffer's last reader finished a slot earlier) and waits for it before
//     the barrier that ends its V phase.  At d = 128 A issues at the start of
//     its V phase; at d = 64, where the softmax phase is the longer of the
//     two, A issues at the end of its M phase, in the time it would otherwise
//     wait at the barrier.  Each row's 16-byte chunks are
//     stored XOR-permuted so that the operand reads hit all LDS banks; the
//     permutation is applied on the global side (lane i of a load always
//     writes LDS bytes 16i..16i+15).
//   * S^T = K Q^T on v_mfma_f32_16x16x32_{f16,bf16}: a wave's 32 queries are
//     two 16-query blocks, the 128-key tile eight 16-key blocks, and each K
//     fragment read from LDS feeds both query blocks.  A lane owns one query
//     of each block (its result column) and 4 keys of each key block; the
//     other 12 keys of a block sit in lanes l^16, l^32, l^48, so a row
//     maximum or sum is in-lane plus two lane swaps.  On this card the 16x16
//     products run about 20% cooler per FLOP than 32x32x16 (their accumulators
//     are a quarter the size), and under the power limit that buys clock: the
//     headline kernel ran 7-8% faster than the same pass on 32x32 tiles.
//     Q stays in registers for the whole loop.
//   * O^T += V^T P^T: P^T is the B operand taken straight from the score
//     registers (rounded to the input type): K rows are fed so that the 4
//     keys a lane holds in key block 2j and the 4 it holds in block 2j+1 are
//     8 consecutive keys of P V step j.  V^T comes from row-major V in LDS
//     through ds_read_b64_tr_b16 transposing loads.  The row sum of the
//     rounded weights is formed next to these products on the matrix pipe
//     (4x4x4 products against an all-ones operand), not on the vector ALU.
//   * exp is exp2 with log2(e) folded into the scale.  The reference maximum
//     is only raised when a tile's maximum exceeds it by more than
//     kRescaleSlack (log2 units); until then the weights are exp2 of at most
//     kRescaleSlack, and in exact arithmetic the result is unchanged because
//     numerator and denominator share the reference.  This removes the
//     accumulator rescale from almost every tile.
#include "fa_device.h"
#include "fa_f16_common.h"
#include "fa_launch.h"

namespace fa {
namespace {

// Row maxima of both 16-query blocks of a wave at once: a and b are a lane's
// partial maxima (its column of block 0 and of block 1); on return each holds
// the maximum over the four lane groups l, l^16, l^32, l^48.  One lane swap
// between the halves leaves block 0's pair maxima in lanes 0-31 and block
// 1's in lanes 32-63, one 16-lane swap finishes both, and a last swap hands
// each lane both results: three swaps and two maxima instead of four and four.
__device__ __forceinline__ void quad_max_pair(float& a, float& b) {
  const auto h = __builtin_amdgcn_permlane32_swap(bits<uint32_t>(a), bits<uint32_t>(b), false, false);
  const float m = fmaxf(bits<float>(h[0]), bits<float>(h[1]));
  const auto q = __builtin_amdgcn_permlane16_swap(bits<uint32_t>(m), bits<uint32_t>(m), false, false);
  const float m2 = fmaxf(bits<float>(q[0]), bits<float>(q[1]));
  const auto r = __builtin_amdgcn_permlane32_swap(bits<uint32_t>(m2), bits<uint32_t>(m2), false, false);
  a = bits<float>(r[0]);
  b = bits<float>(r[1]);
}

// The whole pass from the Q load to the O and LSE stores, for one 256-row
// query block (work item wi) of one (batch, head), or, with STREAM, for the
// R unmasked items j0, j0 + stride, ... (head-major) run back to back as one
// stream of key tiles.  Every wave of the workgroup calls it with the same
// arguments; on return all LDS reads are done (the last statement before the
// stores is a workgroup barrier), so a workgroup may call it again.
//
// The stream fills and drains the two-group pipeline once per workgroup
// rather than once per item: the next item's Q is loaded during the last
// softmax phase of the current one, and the finished item's O is stored
// during the first softmax phase of the next.  Each item's arithmetic is the
// single-item pass's (same products, same order), so O and LSE are bitwise
// equal.  In the stream every wave computes every tile (rows past N are zeros
// and never stored).
template <typename T, int D, bool CAUSAL, bool STREAM>
__device__ __forceinline__ void fwd_f16_tiles(const KernelParams& p, const WorkItem wi,
                                              const int64_t j0, const int64_t stride,
                                              const int R) {
  static_assert(!(CAUSAL && STREAM), "the tile stream is for unmasked items");
  using H = Half<T>;
  using Frag = typename H::Frag;
  using Pair = typename H::Pair;
  using Sw = Swizzle16<D>;
  constexpr int NW = 8;              // waves per workgroup
  constexpr int BR = NW * 32;        // query rows per workgroup
  constexpr int BC = 128;            // keys per tile
  constexpr int RB = D * 2;          // bytes per row of K or V
  constexpr int CPR = D / 8;         // 16-byte chunks per row
  constexpr int TILE = BC * RB;      // bytes of one staged K (or V) tile
  constexpr int NKB = BC / 16;       // 16-key blocks of S^T per tile
  constexpr int NKS = D / 32;        // 32-deep steps per score block
  constexpr int NJ = BC / 32;        // 32-key steps of O^T += V^T P^T
  constexpr int NDB = D / 16;        // 16-row blocks of O^T
  constexpr int RPL = 1024 / RB;     // rows one wave-wide 1 KiB load covers
  constexpr int LPW = TILE / 1024 / 4;  // 1 KiB loads per loading wave per tensor
  static_assert(LPW >= 1 && TILE % 4096 == 0, "tile shape");

  __shared__ __attribute__((aligned(1024))) char smem[2][2][TILE];  // [K, V][buffer]

  const int64_t N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_b = wave >= 4;
  const int gw = wave & 3;  // wave index inside its group
  const int l16 = lane & 15;  // query of the lane within a 16-query block
  const int lg = lane >> 4;   // 16-lane group: keys 4*lg .. of a 16-key block, or 8*lg .. of a 32-key step
  const int64_t q0 = (int64_t)wi.qblk * BR;
  const int64_t qw = q0 + (int64_t)wave * 32;

  const T* __restrict__ Qh = (const T*)p.q + wi.bh * N * D;
  const T* __restrict__ Kh = (const T*)p.k + wi.bh * N * D;
  const T* __restrict__ Vh = (const T*)p.v + wi.bh * N * D;
  T* __restrict__ Oh = (T*)p.o + wi.bh * N * D;
  float* __restrict__ Lh = p.lse + wi.bh * N;

  const int64_t kv_end = CAUSAL ? (q0 + BR < N ? q0 + BR : N) : N;
  const int n_tiles = (int)((kv_end + BC - 1) / BC);
  const int64_t wave_end = CAUSAL ? (qw + 32 < N ? qw + 32 : N) : N;
  const int wave_tiles = qw < N ? (int)((wave_end + BC - 1) / BC) : 0;

  // Stream positions.  Step g of the stream is tile g % n_tiles of item
  // g / n_tiles.  Positions are tracked by cursors that advance one step at a
  // time, so the loop divides nothing: the next item is the current one plus
  // stride, split once into whole heads and query blocks.
  const int total = R * n_tiles;  // steps of the stream
  // Wave-uniform values, pinned to scalar registers.
  auto uniform64 = [](int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
  };
  const int64_t s_bh = uniform64(stride / p.n_qblk);
  const int s_qb = __builtin_amdgcn_readfirstlane((int)(stride % p.n_qblk));
  auto next_item = [&](WorkItem w) {
    w.bh += s_bh;
    w.qblk += s_qb;
    if (w.qblk >= p.n_qblk) {
      w.qblk -= p.n_qblk;
      w.bh += 1;
    }
    return w;
  };
  struct Cursor {
    WorkItem w;  // item of the step
    int t;       // tile of the step within the item
    int g;       // step
  };
  WorkItem first;
  first.bh = uniform64(j0 / p.n_qblk);
  first.qblk = __builtin_amdgcn_readfirstlane((int)(j0 % p.n_qblk));
  auto advance = [&](Cursor& cu) {
    ++cu.g;
    if (++cu.t == n_tiles) {
      cu.t = 0;
      cu.w = next_item(cu.w);
    }
  };
  // Cursor of step cu.g + k (k >= 0), one item at a time.
  auto ahead = [&](Cursor cu, int k) {
    cu.g += k;
    cu.t += k;
    while (cu.t >= n_tiles) {
      cu.t -= n_tiles;
      cu.w = next_item(cu.w);
    }
    return cu;
  };

  // ---- tile loads: global -> LDS, 16 bytes per lane -------------------------
  // The four waves of a group share a tile's load (group B the K tiles,
  // group A the V tiles).  Load j of group-wave gw covers rows (gw*LPW + j)*RPL .. +RPL of the tile; lane i fills LDS chunk
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
  // In the stream, K and V tiles are issued in stream order: the tile of step
  // g goes to LDS buffer g % 2, and the V phase of step g issues K(g + 2) and
  // V(g + 1), derived from the cursor sc of that V phase.
  auto issue_step = [&](const void* base, uint32_t lds, const int* voffs, const Cursor cu) {
    if (cu.g >= total) return;
    const int64_t k0 = (int64_t)cu.t * BC;
    const uint32_t rows = (uint32_t)(N - k0 < BC ? N - k0 : BC);
    const u32x4 rs = buffer_rsrc((const T*)base + (cu.w.bh * N + k0) * D, rows * RB);
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma_load16(rs, lds + (cu.g & 1) * TILE + j * 1024, voffs[j]);
  };
  Cursor sc{first, 0, 0};
  auto issue_k = [&](int t) {
    if constexpr (STREAM) {
      issue_step(p.k, lds_k, kvoff, ahead(sc, t - sc.g));
    } else {
      if (t >= n_tiles) return;
      const int64_t k0 = (int64_t)t * BC;
      const uint32_t rows = (uint32_t)(N - k0 < BC ? N - k0 : BC);
      const u32x4 rs = buffer_rsrc(Kh + k0 * D, rows * RB);
#pragma unroll
      for (int j = 0; j < LPW; ++j) dma_load16(rs, lds_k + (t & 1) * TILE + j * 1024, kvoff[j]);
    }
  };
  auto issue_v = [&](int t) {
    if constexpr (STREAM) {
      issue_step(p.v, lds_v, vvoff, ahead(sc, t - sc.g));
    } else {
      if (t >= n_tiles) return;
      const int64_t k0 = (int64_t)t * BC;
      const uint32_t rows = (uint32_t)(N - k0 < BC ? N - k0 : BC);
      const u32x4 rs = buffer_rsrc(Vh + k0 * D, rows * RB);
#pragma unroll
      for (int j = 0; j < LPW; ++j) dma_load16(rs, lds_v + (t & 1) * TILE + j * 1024, vvoff[j]);
    }
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

  // Q (B operand of S^T = K Q^T, one per 16-query block qb): lane holds
  // Q[qw + 16*qb + l16][32*ks + 8*lg .. +7].
  // The stream loads each item's Q through a buffer resource that ends at row
  // N (rows past it read as zeros), so that nothing waits for the data before
  // the products that use it; only a negative scale (a sign flip of Q) reads
  // it at once.
  Frag qf[2][NKS];
  auto load_q = [&](const WorkItem w) {
    const int64_t q0 = (int64_t)w.qblk * BR;
    const int64_t rows = N - q0 < BR ? N - q0 : BR;
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const T*)p.q + (w.bh * N + q0) * D), (short)0, (int)(rows * RB), 0x00020000);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int off = (wave * 32 + 16 * qb + l16) * RB + lg * 16;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        qf[qb][ks] = bits<Frag>(__builtin_amdgcn_raw_buffer_load_b128(rs, off, 64 * ks, 0));
    }
    if (p.q_sign) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) qf[qb][ks] = bits<Frag>(bits<u32x4>(qf[qb][ks]) ^ p.q_sign);
    }
  };
  if constexpr (STREAM) {
    load_q(first);
  } else {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int64_t qr = qw + 16 * qb + l16;
      const bool ok = qr < N;
      const T* src = Qh + (ok ? qr : 0) * D + lg * 8;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 raw = ok ? *(const u32x4*)(src + ks * 32) : u32x4{0, 0, 0, 0};
        raw ^= p.q_sign;
        qf[qb][ks] = bits<Frag>(raw);
      }
    }
  }
  if (group_b) issue_k(0);

  // ---- lane-constant LDS read offsets ----------------------------------------
  // K A operand for step ks of key block kb: the lane feeds row m = l16 of
  // the block with key 32*(kb/2) + 8*(m/4) + 4*(kb%2) + m%4 of the tile, so
  // that register r of lane group lg in the product holds key
  // 32*(kb/2) + 8*lg + 4*(kb%2) + r: the 8 keys lane group lg contributes to
  // one 32-deep P V step are 8 consecutive keys, 4 from block 2j and 4 from
  // block 2j+1.  Chunk 4*ks + lg of the row; the swizzle ignores row bits 2, 5
  // and 6, so the block only adds a constant.
  const int krow = 8 * (l16 >> 2) + (l16 & 3);
  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = krow * RB + Sw::k(krow, 4 * ks + lg) * 16;
  // V^T A operand for O^T block db, keys 32*j + 8*lg + 0..7: lane j16 of
  // group lg addresses row 32*j + 8*lg + j16/4 (+4 for the second half) at
  // columns 16*db + 4*(j16%4); the swizzle ignores row bits 2, 5 and 6.
  int voff[NDB];
  {
    const int vrow = 8 * lg + (l16 >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int dcol = db * 16 + 4 * (l16 & 3);
      voff[db] = vrow * RB + Sw::v(vrow, dcol >> 3) * 16 + (dcol & 7) * 2;
    }
  }

  // ---- running state ----------------------------------------------------------
  f32x4 o[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) o[db][0] = o[db][1] = f32x4{};
  f32x4 s[NKB][2];
  Frag pf[NJ][2];
  float m[2] = {kNegInf, kNegInf};  // reference maximum of each of the lane's rows, log2 units
  // This lane's share of each row sum (the keys it holds), accumulated on the
  // matrix pipe next to the P V products of the same weights; element 0 is
  // used (the product writes the same value to all four).
  f32x4 lacc[2] = {f32x4{}, f32x4{}};
  const float c = p.c;

  // Epilogue of the stream's item w: O = O_acc / l, written once; LSE =
  // (m + log2 l) * ln 2.
  auto store = [&](const WorkItem w) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int64_t qrow = (int64_t)w.qblk * BR + (int64_t)wave * 32 + 16 * qb + l16;
      const float lt = quad_sum(lacc[qb][0]);
      if (qrow < N) {
        const float inv = 1.0f / lt;
        if (lg == 0) p.lse[w.bh * N + qrow] = (m[qb] + __builtin_amdgcn_logf(lt)) * kLn2;
        T* dst = (T*)p.o + (w.bh * N + qrow) * D + lg * 4;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const Pair lo = H::pack(o[db][qb][0] * inv, o[db][qb][1] * inv);
          const Pair hi = H::pack(o[db][qb][2] * inv, o[db][qb][3] * inv);
          *(u32x2*)(dst + db * 16) = u32x2{bits<uint32_t>(lo), bits<uint32_t>(hi)};
        }
      }
    }
  };

  // M phase of tile t: O += P(t-1) V(t-1), then S(t) = K(t) Q^T: NPV + NS
  // A fragments from LDS, each feeding the two 16-query blocks' products.  In
  // the steady state (m_pv_s) the fragment reads run kPipe fragments ahead of
  // the products, so
  // LDS latency hides under the matrix pipe; the sched_group_barrier pairs
  // pin that order.  A wave's first tile has no P V product and its last
  // (t = wave_tiles, or g = total in the stream) no score product (m_s,
  // m_pv).
  constexpr int NPV = NJ * NDB;   // V^T fragments (each feeds both 16-query blocks)
  constexpr int NS = NKS * NKB;   // K fragments (each feeds both 16-query blocks)
  constexpr int kPipe = 3;
  auto fetch = [&](const char* vl, const char* kl, int i) -> Frag {
    if (i < NPV) {
      const int j = i / NDB, db = i % NDB;
      const int off = 32 * j * RB + voff[db];
      const u32x2 lo = lds_read_tr(vl, off);
      const u32x2 hi = lds_read_tr(vl, off + 4 * RB);
      return bits<Frag>(u32x4{lo[0], lo[1], hi[0], hi[1]});
    }
    const int jj = i - NPV, ks = jj / NKB, kb = jj % NKB;
    return bits<Frag>(*(const u32x4*)(kl + (32 * (kb >> 1) + 4 * (kb & 1)) * RB + koff[ks]));
  };
  auto apply = [&](int i, Frag a) {
    if (i < NPV) {
      const int j = i / NDB, db = i % NDB;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) o[db][qb] = mma16<T>(a, pf[j][qb], o[db][qb]);
      if (db == NDB - 1) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const u32x4 w = bits<u32x4>(pf[j][qb]);
          lacc[qb] = H::sum4(u32x2{w[0], w[1]}, lacc[qb]);
          lacc[qb] = H::sum4(u32x2{w[2], w[3]}, lacc[qb]);
        }
      }
    } else {
      const int jj = i - NPV, ks = jj / NKB, kb = jj % NKB;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = mma16<T>(a, qf[qb][ks], s[kb][qb]);
    }
  };
  auto m_pv_s = [&](int t) {
    const char* vl = &smem[1][(t - 1) & 1][0];
    const char* kl = &smem[0][t & 1][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb][0] = s[kb][1] = f32x4{};
    Frag ring[kPipe];
    constexpr int PRE = 2 * kPipe;  // the first kPipe fragments are V^T fragments
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
      if (i < NPV && i % NDB == NDB - 1) {
        __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);  // with the four row-sum products
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      }
    }
  };
  auto m_pv = [&](int t) {
    const char* vl = &smem[1][(t - 1) & 1][0];
#pragma unroll
    for (int i = 0; i < NPV; ++i) apply(i, fetch(vl, vl, i));
  };
  auto m_s = [&](int t) {
    const char* kl = &smem[0][t & 1][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb][0] = s[kb][1] = f32x4{};
#pragma unroll
    for (int i = NPV; i < NPV + NS; ++i) apply(i, fetch(kl, kl, i));
  };

  // V phase of tile t: online softmax of S(t) into P(t).  In the stream the
  // tile comes from the cursor sc; the first step of an item first stores the
  // previous item (its last P V product ran in the M phase just before) and
  // starts the running state afresh, and the last step of an item loads the
  // next item's Q (the last product that reads Q ran in the M phase just
  // before).
  WorkItem done = first;  // the stream's item before sc's (valid once sc.g >= n_tiles)
  auto v_phase = [&](int t_arg) {
    int t = t_arg;
    if constexpr (STREAM) {
      t = sc.t;
      if (t == 0 && sc.g > 0) {
        store(done);
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db][0] = o[db][1] = f32x4{};
        lacc[0] = lacc[1] = f32x4{};
        m[0] = m[1] = kNegInf;
      }
    }
    const int64_t k0 = (int64_t)t * BC;
    // Keys k0 + i with i >= lim are invisible (past N, or after the query
    // when causal): their scores become -inf.  Register r of block kb, lane
    // group lg, holds key 32*(kb/2) + 8*lg + 4*(kb%2) + r of the tile.
    const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int64_t qr = qw + 16 * qb + l16;
        int64_t lim64 = N - k0;
        if (CAUSAL && qr + 1 - k0 < lim64) lim64 = qr + 1 - k0;
        const int lim = (int)(lim64 < 0 ? 0 : (lim64 > BC ? BC : lim64)) - 8 * lg;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (32 * (kb >> 1) + 4 * (kb & 1) + r >= lim) s[kb][qb][r] = kNegInf;
      }
    }
    // Online softmax per row (two rows per lane, one per query block): raise
    // the reference maximum only when this tile exceeds it by the slack.
    float mxc[2];
    bool grow[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) mxc[qb] = chain_max4<NKB * 4>([&](int i) { return s[i / 4][qb][i % 4]; });
    quad_max_pair(mxc[0], mxc[1]);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      mxc[qb] *= c;  // c > 0, so -inf stays -inf
      grow[qb] = mxc[qb] > m[qb] + kRescaleSlack;
    }
    if (__ballot(grow[0] || grow[1])) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float alpha = grow[qb] ? __builtin_amdgcn_exp2f(m[qb] - mxc[qb]) : 1.0f;
        m[qb] = grow[qb] ? mxc[qb] : m[qb];
        lacc[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db][qb] *= alpha;
      }
    }
    // P = exp2(c*s - m), rounded to T; P V step j takes keys 8*lg .. +7 of
    // its 32 from blocks 2j (registers 0..3) and 2j+1 (registers 0..3).
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float m_use = m[qb] == kNegInf ? 0.f : m[qb];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        u32x4 f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 2; ++e) {
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * j + h][qb][2 * e], c, -m_use));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * j + h][qb][2 * e + 1], c, -m_use));
            f[2 * h + e] = bits<uint32_t>(H::pack(e0, e1));
          }
        pf[j][qb] = bits<Frag>(f);
      }
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      fence(pf[j][0]);
      fence(pf[j][1]);
    }
    fence(lacc[0]);
    fence(lacc[1]);
    fence(m[0]);
    fence(m[1]);
    if constexpr (STREAM) {
      if (t == n_tiles - 1) {
        done = sc.w;
        if (sc.g + 1 < total) load_q(next_item(sc.w));
      }
      advance(sc);
    }
  };

  // K(0) must be resident before slot 0; the Q loads above land with it.
  wait_loads();
  barrier();

  // Global slots: in slot 2t group A runs M(t) and group B runs V(t-1); in
  // slot 2t+1 group A runs V(t) and group B runs M(t).  Both groups execute
  // the same sequence M(0) V(0) M(1) V(1) ... M(n_tiles) V(n_tiles), group B
  // one slot later (it idles through slot 0).  Loads, at the start of V
  // phases: group B issues K(t+2) at the start of slot 2t+2; it overwrites
  // K(t) (last read in slot 2t+1), is first read in slot 2t+4, and B waits
  // for it at the end of its next M phase (slot 2t+3).  Group A issues V(t)
  // at the start of slot 2t+1 (at d = 64: at the end of its M(t) in slot 2t,
  // kEarlyV); it overwrites V(t-2) (last read in slot 2t-1), is first read in
  // slot 2t+2, and A waits for it at the end of its V(t) phase, before the
  // barrier that closes slot 2t+1.  A wave works on
  // tiles t < wave_tiles only (causal waves above the diagonal stop early)
  // but takes part in every slot's barrier.  The stream runs the same slots,
  // counted in stream steps instead of tiles.
  constexpr bool kEarlyV = D == 64;
  auto iteration = [&](int t, auto mwork, auto vwork) {
    wave_priority<1>();
    mwork();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      fence(s[kb][0]);
      fence(s[kb][1]);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      fence(o[db][0]);
      fence(o[db][1]);
    }
    fence(lacc[0]);
    fence(lacc[1]);
    wave_priority<0>();
    if (kEarlyV && !group_b) issue_v(t);
    if (group_b) wait_loads();
    barrier();
    if (group_b)
      issue_k(t + 2);
    else if (!kEarlyV)
      issue_v(t);
    vwork();
    if (!group_b) wait_loads();
    barrier();
  };
  if (group_b) {
    issue_k(1);
    barrier();
  }
  if constexpr (STREAM) {
    iteration(0, [&] { m_s(0); }, [&] { v_phase(0); });
    for (int g = 1; g < total; ++g) iteration(g, [&] { m_pv_s(g); }, [&] { v_phase(g); });
    iteration(total, [&] { m_pv(total); }, [] {});
    if (!group_b) barrier();
    store(done);
    return;
  }
  const int W = wave_tiles;
  iteration(
      0, [&] { if (W >= 1) m_s(0); }, [&] { if (W >= 1) v_phase(0); });
  for (int t = 1; t < W; ++t) iteration(t, [&] { m_pv_s(t); }, [&] { v_phase(t); });
  if (W >= 1) iteration(W, [&] { m_pv(W); }, [] {});
  for (int t = W >= 1 ? W + 1 : 1; t <= n_tiles; ++t) iteration(t, [] {}, [] {});
  if (!group_b) barrier();

  // ---- epilogue: O = O_acc / l, written once; LSE = (m + log2 l) * ln 2 ----
  store(wi);
}


// One workgroup per 256-row block; the hardware dispatcher hands the blocks
// to CUs in the order of work_item (longest first when causal).
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) fwd_f16_kernel(KernelParams p) {
  fwd_f16_tiles<T, D, CAUSAL, false>(p, work_item<CAUSAL>(p.n_qblk), 0, 0, 1);
}

// Persistent schedule ("FlashAttention Evolution", FA-4 card: persistent
// kernels): a grid of G resident workgroups, each looping over the work items
// in rounds of G.  Causal items are ordered longest first (block-major across
// heads) and dealt in a snake: workgroup g takes item r*G + g in even rounds
// and r*G + G-1-g in odd ones, so over two rounds every workgroup gets about
// the same number of tiles.  When G and B*H are multiples of 8, the items of
// a workgroup all share one residue of (b*H + h) mod 8 per round parity, so
// an XCD (workgroup g runs on XCD g % 8) keeps to a few heads.  Unmasked items
// are equal in cost: workgroup g of XCD x takes a contiguous range of items
// per round, head-major, so a head's blocks share that XCD's L2, and runs its
// items as one tile stream (fwd_f16_tiles with STREAM).
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) fwd_f16_persistent_kernel(KernelParams p) {
  const int G = gridDim.x, g = blockIdx.x;
  const int gx = (!CAUSAL && G % 8 == 0) ? (g % 8) * (G / 8) + g / 8 : g;
  if constexpr (!CAUSAL) {
    // Items gx, gx + G, gx + 2G, ... as one tile stream.
    const int R = gx < p.n_items ? (int)((p.n_items - gx + G - 1) / G) : 0;
    if (R > 0) fwd_f16_tiles<T, D, false, true>(p, WorkItem{}, gx, G, R);
    return;
  }
  const int64_t n_bh = p.n_items / p.n_qblk;
  for (int64_t r = 0;; ++r) {
    const int64_t j = r * G + ((CAUSAL && (r & 1)) ? G - 1 - gx : gx);
    if (j >= p.n_items) break;
    WorkItem wi;
    if (CAUSAL) {
      wi.bh = j % n_bh;
      wi.qblk = p.n_qblk - 1 - (int)(j / n_bh);
    } else {
      wi.bh = j / p.n_qblk;
      wi.qblk = (int)(j % p.n_qblk);
    }
    fwd_f16_tiles<T, D, CAUSAL, false>(p, wi, 0, 0, 1);
  }
}

template <typename T, int D, bool CAUSAL>
KernelParams make_params(const FwdArgs& a) {
  constexpr int BR = 256;
  static_assert(BR == kRowsPerWorkgroupF16, "rows per workgroup");
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
  p.n_items = a.BH * p.n_qblk;
  return p;
}

// n_wg == 0: one workgroup per block; else the persistent kernel on n_wg
// workgroups (1 <= n_wg <= blocks).  An unmasked persistent launch whose tile
// stream would count more steps than an int holds takes the grid instead
// (same results, bit for bit).
template <typename T, int D, bool CAUSAL>
hipError_t launch(const FwdArgs& a, int n_wg, hipStream_t stream) {
  const KernelParams p = make_params<T, D, CAUSAL>(a);
  if (!CAUSAL && n_wg > 0 && (p.n_items + n_wg - 1) / n_wg * ((a.N + 127) / 128) > 0x7fffffff)
    n_wg = 0;
  if (n_wg == 0)
    hipLaunchKernelGGL((fwd_f16_kernel<T, D, CAUSAL>), dim3((unsigned)p.n_items), dim3(512), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((fwd_f16_persistent_kernel<T, D, CAUSAL>), dim3((unsigned)n_wg), dim3(512),
                       0, stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const FwdArgs& a, int n_wg, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch<T, 64, true>(a, n_wg, s) : launch<T, 64, false>(a, n_wg, s);
  return a.causal ? launch<T, 128, true>(a, n_wg, s) : launch<T, 128, false>(a, n_wg, s);
}

}  // namespace

hipError_t launch_forward_f16(const FwdArgs& a, hipStream_t stream) {
  return a.dtype == Dtype::BF16 ? launch_t<__bf16>(a, 0, stream) : launch_t<_Float16>(a, 0, stream);
}

hipError_t launch_forward_f16_persistent(const FwdArgs& a, int n_wg, hipStream_t stream) {
  return a.dtype == Dtype::BF16 ? launch_t<__bf16>(a, n_wg, stream)
                                : launch_t<_Float16>(a, n_wg, stream);
}

}  // namespace fa
