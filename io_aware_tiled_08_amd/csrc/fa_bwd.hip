// FlashAttention backward pass for fp16 and bf16 on gfx950.
//
// What is computed: the gradients of the forward pass O = softmax(scale Q K^T) V
// (causal or not) for an upstream gradient dO, from Q, K, V, O, dO and the
// forward's LSE.  With P = exp(scale Q K^T - LSE) (the forward's softmax,
// recomputed tile by tile from the saved row statistics, never stored):
//   dV = P^T dO,  dP = dO V^T,  D = rowsum(dO * O),  dS = P * (dP - D),
//   dQ = scale dS K,  dK = scale dS^T Q.
// The pages only imply training ("FlashAttention: Tiled & Fused"); the
// gradient is the chain rule through the forward's definition ("FlashAttention"
// chapter 15, "Standard vs Flash Attention"), and the tiling follows the
// forward's idea: K/V (or Q/dO) tiles staged on chip, the N x N matrices never
// written to HBM.
//
// Three kernels, no atomics:
//   * bwd_prep: D = rowsum(dO * O) and LSE * log2(e) per row, fp32, into the
//     workspace.
//   * bwd_dkdv: a workgroup owns 128 keys in four groups of 32 and runs eight
//     waves; the two waves of a key group share a SIMD.  One ("P wave", K in
//     registers) computes S = Q K^T, P and dV^T += dO^T P; the other ("dS
//     wave", V in registers) computes dP = dO V^T, takes P from LDS (rounded
//     to the input type: the values of the dV product) and accumulates
//     dK^T += Q^T dS.  With K (or V) as the B operand a lane owns
//     one key and the 16 queries of a 32x32 block sit in its registers, so P
//     and dS feed the next products as B operands straight from registers.
//     32-query tiles of Q and dO (with their LSE and D) are staged through
//     LDS three tiles ahead.  Causal: a workgroup runs key blocks i and
//     n - 1 - i one after the other, so that the triangle's work is spread
//     evenly over the workgroups.
//   * bwd_dq: a workgroup owns 256 queries (8 waves x 32); it walks 64-key
//     tiles of K and V and accumulates dQ^T += K^T dS^T with S^T = K Q^T
//     (lane = query, as in the forward kernel).  Causal: query blocks
//     n - 1 - i and i share a workgroup, as the key blocks above do.
// Every tile is read both by rows (MFMA A operands) and transposed
// (ds_read_b64_tr_b16, for the d x rows operands); one XOR permutation of the
// 16-byte chunks of a row serves both without LDS bank conflicts.
#include <type_traits>

#include "fa_bwd.h"
#include "fa_device.h"
#include "fa_f16_common.h"

namespace fa {
namespace {

constexpr int kBwdRows = 128;  // keys per dK/dV workgroup (4 key groups x 32)
constexpr int kBwdWavesQ = 8;   // waves per dQ workgroup (32 queries each)
constexpr int kBwdTile = 64;   // keys per staged tile of the dQ kernel

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // workspace: D per row
  float* lse2;   // workspace: LSE * log2(e) per row
  int64_t N;
  int32_t n_blk;    // 128-key blocks per (b, h) (dK/dV kernel)
  int32_t n_blk_q;  // query blocks per (b, h) (dQ kernel)
  float c;        // scale * log2(e)
  float scale;
};

// Chunk c of row r sits at slot c ^ f(r).  Row reads (16 lanes: one chunk of
// 16 rows distinct mod 16) and transposing reads (32 lanes: 4 chunks of 4
// aligned rows) both hit 16 distinct 16-byte bank groups.
template <int D>
__device__ __forceinline__ constexpr int bswz(int r, int c) {
  return D == 128 ? c ^ (((r & 3) << 2) | ((r >> 2) & 3))
                  : c ^ ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

// ---- D = rowsum(dO * O) ------------------------------------------------------
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_prep_kernel(BwdParams p, int64_t rows) {
  constexpr int TPR = D / 8;         // threads per row, 8 elements each
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c8 = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const u32x4 a = *(const u32x4*)((const T*)p.dout + row * D + 8 * c8);
    const u32x4 b = *(const u32x4*)((const T*)p.o + row * D + 8 * c8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto x = bits<typename Half<T>::Pair>(a[i]);
      const auto y = bits<typename Half<T>::Pair>(b[i]);
      acc += (float)x[0] * (float)y[0] + (float)x[1] * (float)y[1];
    }
  }
#pragma unroll
  for (int w = TPR / 2; w > 0; w >>= 1) acc += __shfl_xor(acc, w, TPR);
  if (row < rows && c8 == 0) {
    p.delta[row] = acc;
    p.lse2[row] = p.lse[row] * kLog2e;
  }
}

// Row-read and transposing-read helpers over a staged [rows x D] tile.
template <typename T, int D>
struct TileOps {
  using Frag = typename Half<T>::Frag;
  static constexpr int RB = 2 * D;
  // A operand row fragment: row r, chunk c (8 elements).
  static __device__ __forceinline__ Frag row(const char* tile, int r, int c) {
    return bits<Frag>(*(const u32x4*)(tile + r * RB + bswz<D>(r, c) * 16));
  }
  // Transposed A operand: d rows db*32 + (lane column), 8 tile rows
  // r0 + 8*hh + 0..7 (r0 a multiple of 16) for lane half hh.
  static __device__ __forceinline__ Frag rows_t(const char* tile, int r0, int db, int lane) {
    const int g = lane >> 4, j = lane & 15, hh = lane >> 5;
    const int col = db * 32 + 16 * (g & 1) + 4 * (j & 3);
    const int c = col >> 3, off = (col & 7) * 2;
    const int ra = r0 + 8 * hh + (j >> 2), rb = ra + 4;
    const u32x2 lo = lds_read_tr(tile, ra * RB + bswz<D>(ra, c) * 16 + off);
    const u32x2 hi = lds_read_tr(tile, rb * RB + bswz<D>(rb, c) * 16 + off);
    return bits<Frag>(u32x4{lo[0], lo[1], hi[0], hi[1]});
  }
};

// Stage rows [r0, r0 + kBwdTile) of a [N, D] head into an LDS tile: the NWL
// waves each issue kBwdTile*2D/1024/NWL loads of 1 KiB; rows past N read zero.
template <int D, int NWL>
__device__ __forceinline__ void stage_tile(const void* head, int64_t r0, int64_t N, uint32_t lds,
                                           int wave, int lane) {
  constexpr int RB = 2 * D, CPR = D / 8, RPL = 1024 / RB;
  constexpr int LPW = kBwdTile * RB / 1024 / NWL;
  static_assert(LPW >= 1 && LPW * NWL * 1024 == kBwdTile * RB, "tile split");
  const uint32_t rows = (uint32_t)(N - r0 < kBwdTile ? N - r0 : kBwdTile);
  const u32x4 rs = buffer_rsrc((const char*)head + r0 * RB, rows * RB);
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = (wave * LPW + j) * RPL + lane / CPR;
    const int slot = lane % CPR;
    dma_load16(rs, lds + (wave * LPW + j) * 1024, r * RB + bswz<D>(r, slot) * 16);
  }
}

// Workgroup i runs on XCD i % 8: give each XCD a contiguous range of the
// logical blocks so that a head's blocks share one L2.
__device__ __forceinline__ int xcd_order() {
  const int n = gridDim.x, wg = blockIdx.x;
  return (n % 8 == 0) ? (wg % 8) * (n / 8) + wg / 8 : wg;
}

// Wait until at most n of this wave's loads are outstanding (vmcnt(n), gfx9
// encoding); no memory access moves across the wait.
template <int n>
__device__ __forceinline__ void wait_loads() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// ---- dK, dV ------------------------------------------------------------------
// A workgroup owns 128 keys in four groups of 32 and runs eight waves: wave g
// (g < 4, "P wave") and wave g + 4 ("dS wave") share key group g and a SIMD.
// For each 32-query tile the P wave computes S = Q K^T (K in registers),
// P = exp2(c S - LSE log2 e) and dV^T += dO^T P; the dS wave computes
// dP = dO V^T (V in registers), takes P from its partner through LDS, and
// accumulates dK^T += Q^T dS with dS = P (dP - D).  P crosses in the input
// type (the packed values of the dV product, half the bytes of fp32): dS is
// then formed from the rounded P, which adds u |dS| to its error bound.  One
// workgroup barrier per tile separates "P written" from "P read"; while one
// wave of a SIMD runs its vector work the other issues matrix products.
// Q/dO tiles and their LSE and D rows are loaded into LDS kDkvBufs - 1 tiles
// ahead.
constexpr int kDkvQ = 32;    // queries per staged tile
constexpr int kDkvBufs = 4;  // staged tiles: tile t + 3 loads while tile t is used

// The two values of a packed 16-bit pair, widened exactly to fp32 (a bf16
// value is the upper half of an fp32 pattern).
template <typename T>
__device__ __forceinline__ f32x2 unpack_pair(uint32_t w) {
  if constexpr (std::is_same_v<T, __bf16>)
    return f32x2{bits<float>(w << 16), bits<float>(w & 0xffff0000u)};
  else
    return __builtin_convertvector(bits<f16x2>(w), f32x2);
}

// vmcnt(n) and lgkmcnt(0): at most n of this wave's vector-memory loads still
// outstanding, and every LDS access of this wave complete.
template <int n>
__device__ __forceinline__ void wait_loads_lds() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0x0070 | (n & 15) | ((n >> 4) << 14));
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void dkdv_block(const BwdParams& p, const int64_t bh, const int kblk) {
  using H = Half<T>;
  using Frag = typename H::Frag;
  using Pair = typename H::Pair;
  constexpr int RB = 2 * D, CPR = D / 8, RPL = 1024 / RB;
  constexpr int QT = kDkvQ;
  constexpr int NB = kDkvBufs;
  constexpr int TILE = QT * RB;   // bytes of one staged Q (or dO) tile
  constexpr int CH = TILE / 1024;  // 1 KiB pieces per tensor and tile
  constexpr int LPW = 2 * CH / 8;  // pieces (Q's, then dO's) each wave loads
  static_assert(LPW >= 1 && LPW * 8 == 2 * CH, "tile split");
  constexpr int NKS = D / 16;
  constexpr int ND = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem[NB][2][TILE];  // [buffer][Q, dO]
  __shared__ __attribute__((aligned(16))) float stat[NB][2][QT];     // [buffer][LSE log2 e, D]
  // P of the current tile, per key group and slot (tile parity), packed in
  // the input type: 2 chunks of 64 lanes x 4 words (8 values), so each
  // 16-byte access of a wave covers 1 KiB.
  __shared__ __attribute__((aligned(1024))) uint32_t xch[4][2][2][64 * 4];

  const int64_t N = p.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool prole = wave < 4;
  const int kg = wave & 3;
  const int l32 = lane & 31, hh = lane >> 5;
  const int64_t k0 = (int64_t)kblk * kBwdRows;
  const int64_t kw = k0 + 32 * kg;  // the key group's first key
  const int64_t key = kw + l32;     // this lane's key (B-operand column)

  const T* Qh = (const T*)p.q + bh * N * D;
  const T* dOh = (const T*)p.dout + bh * N * D;
  const float* L2h = p.lse2 + bh * N;
  const float* Dh = p.delta + bh * N;

  // K (P wave) or V (dS wave) of this lane's key: B operand of S = Q K^T or
  // dP = dO V^T.
  Frag kv[NKS];
  {
    const bool ok = key < N;
    const T* src = (prole ? (const T*)p.k : (const T*)p.v) + bh * N * D + (ok ? key : 0) * D + 8 * hh;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      kv[ks] = bits<Frag>(ok ? *(const u32x4*)(src + 16 * ks) : u32x4{0, 0, 0, 0});
  }

  // Query tiles: causal blocks start at the first tile holding a query >= k0.
  const int qt_begin = CAUSAL ? (int)(k0 / QT) : 0;
  const int qt_end = (int)((N + QT - 1) / QT);
  const uint32_t lds_tiles = lds_addr(&smem[0][0][0]);
  const uint32_t lds_stat = lds_addr(&stat[0][0][0]);
  // Piece wave*LPW + j of a tile: lane i fills chunk slot i % CPR of row
  // (piece % CH)*RPL + i / CPR, which holds that row's chunk slot ^ swizzle.
  int goff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int r = ((wave * LPW + j) % CH) * RPL + lane / CPR;
    goff[j] = r * RB + bswz<D>(r, lane % CPR) * 16;
  }
  // Tiles past the end are still issued, over an empty range (every lane
  // reads zero), so that each wave issues the same number of loads per tile
  // and the wait counts below are constants.
  auto issue = [&](int qt, int buf) {
    const int64_t r0 = (int64_t)qt * QT;
    const bool real = qt < qt_end;
    const uint32_t rows = real ? (uint32_t)(N - r0 < QT ? N - r0 : QT) : 0u;
    const int64_t base = real ? r0 : 0;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int piece = wave * LPW + j;
      const T* head = piece < CH ? Qh : dOh;
      dma_load16(buffer_rsrc(head + base * D, rows * RB),
                 lds_tiles + (buf * 2 + piece / CH) * TILE + (piece % CH) * 1024, goff[j]);
    }
    if (wave == 0 && lane < QT / 4) {  // 32 floats each: 8 lanes x 16 bytes
      dma_load16(buffer_rsrc(L2h + base, rows * 4), lds_stat + (buf * 2 + 0) * QT * 4, lane * 16);
      dma_load16(buffer_rsrc(Dh + base, rows * 4), lds_stat + (buf * 2 + 1) * QT * 4, lane * 16);
    }
  };

  f32x16 acc[ND];  // dV^T (P wave) or dK^T / scale (dS wave)
#pragma unroll
  for (int db = 0; db < ND; ++db) acc[db] = f32x16{};
  const float c = p.c;
  const int krow = k_row_of_lane(l32);
  // Lane byte offsets inside a staged tile: row reads (A operands of S and
  // dP) and transposing reads (A operands of dV and dK).  The tile loop is
  // unrolled over the NB buffers, so each buffer's base folds into the
  // instructions' immediate offsets.
  int roff[NKS], toff[2 * ND][2];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) roff[ks] = krow * RB + bswz<D>(krow, 2 * ks + hh) * 16;
  {
    const int g = lane >> 4, j = lane & 15;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const int col = db * 32 + 16 * (g & 1) + 4 * (j & 3);
        const int cc = col >> 3, off = (col & 7) * 2;
        const int ra = 16 * jj + 8 * hh + (j >> 2), rb = ra + 4;
        toff[jj * ND + db][0] = ra * RB + bswz<D>(ra, cc) * 16 + off;
        toff[jj * ND + db][1] = rb * RB + bswz<D>(rb, cc) * 16 + off;
      }
  }
  auto row_frag = [&](const char* tile, int ks) -> Frag {
    return bits<Frag>(*(const u32x4*)(tile + roff[ks]));
  };
  auto tr_frag = [&](const char* tile, int i) -> Frag {
    const u32x2 lo = lds_read_tr(tile, toff[i][0]);
    const u32x2 hi = lds_read_tr(tile, toff[i][1]);
    return bits<Frag>(u32x4{lo[0], lo[1], hi[0], hi[1]});
  };
  uint32_t* xlane = &xch[kg][0][0][0] + lane * 4;  // this lane's P slots: + slot*512 + chunk*256

  // Tiles qt_begin .. qt_begin + NB - 2 before the loop (tile qt_begin + i
  // in buffer i % NB); tile t + NB - 1 after the barrier of tile t.  The
  // register loads above land with the first tile (the compiler does not
  // count the tile loads, so a wait it placed inside the loop would drain the
  // prefetch).
#pragma unroll
  for (int j = 0; j < NB - 1; ++j) issue(qt_begin + j, j);
  if (wave == 0)
    wait_loads_lds<(NB - 2) * (LPW + 2)>();
  else
    wait_loads_lds<(NB - 2) * LPW>();
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) fence(kv[ks]);
  block_barrier();

  // One tile.  Register r of a lane holds query qbase + key_of_reg(r, hh) of
  // its key; rows r = 8*half + e are the 8 consecutive queries
  // 16*half + 8*hh + e.
  auto step = [&](auto role, auto bufc, int qt) {
    constexpr bool PW = decltype(role)::value;
    constexpr int buf = decltype(bufc)::value;
    const char* qtile = &smem[buf][0][0];
    const char* dotile = &smem[buf][1][0];
    uint32_t* xs = xlane + (buf & 1) * 512;
    const int64_t qbase = (int64_t)qt * QT;
    // live: some query of the tile sees a key of the group (always, when
    // not causal; written as a run-time test there too, which keeps the
    // compiler from merging the tiles of the unrolled loop into one region
    // and spilling).  full: every (query, key) pair of the block is visible.
    const bool live = CAUSAL ? qbase + QT - 1 >= kw : qbase < N;
    const bool full = qbase + QT <= N && kw + 32 <= N && (!CAUSAL || qbase >= kw + 31);
    Frag pf[2];
    f32x16 dp;
    Frag at[2 * ND];  // A operands of the dV (dO^T) or dK (Q^T) products
    if (live) {
      // All A operands of S (or dP) are read before the products, and the
      // transposed operands of the dV (or dK) products, same tile, right
      // after them: LDS latency is paid once per group, not once per product.
      Frag a[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) a[ks] = row_frag(PW ? qtile : dotile, ks);
      __builtin_amdgcn_sched_group_barrier(0x100, NKS, 0);
      f32x16 sd = f32x16{};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) sd = H::mma(a[ks], kv[ks], sd);
      __builtin_amdgcn_sched_group_barrier(0x008, NKS, 0);
#pragma unroll
      for (int i = 0; i < 2 * ND; ++i) at[i] = tr_frag(PW ? dotile : qtile, i);
      __builtin_amdgcn_sched_group_barrier(0x100, 4 * ND, 0);
      if constexpr (PW) {
        const float* l2t = &stat[buf][0][0];
        float pr[16];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int qi = 16 * half + 8 * hh;
          const float4 a0 = *(const float4*)(l2t + qi), a1 = *(const float4*)(l2t + qi + 4);
          const float la[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pr[8 * half + e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sd[8 * half + e], c, -la[e]));
        }
        if (__builtin_expect(!full, 0)) {
          // Query qbase + kr (kr = key_of_reg(r, hh)) is visible iff
          // kr < N - qbase, and, when causal, kr >= key - qbase.  The bounds
          // are clamped to [0, QT] and shifted by 8*hh so that kr becomes the
          // constant key_of_reg(r, 0).
          const int64_t hi64 = key < N ? N - qbase : 0;
          const int hi = (int)(hi64 > QT ? QT : hi64) - 8 * hh;
          const int64_t lo64 = CAUSAL ? key - qbase : 0;
          const int lo = (int)(lo64 < 0 ? 0 : (lo64 > QT ? QT : lo64)) - 8 * hh;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kr = key_of_reg(r, 0);
            if (kr >= hi || kr < lo) pr[r] = 0.f;
          }
        }
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          u32x4 f;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            f[e] = bits<uint32_t>(H::pack(pr[8 * jj + 2 * e], pr[8 * jj + 2 * e + 1]));
          pf[jj] = bits<Frag>(f);
          *(u32x4*)(xs + jj * 256) = f;
        }
      } else {
        dp = sd;
      }
    }
    // Tile qt + 1 must have landed and this tile's P be written before the
    // barrier; NB - 3 later tiles may still be in flight.
    if (wave == 0)
      wait_loads_lds<(NB - 3) * (LPW + 2)>();
    else
      wait_loads_lds<(NB - 3) * LPW>();
    block_barrier();
    // Into the buffer of tile qt - 1, whose last reads preceded the barrier.
    issue(qt + NB - 1, (buf + NB - 1) % NB);
    if (live) {
      if constexpr (PW) {
        // dV^T += dO^T P.
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int db = 0; db < ND; ++db) acc[db] = H::mma(at[jj * ND + db], pf[jj], acc[db]);
      } else {
        // dS = P (dP - D); masked and out-of-range entries have P = 0.
        const float* dt = &stat[buf][1][0];
        float pr[16], dl[16];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          const u32x4 x = *(const u32x4*)(xs + jj * 256);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f32x2 w = unpack_pair<T>(x[e]);
            pr[8 * jj + 2 * e] = w[0];
            pr[8 * jj + 2 * e + 1] = w[1];
          }
        }
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          const int qi = 16 * half + 8 * hh;
          const float4 b0 = *(const float4*)(dt + qi), b1 = *(const float4*)(dt + qi + 4);
          const float lb[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) dl[8 * half + e] = lb[e];
        }
        Frag sf[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
          u32x4 f;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 8 * jj + 2 * e;
            f[e] = bits<uint32_t>(H::pack(pr[r] * (dp[r] - dl[r]), pr[r + 1] * (dp[r + 1] - dl[r + 1])));
          }
          sf[jj] = bits<Frag>(f);
        }
        // dK^T += Q^T dS.
#pragma unroll
        for (int jj = 0; jj < 2; ++jj)
#pragma unroll
          for (int db = 0; db < ND; ++db) acc[db] = H::mma(at[jj * ND + db], sf[jj], acc[db]);
      }
    }
  };
  // The two roles run separate copies of the loop (same barriers), so that
  // neither carries the other's registers; each copy is unrolled over the NB
  // buffers (tile qt_begin + i uses buffer i % NB and P slot i % 2).
  auto tiles = [&](auto role) {
    for (int qt0 = qt_begin; qt0 < qt_end; qt0 += NB) {
      step(role, std::integral_constant<int, 0>{}, qt0);
      if (qt0 + 1 >= qt_end) break;
      step(role, std::integral_constant<int, 1>{}, qt0 + 1);
      if (qt0 + 2 >= qt_end) break;
      step(role, std::integral_constant<int, 2>{}, qt0 + 2);
      if (qt0 + 3 >= qt_end) break;
      step(role, std::integral_constant<int, 3>{}, qt0 + 3);
    }
  };
  static_assert(NB == 4, "the tile loop above is written out for four buffers");
  if (prole)
    tiles(std::true_type{});
  else
    tiles(std::false_type{});
  // Drain the empty loads issued for tiles past the end.
  wait_loads_lds<0>();

  // dV (P wave) or dK = scale * acc (dS wave): lane `key`, register r of
  // block db is d row db*32 + 8*(r/4) + 4*hh + r%4.
  if (key < N) {
    T* dst = (T*)(prole ? p.dv : p.dk) + (bh * N + key) * D + 4 * hh;
    const float f = prole ? 1.0f : p.scale;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const Pair a = H::pack(acc[db][4 * g] * f, acc[db][4 * g + 1] * f);
        const Pair b = H::pack(acc[db][4 * g + 2] * f, acc[db][4 * g + 3] * f);
        *(u32x2*)(dst + db * 32 + 8 * g) = u32x2{bits<uint32_t>(a), bits<uint32_t>(b)};
      }
  }
}

// XCD-aware order (the blocks of one head share an XCD's L2). Causal: two key
// blocks of one head per workgroup, back to back, block i and then block
// n - 1 - i, so that every workgroup has about the same number of query tiles.
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) bwd_dkdv_kernel(BwdParams p) {
  const int logical = xcd_order();
  if constexpr (!CAUSAL) {
    dkdv_block<T, D, CAUSAL>(p, logical / p.n_blk, logical % p.n_blk);
  } else {
    const int pairs = (p.n_blk + 1) / 2;
    const int64_t bh = logical / pairs;
    const int i = logical % pairs;
    dkdv_block<T, D, CAUSAL>(p, bh, i);
    if (i != p.n_blk - 1 - i) {
      block_barrier();  // every wave's reads of the first block's tiles are done
      dkdv_block<T, D, CAUSAL>(p, bh, p.n_blk - 1 - i);
    }
  }
}

// ---- dQ ----------------------------------------------------------------------
template <typename T, int D, bool CAUSAL>
__device__ __forceinline__ void dq_block(const BwdParams& p, const int64_t bh, const int qblk) {
  constexpr int NWQ = kBwdWavesQ;
  constexpr int BRQ = 32 * NWQ;  // queries per workgroup
  using H = Half<T>;
  using Frag = typename H::Frag;
  using Pair = typename H::Pair;
  constexpr int RB = 2 * D;
  constexpr int TILE = kBwdTile * RB;
  constexpr int NKS = D / 32;   // 32-deep steps of a score product
  constexpr int NDB = D / 16;   // 16-column blocks of dQ^T
  constexpr int NBQ = 4;  // K/V tiles in LDS: tile t + 3 loads while tile t is used
  __shared__ __attribute__((aligned(1024))) char smem[NBQ][2][TILE];  // [buffer][K, V]

  const int64_t N = p.N;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;  // query of the lane within a 16-query block
  const int lg = lane >> 4;   // 16-lane group: keys 4*lg .. of a 16-key block, or 8*lg .. of a 32-key step
  const int64_t q0 = (int64_t)qblk * BRQ;
  const int64_t qw = q0 + 32 * wave;

  const T* Qh = (const T*)p.q + bh * N * D;
  const T* Kh = (const T*)p.k + bh * N * D;
  const T* Vh = (const T*)p.v + bh * N * D;
  const T* dOh = (const T*)p.dout + bh * N * D;

  // Q and dO of the lane's two queries qw + 16*qb + l16 (B operands of
  // S^T = K Q^T and dP^T = V dO^T): d = 32*ks + 8*lg .. +7.
  Frag qf[2][NKS], df[2][NKS];
  float lse2[2] = {0.f, 0.f}, drow[2] = {0.f, 0.f};
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t qr = qw + 16 * qb + l16;
    const bool ok = qr < N;
    const T* qs_ = Qh + (ok ? qr : 0) * D + 8 * lg;
    const T* ds_ = dOh + (ok ? qr : 0) * D + 8 * lg;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      qf[qb][ks] = bits<Frag>(ok ? *(const u32x4*)(qs_ + 32 * ks) : u32x4{0, 0, 0, 0});
      df[qb][ks] = bits<Frag>(ok ? *(const u32x4*)(ds_ + 32 * ks) : u32x4{0, 0, 0, 0});
    }
    if (ok) {
      lse2[qb] = p.lse[bh * N + qr] * kLog2e;
      drow[qb] = p.delta[bh * N + qr];
    }
  }

  const int64_t kv_end = CAUSAL ? (q0 + BRQ < N ? q0 + BRQ : N) : N;
  const int n_tiles = (int)((kv_end + kBwdTile - 1) / kBwdTile);
  const int64_t wave_end = CAUSAL ? (qw + 32 < N ? qw + 32 : N) : N;
  const int wave_tiles = qw < N ? (int)((wave_end + kBwdTile - 1) / kBwdTile) : 0;
  const uint32_t lds_base = lds_addr(&smem[0][0][0]);
  // Tiles past the end are issued over an empty range (every lane reads
  // zero), so that each wave has the same loads in flight at every wait.
  auto issue = [&](int t) {
    const int buf = t % NBQ;
    const bool real = t < n_tiles;
    const int64_t r0 = real ? (int64_t)t * kBwdTile : 0;
    const int64_t rows = real ? N - r0 : 0;
    stage_tile<D, NWQ>(Kh + r0 * D, 0, rows, lds_base + (buf * 2 + 0) * TILE, wave, lane);
    stage_tile<D, NWQ>(Vh + r0 * D, 0, rows, lds_base + (buf * 2 + 1) * TILE, wave, lane);
  };

  f32x4 dq[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db) dq[db][0] = dq[db][1] = f32x4{};
  const float c = p.c;
  // Row operand of 16-key block b (b = 0, 1 within a 32-key step): the lane
  // feeds row m = l16 of the block with tile row 8*(m/4) + 4*b + m%4 (plus the
  // step's 32), so that register r of lane group lg in the product holds key
  // 8*lg + 4*b + r of the step: the 8 keys lane group lg contributes to the
  // dQ product are 8 consecutive keys, 4 from each block.
  const int krow = 8 * (l16 >> 2) + (l16 & 3);
  auto row_frag = [&](const char* tile, int r, int ch) -> Frag {
    return bits<Frag>(*(const u32x4*)(tile + r * RB + bswz<D>(r, ch) * 16));
  };
  // K^T operand of dQ^T block db for keys 8*lg .. +7 of the step at row0:
  // lane j16 of group lg addresses row row0 + 8*lg + j16/4 (+4 for the second
  // half) at columns 16*db + 4*(j16%4).
  auto kt_frag = [&](const char* tile, int row0, int db) -> Frag {
    const int col = 16 * db + 4 * (l16 & 3);
    const int ch = col >> 3, off = (col & 7) * 2;
    const int ra = row0 + 8 * lg + (l16 >> 2), rb = ra + 4;
    const u32x2 lo = lds_read_tr(tile, ra * RB + bswz<D>(ra, ch) * 16 + off);
    const u32x2 hi = lds_read_tr(tile, rb * RB + bswz<D>(rb, ch) * 16 + off);
    return bits<Frag>(u32x4{lo[0], lo[1], hi[0], hi[1]});
  };

  // Tiles 0 to 2 before the loop, tile t + 3 after the barrier of tile t
  // (into the buffer of tile t - 1, whose reads all precede that barrier).
  // The register loads above land with tile 0.
  constexpr int LPW = TILE / 1024 / NWQ;
  issue(0);
  issue(1);
  issue(2);
  wait_loads<4 * LPW>();
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      fence(qf[qb][ks]);
      fence(df[qb][ks]);
    }
    fence(lse2[qb]);
    fence(drow[qb]);
  }
  for (int t = 0; t < n_tiles; ++t) {
    wait_loads<4 * LPW>();  // tile t has landed; tiles t + 1, t + 2 may be in flight
    block_barrier();
    issue(t + 3);
    if (t < wave_tiles) {
      const int buf = t % NBQ;
      const char* ktile = &smem[buf][0][0];
      const char* vtile = &smem[buf][1][0];
      const int64_t k0 = (int64_t)t * kBwdTile;
#pragma unroll
      for (int st = 0; st < kBwdTile / 32; ++st) {
        // S^T = K Q^T and dP^T = V dO^T for the step's two 16-key blocks:
        // register r of block b holds key 8*lg + 4*b + r of the step.
        f32x4 s[2][2], dp[2][2];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) s[b][qb] = dp[b][qb] = f32x4{};
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int ks = 0; ks < NKS; ++ks) {
            const int r = 32 * st + 4 * b + krow;
            const Frag ak = row_frag(ktile, r, 4 * ks + lg);
            const Frag av = row_frag(vtile, r, 4 * ks + lg);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
              s[b][qb] = mma16<T>(ak, qf[qb][ks], s[b][qb]);
              dp[b][qb] = mma16<T>(av, df[qb][ks], dp[b][qb]);
            }
          }
        // Key kbase + kr (kr = 8*lg + 4*b + r) is visible iff kr < N - kbase,
        // the query exists, and, when causal, kr <= query - kbase.
        const int64_t kbase = k0 + 32 * st;
        const bool full = kbase + 32 <= N && qw + 32 <= N && (!CAUSAL || kbase + 31 <= qw);
        Frag sf[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          float pr[2][4];
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              pr[b][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][qb][r], c, -lse2[qb]));
          if (__builtin_expect(!full, 0)) {
            const int64_t qr = qw + 16 * qb + l16;
            int64_t hi64 = qr < N ? N - kbase : 0;
            if (CAUSAL && qr - kbase + 1 < hi64) hi64 = qr - kbase + 1;
            const int hi = (int)(hi64 < 0 ? 0 : (hi64 > 32 ? 32 : hi64)) - 8 * lg;
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * b + r >= hi) pr[b][r] = 0.f;
          }
          // dS^T as the B operand of dQ^T += K^T dS^T: keys 8*lg + 0..7.
          u32x4 fs;
#pragma unroll
          for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              const int r = 2 * e;
              fs[2 * b + e] = bits<uint32_t>(H::pack(pr[b][r] * (dp[b][qb][r] - drow[qb]),
                                                     pr[b][r + 1] * (dp[b][qb][r + 1] - drow[qb])));
            }
          sf[qb] = bits<Frag>(fs);
        }
        // dQ^T += K^T dS^T.
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const Frag a = kt_frag(ktile, 32 * st, db);
#pragma unroll
          for (int qb = 0; qb < 2; ++qb) dq[db][qb] = mma16<T>(a, sf[qb], dq[db][qb]);
        }
      }
    }
  }
  wait_loads<0>();  // the empty loads past the end land before the workgroup ends

  // Lane (l16, lg) holds dQ[query][16*db + 4*lg .. +3] of query qw + 16*qb + l16.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int64_t qr = qw + 16 * qb + l16;
    if (qr < N) {
      T* dst = (T*)p.dq + (bh * N + qr) * D + 4 * lg;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const Pair a = H::pack(dq[db][qb][0] * p.scale, dq[db][qb][1] * p.scale);
        const Pair b2 = H::pack(dq[db][qb][2] * p.scale, dq[db][qb][3] * p.scale);
        *(u32x2*)(dst + 16 * db) = u32x2{bits<uint32_t>(a), bits<uint32_t>(b2)};
      }
    }
  }
}

// XCD-aware order. Causal: two query blocks of one head per workgroup, back to
// back, block n - 1 - i and then block i, so that every workgroup has about
// the same number of visible key tiles.
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(kBwdWavesQ * 64, 1) bwd_dq_kernel(BwdParams p) {
  const int logical = xcd_order();
  if constexpr (!CAUSAL) {
    dq_block<T, D, CAUSAL>(p, logical / p.n_blk_q, logical % p.n_blk_q);
  } else {
    const int pairs = (p.n_blk_q + 1) / 2;
    const int64_t bh = logical / pairs;
    const int i = logical % pairs;
    dq_block<T, D, CAUSAL>(p, bh, p.n_blk_q - 1 - i);
    if (i != p.n_blk_q - 1 - i) {
      block_barrier();  // every wave's reads of the first block's tiles are done
      dq_block<T, D, CAUSAL>(p, bh, i);
    }
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch(const BwdArgs& a, hipStream_t stream) {
  BwdParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.dout = a.dout;
  p.lse = a.lse;
  p.dq = a.dq;
  p.dk = a.dk;
  p.dv = a.dv;
  p.delta = (float*)a.workspace;
  p.lse2 = p.delta + a.BH * a.N;
  p.N = a.N;
  p.n_blk = (int32_t)((a.N + kBwdRows - 1) / kBwdRows);
  p.n_blk_q = (int32_t)((a.N + 32 * kBwdWavesQ - 1) / (32 * kBwdWavesQ));
  p.c = a.scale * kLog2e;
  p.scale = a.scale;
  const int64_t rows = a.BH * a.N;
  constexpr int RPB = 256 / (D / 8);
  hipLaunchKernelGGL((bwd_prep_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                     stream, p, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const unsigned grid = (unsigned)(a.BH * (CAUSAL ? (p.n_blk + 1) / 2 : p.n_blk));
  hipLaunchKernelGGL((bwd_dkdv_kernel<T, D, CAUSAL>), dim3(grid), dim3(512), 0, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL>), dim3((unsigned)(a.BH * (CAUSAL ? (p.n_blk_q + 1) / 2 : p.n_blk_q))),
                     dim3(kBwdWavesQ * 64), 0, stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const BwdArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch<T, 64, true>(a, s) : launch<T, 64, false>(a, s);
  return a.causal ? launch<T, 128, true>(a, s) : launch<T, 128, false>(a, s);
}

}  // namespace

hipError_t launch_backward(const BwdArgs& a, hipStream_t stream) {
  return a.dtype == Dtype::BF16 ? launch_t<__bf16>(a, stream) : launch_t<_Float16>(a, stream);
}

}  // namespace fa
