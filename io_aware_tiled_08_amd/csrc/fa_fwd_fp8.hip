// FlashAttention forward pass with 8-bit (e4m3) Q, K and V on gfx950.
//
// What is computed: for every (batch, head), with q, k, v holding e4m3 codes
// and per-tensor descale factors (the real values are code * descale),
//   O = softmax(scale * Q K^T) V   (written as bf16)   and   LSE per row,
// by the method of the 16-bit kernel: K and V tiles staged on chip, a running
// maximum and sum per query row, accumulated output rescaled when the maximum
// grows, O written once ("FlashAttention, Playable", EP 03 and EP 04; chapter
// 15 "The Tiling Strategy"; "FlashAttention: Tiled & Fused", hero diagram).
// The 8-bit variant is the one the FlashAttention chapter lists among the
// later versions ("FlashAttention Evolution": FP8 support).
//
// CDNA4 mapping: the 16-bit kernel's workgroup (8 waves x 32 query rows, two
// wave groups in alternating matrix / softmax phases, 128-key tiles double
// buffered in LDS by direct-to-LDS loads), with these differences:
//   * both products run on v_mfma_scale_f32_32x32x64_f8f6f4 with e4m3
//     operands and unit block scales: 64 products deep, twice the 16-bit rate.
//     Operand k slot (h, j) is byte j of the 32 a lane in half h supplies.
//   * S^T = K Q^T: d slot (h, j) of a 64-wide d chunk is d = 32h + j, so a
//     lane reads 32 contiguous bytes of its K row and of its Q row.
//   * Keys: within each 64-key chunk of a tile, score row rho of 32-key block
//     b stands for key 32*((rho>>2)&1) + 16b + 4*(rho>>3) + (rho&3).  Then the
//     32 scores a lane of half h holds for the chunk are keys 32h .. 32h+31 in
//     register order, which is exactly k slot (h, j) = key 32h + j of the P V
//     product: P^T is packed from the score registers (rounded to e4m3, RNE)
//     and V^T rows 32h + j are read from row-major V in LDS with transposing
//     8-bit reads (ds_read_b64_tr_b8).
//   * The row sum l is the sum of the rounded weights, computed by the matrix
//     unit: per chunk, one 16x16x128 product of the P fragment against a
//     patterned ones operand, which gives every lane its own query's sum.
//   * The softmax weights are at most 2^8 (the lazy-rescale slack) and the
//     largest e4m3 value is 448, so rounding P never overflows.
// Accuracy: every step is exact or fp32 except the rounding of the weights to
// e4m3 (and of O to bf16); the bound that follows from that rounding is the
// accuracy contract (per element: sum_j max(2^-4 w_j, 2^-10)|v_j - O| /
// (sum w - sum of those terms), weights w_j = exp(s_j - s_max)).
#include "fa_device.h"
#include "fa_f16_common.h"
#include "fa_fp8.h"

namespace fa {
namespace {

struct Fp8Params {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t N;
  int32_t n_qblk;   // query blocks per (b, h)
  float c;          // |scale| * q_descale * k_descale * log2(e)
  uint32_t q_sign;  // XOR mask on Q's bytes: flips Q's sign when scale < 0
  float o_scale;    // v_descale
};

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// ds_read_b64_tr_b8: within each group of 16 lanes, output lane i, byte e
// receives byte i%8 of the 8 bytes addressed by lane 2e + i/8 of the group.
// When lanes 2e and 2e+1 address columns c0..c0+7 and c0+8..c0+15 of row r_e
// of a row-major byte matrix, output lane i receives column c0 + i of rows
// r_0 .. r_7.
__device__ __forceinline__ u32x2 lds_read_tr8(const char* base, int byte_off) {
  lds_i32x2* ptr = (lds_i32x2*)((lds_char*)const_cast<char*>(base) + byte_off);
  return bits<u32x2>(__builtin_amdgcn_ds_read_tr8_b64_v2i32(ptr));
}

// e4m3 x e4m3 (format code 0 for A and B), block scales 2^0 (E8M0 127).
__device__ __forceinline__ f32x16 mma8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// Row sums of a P^T fragment in the 32x32x64 B layout (lane l: query l%32,
// keys 32*(l/32) .. +31 of the chunk), by one 16x16x128 product (same formats
// and scales).  Read as a 16x16x128 B operand, lane l = n + 16g is column n of
// k group g and holds query n + 16*(g%2), keys 32*(g/2) ..; the A operand
// row m (lanes m + 16g) is all ones in the k groups g with g%2 == (m/4)%2 and
// zero elsewhere.  Output row m, column n then sums both key halves of query
// n + 16*((m/4)%2), and the 16x16 output layout puts rows 4(l/16) .. +3 of
// column l%16 in lane l: the sum of lane l's own query l%32, in all four
// registers.
__device__ __forceinline__ f32x4 rowsum8(i32x8 sel_ones, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel_ones, b, c, 0, 0, 0, 127, 0, 127);
}

// Four floats to four e4m3 bytes (round to nearest even), first in byte 0.
__device__ __forceinline__ uint32_t pack4_e4m3(float a, float b, float c, float d) {
  // The first conversion writes bytes 0-1 and the second bytes 2-3, so the
  // word's initial contents do not matter; starting from a's bits (a register
  // that dies here) saves clearing one.
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __builtin_bit_cast(int, a), false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Position of 16-byte chunk c of row r inside the LDS row (rows are D bytes;
// an XOR with a row-dependent mask, so its own inverse).  K: the 16 lanes of a
// 16-byte read hit 16 rows {0..7, 32..39} (+16b) of a chunk; V: the 32 lanes
// of an 8-byte transposing read hit 8 consecutive rows, two chunks each.
template <int D>
struct Swizzle8 {
  static_assert(D == 64 || D == 128, "head dim");
  static __device__ __forceinline__ constexpr int k(int r, int c) {
    return D == 128 ? c ^ (((r >> 1) & 3) | (((r >> 5) & 1) << 2))
                    : c ^ (((r >> 2) & 1) | (((r >> 5) & 1) << 1));
  }
  static __device__ __forceinline__ constexpr int v(int r, int c) {
    return D == 128 ? c ^ (((r >> 1) & 3) << 1) : c ^ (((r >> 2) & 1) << 1);
  }
};

// Key (within a 64-key chunk) that score row rho of 32-key block b stands for.
__device__ __forceinline__ constexpr int key8(int b, int rho) {
  return 32 * ((rho >> 2) & 1) + 16 * b + 4 * (rho >> 3) + (rho & 3);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(512, 1) fwd_fp8_kernel(Fp8Params p) {
  using Sw = Swizzle8<D>;
  constexpr int NW = 8;            // waves per workgroup
  constexpr int BR = NW * 32;      // query rows per workgroup
  constexpr int BC = 128;          // keys per tile
  constexpr int RB = D;            // bytes per row of K or V
  constexpr int CPR = D / 16;      // 16-byte chunks per row
  constexpr int TILE = BC * RB;    // bytes of one staged K (or V) tile
  constexpr int NKB = BC / 32;     // 32-key score blocks per tile
  constexpr int NKC = BC / 64;     // 64-key chunks per tile (P V depth)
  constexpr int NKS = D / 64;      // MFMAs per score block
  constexpr int ND = D / 32;       // 32-row blocks of O^T (product slot ND: row sums)
  constexpr int RPL = 1024 / RB;   // rows one wave-wide 1 KiB load covers
  constexpr int LPW = TILE / 1024 / 4;  // 1 KiB loads per loading wave per tensor
  static_assert(LPW >= 1 && TILE % 4096 == 0, "tile shape");

  __shared__ __attribute__((aligned(1024))) char smem[2][2][TILE];  // [K, V][buffer]

  const WorkItem wi = work_item<CAUSAL>(p.n_qblk);
  const int64_t N = p.N;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool group_b = wave >= 4;
  const int gw = wave & 3;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int64_t q0 = (int64_t)wi.qblk * BR;
  const int64_t qw = q0 + (int64_t)wave * 32;
  const int64_t qrow = qw + l32;

  const uint8_t* __restrict__ Qh = (const uint8_t*)p.q + wi.bh * N * D;
  const uint8_t* __restrict__ Kh = (const uint8_t*)p.k + wi.bh * N * D;
  const uint8_t* __restrict__ Vh = (const uint8_t*)p.v + wi.bh * N * D;
  __bf16* __restrict__ Oh = (__bf16*)p.o + wi.bh * N * D;
  float* __restrict__ Lh = p.lse + wi.bh * N;

  const int64_t kv_end = CAUSAL ? (q0 + BR < N ? q0 + BR : N) : N;
  const int n_tiles = (int)((kv_end + BC - 1) / BC);
  const int64_t wave_end = CAUSAL ? (qw + 32 < N ? qw + 32 : N) : N;
  const int wave_tiles = qw < N ? (int)((wave_end + BC - 1) / BC) : 0;

  // ---- tile loads: global -> LDS, 16 bytes per lane (K: group B, V: group A) 
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
    for (int j = 0; j < LPW; ++j) dma_load16(rs, lds_k + (t & 1) * TILE + j * 1024, kvoff[j]);
  };
  auto issue_v = [&](int t) {
    if (t >= n_tiles) return;
    const int64_t k0 = (int64_t)t * BC;
    const uint32_t rows = (uint32_t)(N - k0 < BC ? N - k0 : BC);
    const u32x4 rs = buffer_rsrc(Vh + k0 * D, rows * RB);
#pragma unroll
    for (int j = 0; j < LPW; ++j) dma_load16(rs, lds_v + (t & 1) * TILE + j * 1024, vvoff[j]);
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

  // Q (B operand of S^T = K Q^T): lane holds Q[qrow][64*ks + 32*hh .. +31].
  i32x8 qf[NKS];
  {
    const bool ok = qrow < N;
    const uint8_t* src = Qh + (ok ? qrow : 0) * D + hh * 32;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 lo = ok ? *(const u32x4*)(src + ks * 64) : u32x4{0, 0, 0, 0};
      u32x4 hi = ok ? *(const u32x4*)(src + ks * 64 + 16) : u32x4{0, 0, 0, 0};
      lo ^= p.q_sign;
      hi ^= p.q_sign;
      qf[ks] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  }
  if (group_b) issue_k(0);

  // ---- lane-constant LDS read offsets ----------------------------------------
  // K A operand of score block b (of a 64-key chunk), d chunk ks: row key8(b,
  // l32), bytes 64*ks + 32*hh .. +31 (two 16-byte chunks).  The swizzle does
  // not see the chunk's base row (a multiple of 64).
  int koff[2][NKS][2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int r = key8(b, l32);
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
      for (int u = 0; u < 2; ++u) koff[b][ks][u] = r * RB + Sw::k(r, 4 * ks + 2 * hh + u) * 16;
  }
  // V^T A operand of O^T block db, key chunk c, read t (keys 32*hh + 8t .. +7):
  // lane i of 16-lane group g addresses row 64c + 32*hh + 8t + i/2, columns
  // 32*db + 16*(g%2) + 8*(i%2) .. +7.  The swizzle only sees row bits 0-2.
  int voff[ND];
  {
    const int g = lane >> 4, i16 = lane & 15;
    const int vrow = 32 * hh + (i16 >> 1);
#pragma unroll
    for (int db = 0; db < ND; ++db)
      voff[db] = vrow * RB + Sw::v(vrow, 2 * db + (g & 1)) * 16 + 8 * (i16 & 1);
  }
  // e4m3 1.0 in every byte of the lanes whose k group parity matches their
  // output row block parity (rowsum8).
  const int one_w = ((lane >> 4) & 1) == ((lane >> 2) & 1) ? 0x38383838 : 0;
  const i32x8 ones = {one_w, one_w, one_w, one_w, one_w, one_w, one_w, one_w};

  // ---- running state ----------------------------------------------------------
  f32x16 o[ND];        // O^T blocks
  f32x4 lsum = f32x4{};  // the row sum l (every register holds it)
#pragma unroll
  for (int db = 0; db < ND; ++db) o[db] = f32x16{};
  f32x16 s[NKB];
  i32x8 pf[NKC];
  float m = kNegInf;  // reference maximum of the row, log2 units
  const float c = p.c;

  // M phase of tile t: O += P(t-1) V(t-1) (with the row-sum product), then
  // S(t) = K(t) Q^T.  Operand reads run kPipe products ahead of the products.
  constexpr int NPV = NKC * (ND + 1);
  constexpr int NS = NKB * NKS;
  constexpr int kPipe = 3;
  auto fetch = [&](const char* vl, const char* kl, int i) -> i32x8 {
    if (i < NPV) {
      const int ch = i / (ND + 1), db = i % (ND + 1);
      if (db == ND) return ones;
      u32x2 r[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) r[t] = lds_read_tr8(vl, (64 * ch + 8 * t) * RB + voff[db]);
      return i32x8{(int)r[0][0], (int)r[0][1], (int)r[1][0], (int)r[1][1],
                   (int)r[2][0], (int)r[2][1], (int)r[3][0], (int)r[3][1]};
    }
    const int j = i - NPV, ks = j / NKB, kb = j % NKB;
    const char* row = kl + 64 * (kb >> 1) * RB;
    const u32x4 lo = *(const u32x4*)(row + koff[kb & 1][ks][0]);
    const u32x4 hi = *(const u32x4*)(row + koff[kb & 1][ks][1]);
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                 (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto apply = [&](int i, i32x8 a) {
    if (i < NPV) {
      const int ch = i / (ND + 1), db = i % (ND + 1);
      if (db == ND)
        lsum = rowsum8(a, pf[ch], lsum);
      else
        o[db] = mma8(a, pf[ch], o[db]);
    } else {
      const int j = i - NPV, ks = j / NKB, kb = j % NKB;
      s[kb] = mma8(a, qf[ks], s[kb]);
    }
  };
  auto m_pv_s = [&](int t) {
    const char* vl = &smem[1][(t - 1) & 1][0];
    const char* kl = &smem[0][t & 1][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
    i32x8 ring[kPipe];
#pragma unroll
    for (int i = 0; i < kPipe; ++i) ring[i] = fetch(vl, kl, i);
#pragma unroll
    for (int i = 0; i < NPV + NS; ++i) {
      const i32x8 a = ring[i % kPipe];
      if (i + kPipe < NPV + NS) ring[i % kPipe] = fetch(vl, kl, i + kPipe);
      apply(i, a);
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
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int i = NPV; i < NPV + NS; ++i) apply(i, fetch(kl, kl, i));
  };

  // V phase of tile t: online softmax of S(t) into P(t).
  auto v_phase = [&](int t) {
    const int64_t k0 = (int64_t)t * BC;
    int64_t lim64 = N - k0;
    if (CAUSAL && qrow + 1 - k0 < lim64) lim64 = qrow + 1 - k0;
    const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > qw);
    if (need_mask) {
      // Register r of block kb holds key 64*(kb/2) + 32*hh + 16*(kb%2) + r.
      const int lim = (int)(lim64 < 0 ? 0 : (lim64 > BC ? BC : lim64)) - 32 * hh;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (64 * (kb >> 1) + 16 * (kb & 1) + r >= lim) s[kb][r] = kNegInf;
    }
    float mx = chain_max4<NKB * 16>([&](int i) { return s[i / 16][i % 16]; });
    mx = halves_max(mx);
    const float mxc = mx * c;  // c > 0, so -inf stays -inf
    const bool grow = mxc > m + kRescaleSlack;
    if (__ballot(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - mxc) : 1.0f;
      m = grow ? mxc : m;
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] *= alpha;
      lsum *= alpha;
    }
    const float m_use = m == kNegInf ? 0.f : m;
    // P = exp2(c*s - m), rounded to e4m3; byte j of chunk ch's operand is
    // register j%16 of score block 2*ch + j/16.
#pragma unroll
    for (int ch = 0; ch < NKC; ++ch) {
      i32x8 f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int kb = 2 * ch + (w >> 2), r = 4 * (w & 3);
        float e[4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
          e[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + x], c, -m_use));
        f[w] = (int)pack4_e4m3(e[0], e[1], e[2], e[3]);
      }
      pf[ch] = f;
    }
#pragma unroll
    for (int ch = 0; ch < NKC; ++ch) fence(pf[ch]);
    fence(m);
  };

  wait_loads();
  barrier();

  // The same slot schedule as the 16-bit kernel: group A runs M(t) while group
  // B runs V(t-1), then they swap.  Loads as in the 16-bit kernel at d = 64:
  // group B issues K(t+2) at the start of its V phase; group A issues V(t) at
  // the end of its M(t) (its buffer's last reader, B's M(t-1), finished a slot
  // earlier) and waits for it at the end of its V(t) phase, before V(t)'s first
  // reader in slot 2t+2.  With the products at twice the 16-bit rate the
  // softmax phase is the longer one, so A issues in time it would otherwise
  // spend waiting at the barrier.
  auto iteration = [&](int t, auto mwork, auto vwork) {
    wave_priority<1>();
    mwork();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) fence(s[kb]);
#pragma unroll
    for (int db = 0; db < ND; ++db) fence(o[db]);
    fence(lsum);
    wave_priority<0>();
    if (!group_b) issue_v(t);  // A: V(t) at the end of its M(t), in slot 2t
    if (group_b) wait_loads();
    barrier();
    if (group_b) issue_k(t + 2);
    vwork();
    if (!group_b) wait_loads();
    barrier();
  };
  const int W = wave_tiles;
  if (group_b) {
    issue_k(1);
    barrier();
  }
  iteration(
      0, [&] { if (W >= 1) m_s(0); }, [&] { if (W >= 1) v_phase(0); });
  for (int t = 1; t < W; ++t) iteration(t, [&] { m_pv_s(t); }, [&] { v_phase(t); });
  if (W >= 1) iteration(W, [&] { m_pv(W); }, [] {});
  for (int t = W >= 1 ? W + 1 : 1; t <= n_tiles; ++t) iteration(t, [] {}, [] {});
  if (!group_b) barrier();

  // ---- epilogue: O = O_acc * v_descale / l (bf16), LSE = (m + log2 l) ln 2 --
  const float lt = lsum[0];
  if (qrow < N) {
    const float inv = p.o_scale / lt;
    if (hh == 0) Lh[qrow] = (m + __builtin_amdgcn_logf(lt)) * kLn2;
    __bf16* dst = Oh + qrow * D + hh * 4;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const bf16x2 lo = __builtin_convertvector((f32x2){o[db][4 * g] * inv, o[db][4 * g + 1] * inv}, bf16x2);
        const bf16x2 hi =
            __builtin_convertvector((f32x2){o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv}, bf16x2);
        *(u32x2*)(dst + db * 32 + g * 8) = u32x2{bits<uint32_t>(lo), bits<uint32_t>(hi)};
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const Fp8Args& a, hipStream_t stream) {
  constexpr int BR = 256;
  static_assert(BR == kRowsPerWorkgroupFp8, "rows per workgroup");
  Fp8Params p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.N = a.N;
  p.n_qblk = (int32_t)((a.N + BR - 1) / BR);
  // |scale| * q_descale * k_descale * log2(e), at least the smallest normal float.
  p.c = __builtin_fmaxf(__builtin_fabsf(a.scale) * a.q_descale * a.k_descale * kLog2e,
                        1.17549435e-38f);
  p.q_sign = a.scale < 0.f ? 0x80808080u : 0u;
  p.o_scale = a.v_descale;
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3((unsigned)(a.BH * p.n_qblk)), dim3(512), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_fp8(const Fp8Args& a, hipStream_t stream) {
  if (a.d == 64) return a.causal ? launch<64, true>(a, stream) : launch<64, false>(a, stream);
  return a.causal ? launch<128, true>(a, stream) : launch<128, false>(a, stream);
}

}  // namespace fa
