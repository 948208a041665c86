// Attention of new queries against a key/value cache (decode), fp16 and bf16,
// on gfx950.
//
// What is computed: for every (batch, head), the Nq query rows are the last Nq
// positions of a sequence whose keys and values are all in the cache (Nk rows;
// "FlashAttention: Tiled & Fused", related-diagram card "KV Cache: Why
// Generation Speeds Up": generation stores and reuses the keys and values of
// earlier tokens).  O = softmax(scale * Q K^T) V and the
// natural-log LSE of each score row, where a causal query i sees the keys
// j <= i + (Nk - Nq).  The method is the one of the square kernel: K and V
// tiles staged on chip, an online softmax with a running maximum and sum
// ("FlashAttention, Playable", EP 03 and EP 04; chapter 15 "The Tiling
// Strategy"), O written once.
//
// CDNA4 design.  With few queries, every cached key is read once per 32-query
// block and used for little arithmetic, so the kernel is bound by HBM, and the
// design is about bytes in flight, not matrix throughput:
//   * the keys are split into ranges (splits); one workgroup per (batch*head,
//     32-query block, split), so that a single head at batch 1 still fills
//     the GPU;
//   * inside a workgroup every wave walks its own 32-key tiles (wave w takes
//     every NW-th tile of the range) through its own LDS stages (kv_bufs),
//     filled by buffer_load ... lds one tile ahead and waited for with the
//     wave's own vmcnt, so waves never wait for each other in the loop;
//   * per tile: S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16 (query
//     rows past Nq are zero and never stored), the online softmax in between;
//   * the waves' partial (m, l, O) are merged through LDS with weights
//     2^(m_w - M) -- the rescale rule of the online softmax, applied once
//     across waves.  A workgroup writes the final O and LSE when there is one
//     split, otherwise its range's normalised O and its LSE to the workspace,
//     and the merge kernel below combines the ranges with the same rule.
#include <mutex>

#include "fa_device.h"
#include "fa_f16_common.h"
#include "fa_kvcache.h"

#include <type_traits>

namespace fa {
namespace {

struct KvParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* ws_o;    // [n_split][BH * Nq][D] fp32, used when n_split > 1
  float* ws_lse;  // [n_split][BH * Nq]
  int64_t Nq;
  int64_t Nk;
  int64_t off;         // Nk - Nq: key index of query 0's own position (causal)
  int64_t rows_total;  // BH * Nq
  int32_t n_qblk;
  int32_t n_split;
  int32_t tiles_per_split;
  float c;          // |scale| * log2(e)
  uint32_t q_sign;  // XOR mask flipping Q's sign when scale < 0
};

template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(kv_waves(D) * 64, 1) kvcache_fwd_kernel(KvParams p) {
  using H = Half<T>;
  using Frag = typename H::Frag;
  using Pair = typename H::Pair;
  using Sw = Swizzle<D>;
  constexpr int NW = kv_waves(D);
  constexpr int NT = NW * 64;
  constexpr int RB = D * 2;              // bytes per row of K or V
  constexpr int CPR = D / 8;             // 16-byte chunks per row
  constexpr int TILE = kKvKeys * RB;     // bytes of one K (or V) tile
  constexpr int LPT = TILE / 1024;       // 1 KiB loads per tensor per tile
  constexpr int RPL = 1024 / RB;         // rows one 1 KiB load covers
  constexpr int NKS = D / 16;            // MFMAs per score block
  constexpr int ND = D / 32;             // 32-row blocks of O^T
  constexpr int NBUF = kv_bufs(D);       // LDS stages per wave
  constexpr int WAVE_LDS = NBUF * 2 * TILE;  // [stage][K, V][tile]
  constexpr int OS = D + 4;              // row stride (floats) of a wave's partial O
  static_assert(NW * kKvRows * OS * 4 <= NW * WAVE_LDS, "merge area fits the tile buffers");
  static_assert(NBUF >= 2 && NBUF <= 4, "stages");

  __shared__ __attribute__((aligned(1024))) char smem[NW * WAVE_LDS];
  __shared__ float m_lds[NW][kKvRows];
  __shared__ float l_lds[NW][kKvRows];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // Work item: split fastest, then query block, then batch*head.
  const int split = blockIdx.x % p.n_split;
  const int rest = blockIdx.x / p.n_split;
  const int qblk = rest % p.n_qblk;
  const int64_t bh = rest / p.n_qblk;
  const int64_t Nq = p.Nq, Nk = p.Nk;
  const int64_t q0 = (int64_t)qblk * kKvRows;
  const int64_t qrow = q0 + l32;

  const T* __restrict__ Qh = (const T*)p.q + bh * Nq * D;
  const T* __restrict__ Kh = (const T*)p.k + bh * Nk * D;
  const T* __restrict__ Vh = (const T*)p.v + bh * Nk * D;

  // Keys this block can see, and this split's tiles of them.
  const int64_t kv_end = CAUSAL ? (q0 + kKvRows + p.off < Nk ? q0 + kKvRows + p.off : Nk) : Nk;
  const int vis_tiles = (int)((kv_end + kKvKeys - 1) / kKvKeys);
  const int t_begin = split * p.tiles_per_split;
  const int t_end = t_begin + p.tiles_per_split < vis_tiles ? t_begin + p.tiles_per_split : vis_tiles;
  const int first = t_begin + wave;
  const int n_my = first < t_end ? (t_end - 1 - first) / NW + 1 : 0;

  // ---- per-wave tile loads: global -> this wave's LDS buffers -------------
  // Load j covers rows j*RPL .. +RPL; lane i fills LDS chunk slot i%CPR of row
  // j*RPL + i/CPR, which holds global chunk slot ^ mask(row).
  int kvoff[LPT], vvoff[LPT];
#pragma unroll
  for (int j = 0; j < LPT; ++j) {
    const int r = j * RPL + lane / CPR;
    const int slot = lane % CPR;
    kvoff[j] = r * RB + Sw::k(r, slot) * 16;
    vvoff[j] = r * RB + Sw::v(r, slot) * 16;
  }
  char* wlds = smem + wave * WAVE_LDS;
  const uint32_t wlds_addr = lds_addr(wlds);
  auto issue = [&](int i) {  // tile first + i*NW into stage i % NBUF
    const int64_t k0 = (int64_t)(first + i * NW) * kKvKeys;
    const uint32_t rows = (uint32_t)(Nk - k0 < kKvKeys ? Nk - k0 : kKvKeys);
    const u32x4 rk = buffer_rsrc(Kh + k0 * D, rows * RB);
    const u32x4 rv = buffer_rsrc(Vh + k0 * D, rows * RB);
    const uint32_t base = wlds_addr + (i % NBUF) * 2 * TILE;
#pragma unroll
    for (int j = 0; j < LPT; ++j) dma_load16(rk, base + j * 1024, kvoff[j]);
#pragma unroll
    for (int j = 0; j < LPT; ++j) dma_load16(rv, base + TILE + j * 1024, vvoff[j]);
  };
  // Wait until at most `tiles` tiles' loads of this wave are outstanding:
  // vmcnt(tiles * 2 * LPT) with the other counters left alone (gfx9
  // s_waitcnt encoding); no LDS read may move above the wait.
  auto wait_tiles = [](auto tiles) {
    constexpr int n = decltype(tiles)::value * 2 * LPT;
    static_assert(n < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70 | (n & 15) | ((n >> 4) << 14));
    asm volatile("" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // Q (B operand of S^T = K Q^T): lane holds Q[qrow][16*ks + 8*hh .. +7].
  Frag qf[NKS];
  {
    const bool ok = qrow < Nq;
    const T* src = Qh + (ok ? qrow : 0) * D + hh * 8;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      u32x4 raw = ok ? *(const u32x4*)(src + ks * 16) : u32x4{0, 0, 0, 0};
      raw ^= p.q_sign;
      qf[ks] = bits<Frag>(raw);
    }
  }
#pragma unroll
  for (int j = 0; j < NBUF - 1; ++j)
    if (j < n_my) issue(j);
  // The Q loads must land now: the compiler does not count the tile loads,
  // so a wait it placed for Q inside the loop would also drain the prefetch.
  wait_tiles(std::integral_constant<int, 0>{});
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) fence(qf[ks]);

  // Lane-constant LDS read offsets (same operand layout as the square kernel).
  const int krow = k_row_of_lane(l32);
  int koff[NKS];
#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) koff[ks] = krow * RB + Sw::k(krow, 2 * ks + hh) * 16;
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

  f32x16 o[ND];
#pragma unroll
  for (int db = 0; db < ND; ++db) o[db] = f32x16{};
  float m = kNegInf;  // reference maximum of the row, log2 units
  float l = 0.f;      // this lane's share of the row sum
  const float c = p.c;
  // Last key this lane's query may see, plus one.
  const int64_t row_end = CAUSAL ? (qrow + 1 + p.off < Nk ? qrow + 1 + p.off : Nk) : Nk;

  for (int i = 0; i < n_my; ++i) {
    // Keep NBUF - 1 tiles in flight; then tile i is the oldest outstanding.
    if (i + NBUF - 1 < n_my) {
      issue(i + NBUF - 1);
      wait_tiles(std::integral_constant<int, NBUF - 1>{});
    } else if (NBUF >= 3 && n_my - 1 - i == 1) {
      wait_tiles(std::integral_constant<int, 1>{});
    } else if (NBUF >= 4 && n_my - 1 - i == 2) {
      wait_tiles(std::integral_constant<int, (NBUF >= 4 ? 2 : 0)>{});
    } else {
      wait_tiles(std::integral_constant<int, 0>{});
    }
    const char* kl = wlds + (i % NBUF) * 2 * TILE;
    const char* vl = kl + TILE;
    const int64_t k0 = (int64_t)(first + i * NW) * kKvKeys;

    // S^T = K Q^T for the tile's 32 keys.
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
      s = H::mma(bits<Frag>(*(const u32x4*)(kl + koff[ks])), qf[ks], s);

    // Keys k0 + r with r >= lim are invisible: past Nk, or after the query.
    const bool need_mask = (k0 + kKvKeys > Nk) || (CAUSAL && k0 + kKvKeys - 1 > q0 + p.off);
    if (need_mask) {
      int64_t lim64 = row_end - k0;
      const int lim = (int)(lim64 < 0 ? 0 : (lim64 > kKvKeys ? kKvKeys : lim64)) - 8 * hh;
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key_of_reg(r, 0) >= lim) s[r] = kNegInf;
    }
    float mx = tree_max<16>([&](int r) { return s[r]; });
    mx = halves_max(mx);
    const float mxc = mx * c;  // c > 0, so -inf stays -inf
    // Raise the reference maximum only when the tile exceeds it by the slack.
    const bool grow = mxc > m + kRescaleSlack;
    if (__ballot(grow)) {
      const float alpha = grow ? __builtin_amdgcn_exp2f(m - mxc) : 1.0f;
      m = grow ? mxc : m;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < ND; ++db) o[db] *= alpha;
    }
    const float m_use = m == kNegInf ? 0.f : m;
    // P = exp2(c*s - m) rounded to T; l sums the rounded weights.
    Frag pf[2];
    float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      u32x4 f;
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * jj + 2 * e], c, -m_use));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[8 * jj + 2 * e + 1], c, -m_use));
        const Pair pr = H::pack(e0, e1);
        acc = H::sum2(pr, acc);
        f[e] = bits<uint32_t>(pr);
      }
      (jj == 0 ? rs0 : rs1) = acc;
      pf[jj] = bits<Frag>(f);
    }
    l += rs0 + rs1;
    // O^T += V^T P^T.
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const int off = 16 * jj * RB + voff[db];
        const u32x2 lo = lds_read_tr(vl, off);
        const u32x2 hi = lds_read_tr(vl, off + 4 * RB);
        o[db] = H::mma(bits<Frag>(u32x4{lo[0], lo[1], hi[0], hi[1]}), pf[jj], o[db]);
      }
  }

  // ---- merge the waves' partial results (the tile buffers are reused) ----
  const float lt = halves_sum(l);
  __syncthreads();
  float* mo = (float*)smem;
  {
    float* ow = mo + (wave * kKvRows + l32) * OS + 4 * hh;
    // Accumulator register r holds O^T row 8*(r/4) + 4*hh + r%4 of its block.
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        *(float4*)(ow + db * 32 + 8 * g) =
            make_float4(o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]);
    if (hh == 0) {
      m_lds[wave][l32] = m;
      l_lds[wave][l32] = lt;
    }
  }
  __syncthreads();

  for (int item = tid; item < kKvRows * D / 4; item += NT) {
    const int row = item / (D / 4), c4 = item % (D / 4);
    const int64_t qi = q0 + row;
    if (qi >= Nq) continue;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, m_lds[w][row]);
    const float M_use = M == kNegInf ? 0.f : M;
    float L = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float wt = __builtin_amdgcn_exp2f(m_lds[w][row] - M_use);
      L += wt * l_lds[w][row];
      const float4 x = *(const float4*)(mo + (w * kKvRows + row) * OS + 4 * c4);
      acc.x += wt * x.x;
      acc.y += wt * x.y;
      acc.z += wt * x.z;
      acc.w += wt * x.w;
    }
    const int64_t grow_idx = bh * Nq + qi;
    if (p.n_split == 1) {
      const float inv = 1.0f / L;
      const Pair a = H::pack(acc.x * inv, acc.y * inv);
      const Pair b = H::pack(acc.z * inv, acc.w * inv);
      *(u32x2*)((T*)p.o + grow_idx * D + 4 * c4) = u32x2{bits<uint32_t>(a), bits<uint32_t>(b)};
      if (c4 == 0) p.lse[grow_idx] = (M + __builtin_amdgcn_logf(L)) * kLn2;
    } else {
      // A row that sees no key of this range: weight zero in the merge.
      const bool seen = L > 0.f;
      const float inv = seen ? 1.0f / L : 0.f;
      float* dst = p.ws_o + ((int64_t)split * p.rows_total + grow_idx) * D + 4 * c4;
      *(float4*)dst = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
      if (c4 == 0)
        p.ws_lse[(int64_t)split * p.rows_total + grow_idx] =
            seen ? (M + __builtin_amdgcn_logf(L)) * kLn2 : kNegInf;
    }
  }
}

// Merge of the splits' partial results: LSE = M + ln sum_s exp(lse_s - M),
// O = sum_s exp(lse_s - M) O_s / that sum, with M the largest lse_s (the
// online-softmax rescale rule).  One workgroup per output row: thread (g, c)
// owns output columns 4c..4c+3 and the splits s = g (mod G), so a row's
// splits are read in parallel; the G partial sums are added through LDS.
template <typename T, int D>
__global__ void __launch_bounds__(256) kvcache_merge_kernel(KvParams p) {
  using H = Half<T>;
  using Pair = typename H::Pair;
  constexpr int TPR = D / 4;     // threads per output row slice
  constexpr int G = 256 / TPR;   // split groups
  __shared__ float red[256];
  __shared__ float4 part[G][TPR];
  __shared__ float part_l[G];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int c4 = tid % TPR, g = tid / TPR;
  const int S = p.n_split;
  const float* lse_s = p.ws_lse + row;
  const int64_t stride = p.rows_total;

  float mx = kNegInf;
  for (int s = tid; s < S; s += 256) mx = fmaxf(mx, lse_s[s * stride]);
  red[tid] = mx;
  __syncthreads();
#pragma unroll
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  const float M_use = M == kNegInf ? 0.f : M;

  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = g; s < S; s += G) {
    const float wt = __builtin_amdgcn_exp2f((lse_s[s * stride] - M_use) * kLog2e);
    const float4 x = *(const float4*)(p.ws_o + ((int64_t)s * stride + row) * D + 4 * c4);
    L += wt;
    acc.x += wt * x.x;
    acc.y += wt * x.y;
    acc.z += wt * x.z;
    acc.w += wt * x.w;
  }
  part[g][c4] = acc;
  if (c4 == 0) part_l[g] = L;
  __syncthreads();
  if (g == 0) {
    L = 0.f;
    acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const float4 x = part[j][c4];
      L += part_l[j];
      acc.x += x.x;
      acc.y += x.y;
      acc.z += x.z;
      acc.w += x.w;
    }
    const float inv = 1.0f / L;
    const Pair a = H::pack(acc.x * inv, acc.y * inv);
    const Pair b = H::pack(acc.z * inv, acc.w * inv);
    *(u32x2*)((T*)p.o + row * D + 4 * c4) = u32x2{bits<uint32_t>(a), bits<uint32_t>(b)};
    if (c4 == 0) p.lse[row] = M + __builtin_amdgcn_logf(L) * kLn2;
  }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch(const KvArgs& a, hipStream_t stream) {
  KvParams p;
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.o = a.o;
  p.lse = a.lse;
  p.ws_o = (float*)a.workspace;
  p.ws_lse = a.workspace ? (float*)a.workspace + (int64_t)a.n_split * a.BH * a.Nq * D : nullptr;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.off = a.Nk - a.Nq;
  p.rows_total = a.BH * a.Nq;
  p.n_qblk = (int32_t)((a.Nq + kKvRows - 1) / kKvRows);
  p.n_split = a.n_split;
  p.tiles_per_split = a.tiles_per_split;
  p.c = __builtin_fmaxf(__builtin_fabsf(a.scale) * kLog2e, 1.17549435e-38f);
  p.q_sign = a.scale < 0.f ? 0x80008000u : 0u;
  const unsigned grid = (unsigned)(a.BH * p.n_qblk * p.n_split);
  hipLaunchKernelGGL((kvcache_fwd_kernel<T, D, CAUSAL>), dim3(grid), dim3(kv_waves(D) * 64), 0,
                     stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.n_split == 1) return e;
  hipLaunchKernelGGL((kvcache_merge_kernel<T, D>), dim3((unsigned)p.rows_total), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const KvArgs& a, hipStream_t s) {
  if (a.d == 64) return a.causal ? launch<T, 64, true>(a, s) : launch<T, 64, false>(a, s);
  return a.causal ? launch<T, 128, true>(a, s) : launch<T, 128, false>(a, s);
}

}  // namespace

hipError_t launch_kvcache(const KvArgs& a, hipStream_t stream) {
  return a.dtype == Dtype::BF16 ? launch_t<__bf16>(a, stream) : launch_t<_Float16>(a, stream);
}

// Split partials of the allocation-free entry point.  Each GPU holds its own
// copy of this array at its own address; host code never uses the name as an
// address (it is a host-side stand-in), only the pointer that
// hipGetSymbolAddress returns for the current device.  Every entry is written
// by the split kernel before the merge kernel reads it, so nothing needs
// clearing between calls; calls that overlap on one GPU share the array and
// race.
static __device__ __align__(256) char scratch[kKvScratchBytes];

hipError_t kvcache_scratch(void** ptr) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* addr[kMaxDev] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace fa
