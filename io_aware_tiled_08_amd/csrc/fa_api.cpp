// C ABI of the gfx950 FlashAttention forward library: argument validation,
// device checks and dispatch to the kernels.  The contract of every entry
// point is documented in include/fa_mi355x.h.
#include "fa_mi355x.h"

#include <hip/hip_runtime_api.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fa_bwd.h"
#include "fa_fp8.h"
#include "fa_kvcache.h"
#include "fa_launch.h"

namespace {

thread_local char g_last_error[512] = "";

fa_status fail(fa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

fa_status fail(fa_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return s;
}

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];
char g_arch_name[kMaxDevices][64];
int g_cu_count[kMaxDevices];  // compute units, valid once g_arch_ok[dev] != 0

fa_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0)
    return fail(FA_ERR_NO_DEVICE, "no usable HIP device: %s", hipGetErrorString(e));
  if (dev >= kMaxDevices) return fail(FA_ERR_NO_DEVICE, "device index %d too large", dev);
  int state = g_arch_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(FA_ERR_NO_DEVICE, "hipGetDeviceProperties(%d): %s", dev, hipGetErrorString(e));
    // gcnArchName looks like "gfx950:sramecc+:xnack-".
    std::snprintf(g_arch_name[dev], sizeof(g_arch_name[dev]), "%s", prop.gcnArchName);
    g_cu_count[dev] = prop.multiProcessorCount;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                    (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':')
                ? 1
                : 2;
    g_arch_ok[dev].store(state, std::memory_order_release);
  }
  if (state != 1)
    return fail(FA_ERR_ARCH, "device %d is %s; this library is built for gfx950", dev,
                g_arch_name[dev]);
  return FA_OK;
}

// Split count and 32-key tiles per split for the key/value-cache path:
// enough workgroups to give every CU of the MI355X (256) two of them, while
// every wave keeps at least four tiles to stream; never more splits than
// tiles or kKvMaxSplits.  `requested` > 0 overrides the first goal.
struct KvSplit {
  int n_split;
  int tiles_per_split;
};
KvSplit kv_split(int64_t BH, int64_t Nq, int64_t Nk, int64_t d, int requested) {
  const int64_t tiles = (Nk + fa::kKvKeys - 1) / fa::kKvKeys;
  const int64_t blocks = BH * ((Nq + fa::kKvRows - 1) / fa::kKvRows);
  int64_t S;
  if (requested > 0) {
    S = requested;
  } else {
    const int64_t want = (2 * 256 + blocks - 1) / (blocks > 0 ? blocks : 1);
    const int64_t most = tiles / (4 * fa::kv_waves((int)d));
    S = want < most ? want : most;
  }
  if (S > tiles) S = tiles;
  if (S > fa::kKvMaxSplits) S = fa::kKvMaxSplits;
  if (S < 1) S = 1;
  const int64_t tps = (tiles + S - 1) / S;
  KvSplit r;
  r.tiles_per_split = (int)(tps > 0 ? tps : 1);
  r.n_split = (int)((tiles + r.tiles_per_split - 1) / r.tiles_per_split);
  if (r.n_split < 1) r.n_split = 1;
  return r;
}

int64_t kv_workspace_bytes(int64_t BH, int64_t Nq, int64_t d, int n_split) {
  return n_split > 1 ? (int64_t)n_split * BH * Nq * (d + 1) * 4 : 0;
}

// Argument checks of flash_attn_fwd and flash_attn_fwd_persistent (the latter
// always uses 256-row blocks): FA_OK with *a filled and *empty false when a
// kernel is to be launched, FA_OK with *empty true for an empty problem.
fa_status check_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                        fa_dtype dtype, bool persistent, fa::FwdArgs* a, bool* keysplit,
                        bool* empty) {
  *empty = true;
  if (B < 0 || H < 0 || N < 0)
    return fail(FA_ERR_SHAPE, "B, H, N must be >= 0 (got %lld, %lld, %lld)", (long long)B,
                (long long)H, (long long)N);
  if (d != 64 && d != 128) return fail(FA_ERR_HEAD_DIM, "d must be 64 or 128 (got %lld)", (long long)d);
  if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_DTYPE, "unknown dtype %d", (int)dtype);
  if (persistent && dtype == FA_F32)
    return fail(FA_ERR_DTYPE, "the persistent schedule runs fp16 and bf16 only");
  if (!std::isfinite(scale)) return fail(FA_ERR_SCALE, "scale must be finite");
  // An empty problem reads no pointer (zero-size buffers may be NULL).
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_NULL, "q, k, v, o and lse must be non-NULL");
  const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15u;
  if (mis) return fail(FA_ERR_ALIGN, "q, k, v, o and lse must be 16-byte aligned");

  // Index math uses int64 element offsets and a 32-bit grid.
  const int64_t elem = dtype == FA_F32 ? 4 : 2;
  const int64_t kLimit = (int64_t)1 << 62;
  if (B > kLimit / H || N > kLimit / (B * H) || d * elem > kLimit / (B * H * N))
    return fail(FA_ERR_SHAPE, "B*H*N*d*elem overflows");
  const int64_t BH = B * H;
  *keysplit = !persistent && fa::use_keysplit((fa::Dtype)dtype, (int)d, causal != 0, BH, N);
  const int br = *keysplit ? fa::kRowsPerWorkgroupF16KeySplit : fa::rows_per_workgroup((fa::Dtype)dtype);
  const int64_t n_qblk = (N + br - 1) / br;
  const int64_t tpw = fa::threads_per_workgroup((fa::Dtype)dtype, (int)d);
  if (n_qblk > INT32_MAX || BH * n_qblk > (int64_t)UINT32_MAX / tpw)
    return fail(FA_ERR_SHAPE, "B*H*ceil(N/%d) = %lld workgroups exceeds the grid limit", br,
                (long long)(BH * n_qblk));

  const int64_t tbytes = BH * N * d * elem;
  const int64_t lbytes = BH * N * 4;
  if (overlaps(o, tbytes, q, tbytes) || overlaps(o, tbytes, k, tbytes) ||
      overlaps(o, tbytes, v, tbytes) || overlaps(lse, lbytes, q, tbytes) ||
      overlaps(lse, lbytes, k, tbytes) || overlaps(lse, lbytes, v, tbytes) ||
      overlaps(lse, lbytes, o, tbytes))
    return fail(FA_ERR_ALIAS, "o and lse must not overlap q, k, v or each other");

  a->q = q;
  a->k = k;
  a->v = v;
  a->o = o;
  a->lse = lse;
  a->BH = BH;
  a->N = N;
  a->d = (int)d;
  a->scale = scale;
  a->causal = causal != 0;
  a->dtype = (fa::Dtype)dtype;
  *empty = false;
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status flash_attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                         fa_dtype dtype, void* stream) {
  g_last_error[0] = '\0';
  fa::FwdArgs a;
  bool keysplit = false, empty = true;
  fa_status st = check_forward(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, false, &a,
                               &keysplit, &empty);
  if (st != FA_OK || empty) return st;
  st = check_device();
  if (st != FA_OK) return st;
  int dev = 0;
  (void)hipGetDevice(&dev);  // succeeded inside check_device
  const int cus = g_cu_count[dev];
  (void)hipGetLastError();  // do not report an earlier, unrelated error
  const hipError_t e =
      dtype == FA_F32 ? fa::launch_forward_f32(a, (hipStream_t)stream)
      : keysplit      ? fa::launch_forward_f16_keysplit(a, (hipStream_t)stream)
      : fa::use_stream(a.dtype, a.causal, a.BH, N, cus)
          ? fa::launch_forward_f16_persistent(a, cus, (hipStream_t)stream)
          : fa::launch_forward_f16(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

fa_status flash_attn_fwd_persistent(const void* q, const void* k, const void* v, void* o,
                                    float* lse, int64_t B, int64_t H, int64_t N, int64_t d,
                                    float scale, int causal, int num_workgroups, fa_dtype dtype,
                                    void* stream) {
  g_last_error[0] = '\0';
  if (num_workgroups < 0)
    return fail(FA_ERR_SHAPE, "num_workgroups must be >= 0 (got %d)", num_workgroups);
  fa::FwdArgs a;
  bool keysplit = false, empty = true;
  fa_status st = check_forward(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, true, &a,
                               &keysplit, &empty);
  if (st != FA_OK || empty) return st;
  st = check_device();
  if (st != FA_OK) return st;
  int dev = 0;
  (void)hipGetDevice(&dev);  // succeeded inside check_device
  const int64_t items = a.BH * ((N + fa::kRowsPerWorkgroupF16 - 1) / fa::kRowsPerWorkgroupF16);
  int64_t n_wg = num_workgroups > 0 ? num_workgroups : g_cu_count[dev];
  if (n_wg < 1) n_wg = 1;
  if (n_wg > items) n_wg = items;
  (void)hipGetLastError();
  const hipError_t e = fa::launch_forward_f16_persistent(a, (int)n_wg, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

fa_status flash_attn_fwd_fp8(const void* q, const void* k, const void* v, void* o, float* lse,
                             int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                             float q_descale, float k_descale, float v_descale, void* stream) {
  g_last_error[0] = '\0';
  if (B < 0 || H < 0 || N < 0)
    return fail(FA_ERR_SHAPE, "B, H, N must be >= 0 (got %lld, %lld, %lld)", (long long)B,
                (long long)H, (long long)N);
  if (d != 64 && d != 128) return fail(FA_ERR_HEAD_DIM, "d must be 64 or 128 (got %lld)", (long long)d);
  if (!std::isfinite(scale)) return fail(FA_ERR_SCALE, "scale must be finite");
  if (!(std::isfinite(q_descale) && q_descale > 0.f && std::isfinite(k_descale) &&
        k_descale > 0.f && std::isfinite(v_descale) && v_descale > 0.f))
    return fail(FA_ERR_SCALE, "descale factors must be finite and > 0");
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_NULL, "q, k, v, o and lse must be non-NULL");
  const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15u;
  if (mis) return fail(FA_ERR_ALIGN, "q, k, v, o and lse must be 16-byte aligned");
  const int64_t kLimit = (int64_t)1 << 62;
  if (B > kLimit / H || N > kLimit / (B * H) || d * 2 > kLimit / (B * H * N))
    return fail(FA_ERR_SHAPE, "B*H*N*d*elem overflows");
  const int64_t BH = B * H;
  const int64_t n_qblk = (N + fa::kRowsPerWorkgroupFp8 - 1) / fa::kRowsPerWorkgroupFp8;
  if (n_qblk > INT32_MAX || BH * n_qblk > (int64_t)UINT32_MAX / 512)
    return fail(FA_ERR_SHAPE, "B*H*ceil(N/%d) = %lld workgroups exceeds the grid limit",
                fa::kRowsPerWorkgroupFp8, (long long)(BH * n_qblk));
  const int64_t ibytes = BH * N * d;      // e4m3 inputs
  const int64_t obytes = BH * N * d * 2;  // bf16 output
  const int64_t lbytes = BH * N * 4;
  if (overlaps(o, obytes, q, ibytes) || overlaps(o, obytes, k, ibytes) ||
      overlaps(o, obytes, v, ibytes) || overlaps(lse, lbytes, q, ibytes) ||
      overlaps(lse, lbytes, k, ibytes) || overlaps(lse, lbytes, v, ibytes) ||
      overlaps(lse, lbytes, o, obytes))
    return fail(FA_ERR_ALIAS, "o and lse must not overlap q, k, v or each other");

  fa_status st = check_device();
  if (st != FA_OK) return st;

  fa::Fp8Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = BH;
  a.N = N;
  a.d = (int)d;
  a.scale = scale;
  a.causal = causal != 0;
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  (void)hipGetLastError();
  const hipError_t e = fa::launch_forward_fp8(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

int64_t flash_attn_bwd_workspace_size(int64_t B, int64_t H, int64_t N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  if (B > ((int64_t)1 << 40) / H || N > ((int64_t)1 << 40) / (B * H)) return -1;
  return B * H * N * 8;
}

fa_status flash_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         int64_t B, int64_t H, int64_t N, int64_t d, float scale, int causal,
                         void* workspace, int64_t workspace_bytes, fa_dtype dtype, void* stream) {
  g_last_error[0] = '\0';
  if (B < 0 || H < 0 || N < 0)
    return fail(FA_ERR_SHAPE, "B, H, N must be >= 0 (got %lld, %lld, %lld)", (long long)B,
                (long long)H, (long long)N);
  if (d != 64 && d != 128) return fail(FA_ERR_HEAD_DIM, "d must be 64 or 128 (got %lld)", (long long)d);
  if (dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_DTYPE, "the backward pass takes FA_F16 or FA_BF16 (got %d)", (int)dtype);
  if (!std::isfinite(scale)) return fail(FA_ERR_SCALE, "scale must be finite");
  if (B == 0 || H == 0 || N == 0) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv)
    return fail(FA_ERR_NULL, "q, k, v, o, dout, lse, dq, dk and dv must be non-NULL");
  const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o |
                         (uintptr_t)dout | (uintptr_t)lse | (uintptr_t)dq | (uintptr_t)dk |
                         (uintptr_t)dv) & 15u;
  if (mis) return fail(FA_ERR_ALIGN, "all tensors must be 16-byte aligned");
  const int64_t kLimit = (int64_t)1 << 62;
  if (B > kLimit / H || N > kLimit / (B * H) || d * 2 > kLimit / (B * H * N))
    return fail(FA_ERR_SHAPE, "B*H*N*d*elem overflows");
  const int64_t BH = B * H;
  const int64_t n_blk = (N + fa::kBwdRowsPerWorkgroup - 1) / fa::kBwdRowsPerWorkgroup;
  if (n_blk > INT32_MAX || BH * n_blk > (int64_t)UINT32_MAX / fa::kBwdThreads ||
      BH * N > (int64_t)UINT32_MAX / 16)
    return fail(FA_ERR_SHAPE, "B*H*ceil(N/%d) = %lld workgroups exceeds the grid limit",
                fa::kBwdRowsPerWorkgroup, (long long)(BH * n_blk));
  // D and LSE * log2(e) for every row (flash_attn_bwd_workspace_size): the
  // prep kernel writes both halves, so the whole size is required and the
  // whole range takes part in the overlap checks.
  const int64_t need = flash_attn_bwd_workspace_size(B, H, N);
  if (need <= 0) return fail(FA_ERR_SHAPE, "B*H*N overflows the workspace size");
  if (!workspace) return fail(FA_ERR_WORKSPACE, "the backward pass needs a workspace of %lld bytes", (long long)need);
  if ((uintptr_t)workspace & 15u) return fail(FA_ERR_ALIGN, "workspace must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(FA_ERR_WORKSPACE, "workspace has %lld bytes, the backward pass needs %lld",
                (long long)workspace_bytes, (long long)need);
  const int64_t tb = BH * N * d * 2, lb = BH * N * 4;
  const void* ins[6] = {q, k, v, o, dout, lse};
  const int64_t in_bytes[6] = {tb, tb, tb, tb, tb, lb};
  void* outs[4] = {dq, dk, dv, workspace};
  const int64_t out_bytes[4] = {tb, tb, tb, need};
  for (int i = 0; i < 4; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps(outs[i], out_bytes[i], ins[j], in_bytes[j]))
        return fail(FA_ERR_ALIAS, "dq, dk, dv and the workspace must not overlap an input");
    for (int j = i + 1; j < 4; ++j)
      if (overlaps(outs[i], out_bytes[i], outs[j], out_bytes[j]))
        return fail(FA_ERR_ALIAS, "dq, dk, dv and the workspace must not overlap each other");
  }

  fa_status st = check_device();
  if (st != FA_OK) return st;

  fa::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.workspace = workspace;
  a.BH = BH;
  a.N = N;
  a.d = (int)d;
  a.scale = scale;
  a.causal = causal != 0;
  a.dtype = (fa::Dtype)dtype;
  (void)hipGetLastError();
  const hipError_t e = fa::launch_backward(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

int flash_attn_kvcache_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                              int num_splits) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || (d != 64 && d != 128)) return 1;
  if (B > ((int64_t)1 << 40) / H) return 1;
  return kv_split(B * H, Nq, Nk, d, num_splits).n_split;
}

int64_t flash_attn_kvcache_workspace_size(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                          int64_t d, int num_splits) {
  if (B <= 0 || H <= 0 || Nq <= 0 || Nk <= 0 || (d != 64 && d != 128)) return 0;
  if (B > ((int64_t)1 << 40) / H || Nq > ((int64_t)1 << 40) / (B * H)) return -1;
  const int S = kv_split(B * H, Nq, Nk, d, num_splits).n_split;
  return kv_workspace_bytes(B * H, Nq, d, S);
}

namespace {

// Argument checks shared by the two cache entry points, in the order both
// document (everything before any HIP call).  FA_OK with *empty true for an
// empty problem; otherwise *a is filled except for the workspace, and *need
// is the scratch the chosen key splits take (0 for one split).
fa_status check_kvcache(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale,
                        int causal, int num_splits, fa_dtype dtype, fa::KvArgs* a,
                        int64_t* need, bool* empty) {
  *empty = false;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(FA_ERR_SHAPE, "B, H, Nq, Nk must be >= 0 (got %lld, %lld, %lld, %lld)",
                (long long)B, (long long)H, (long long)Nq, (long long)Nk);
  if (d != 64 && d != 128) return fail(FA_ERR_HEAD_DIM, "d must be 64 or 128 (got %lld)", (long long)d);
  if (dtype != FA_F16 && dtype != FA_BF16)
    return fail(FA_ERR_DTYPE, "the key/value-cache path takes FA_F16 or FA_BF16 (got %d)", (int)dtype);
  if (!std::isfinite(scale)) return fail(FA_ERR_SCALE, "scale must be finite");
  if (B == 0 || H == 0 || Nq == 0) {
    *empty = true;
    return FA_OK;
  }
  if (Nk == 0) return fail(FA_ERR_SHAPE, "Nk = 0: the queries see no key");
  if (causal && Nk < Nq)
    return fail(FA_ERR_SHAPE, "causal queries are the last Nq of Nk positions: need Nk >= Nq "
                "(got Nq = %lld, Nk = %lld)", (long long)Nq, (long long)Nk);
  if (!q || !k || !v || !o || !lse) return fail(FA_ERR_NULL, "q, k, v, o and lse must be non-NULL");
  const uintptr_t mis = ((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)lse) & 15u;
  if (mis) return fail(FA_ERR_ALIGN, "q, k, v, o and lse must be 16-byte aligned");

  const int64_t elem = 2;
  const int64_t kLimit = (int64_t)1 << 62;
  const int64_t nmax = Nq > Nk ? Nq : Nk;
  if (B > kLimit / H || nmax > kLimit / (B * H) || (d + 1) * elem * 2 > kLimit / (B * H * nmax))
    return fail(FA_ERR_SHAPE, "B*H*N*d*elem overflows");
  const int64_t BH = B * H;
  const KvSplit sp = kv_split(BH, Nq, Nk, d, num_splits);
  const int64_t nqb = (Nq + fa::kKvRows - 1) / fa::kKvRows;
  const int64_t kv_tpw = fa::kv_waves((int)d) * 64;
  if (BH * nqb > (int64_t)UINT32_MAX / kv_tpw / sp.n_split ||
      (sp.n_split > 1 && BH * Nq > (int64_t)UINT32_MAX / 256))
    return fail(FA_ERR_SHAPE, "B*H*ceil(Nq/%d)*splits = %lld workgroups exceeds the grid limit",
                fa::kKvRows, (long long)(BH * nqb * sp.n_split));
  *need = kv_workspace_bytes(BH, Nq, d, sp.n_split);

  const int64_t qbytes = BH * Nq * d * elem;
  const int64_t kbytes = BH * Nk * d * elem;
  const int64_t lbytes = BH * Nq * 4;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kbytes) ||
      overlaps(o, qbytes, v, kbytes) || overlaps(lse, lbytes, q, qbytes) ||
      overlaps(lse, lbytes, k, kbytes) || overlaps(lse, lbytes, v, kbytes) ||
      overlaps(lse, lbytes, o, qbytes))
    return fail(FA_ERR_ALIAS, "o and lse must not overlap q, k, v or each other");

  a->q = q;
  a->k = k;
  a->v = v;
  a->o = o;
  a->lse = lse;
  a->workspace = nullptr;
  a->BH = BH;
  a->Nq = Nq;
  a->Nk = Nk;
  a->d = (int)d;
  a->scale = scale;
  a->causal = causal != 0;
  a->dtype = (fa::Dtype)dtype;
  a->n_split = sp.n_split;
  a->tiles_per_split = sp.tiles_per_split;
  return FA_OK;
}

fa_status launch_kvcache_checked(const fa::KvArgs& a, void* stream) {
  (void)hipGetLastError();
  const hipError_t e = fa::launch_kvcache(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(FA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return FA_OK;
}

}  // namespace

fa_status flash_attn_fwd_kvcache(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                 int64_t d, float scale, int causal, int num_splits,
                                 void* workspace, int64_t workspace_bytes, fa_dtype dtype,
                                 void* stream) {
  g_last_error[0] = '\0';
  fa::KvArgs a;
  int64_t need = 0;
  bool empty = false;
  fa_status st = check_kvcache(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, num_splits,
                               dtype, &a, &need, &empty);
  if (st != FA_OK || empty) return st;
  if (need > 0) {
    if (!workspace)
      return fail(FA_ERR_WORKSPACE, "%d key splits need a workspace of %lld bytes", a.n_split,
                  (long long)need);
    if ((uintptr_t)workspace & 15u) return fail(FA_ERR_ALIGN, "workspace must be 16-byte aligned");
    if (workspace_bytes < need)
      return fail(FA_ERR_WORKSPACE, "workspace has %lld bytes, %d key splits need %lld",
                  (long long)workspace_bytes, a.n_split, (long long)need);
    const int64_t qbytes = a.BH * Nq * d * 2, kbytes = a.BH * Nk * d * 2, lbytes = a.BH * Nq * 4;
    if (overlaps(workspace, need, q, qbytes) || overlaps(workspace, need, k, kbytes) ||
        overlaps(workspace, need, v, kbytes) || overlaps(workspace, need, o, qbytes) ||
        overlaps(workspace, need, lse, lbytes))
      return fail(FA_ERR_ALIAS, "the workspace must not overlap q, k, v, o or lse");
    a.workspace = workspace;
  }
  st = check_device();
  if (st != FA_OK) return st;
  return launch_kvcache_checked(a, stream);
}

fa_status flash_attn_fwd_kvcache_noalloc(const void* q, const void* k, const void* v, void* o,
                                         float* lse, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                         int64_t d, float scale, int causal, int num_splits,
                                         fa_dtype dtype, void* stream) {
  g_last_error[0] = '\0';
  fa::KvArgs a;
  int64_t need = 0;
  bool empty = false;
  fa_status st = check_kvcache(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, num_splits,
                               dtype, &a, &need, &empty);
  if (st != FA_OK || empty) return st;
  if (need > fa::kKvScratchBytes)
    return fail(FA_ERR_WORKSPACE,
                "%d key splits need %lld bytes of scratch; the library's scratch holds %lld "
                "(fewer splits, or flash_attn_fwd_kvcache with a workspace)",
                a.n_split, (long long)need, (long long)fa::kKvScratchBytes);
  st = check_device();
  if (st != FA_OK) return st;
  if (need > 0) {
    const hipError_t e = fa::kvcache_scratch(&a.workspace);
    if (e != hipSuccess)
      return fail(FA_ERR_HIP, "scratch address lookup failed: %s", hipGetErrorString(e));
  }
  return launch_kvcache_checked(a, stream);
}

const char* flash_attn_status_str(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_NULL: return "FA_ERR_NULL: a required pointer is NULL";
    case FA_ERR_SHAPE: return "FA_ERR_SHAPE: invalid B, H or N";
    case FA_ERR_HEAD_DIM: return "FA_ERR_HEAD_DIM: unsupported head dimension";
    case FA_ERR_DTYPE: return "FA_ERR_DTYPE: unknown dtype";
    case FA_ERR_ALIGN: return "FA_ERR_ALIGN: pointer not 16-byte aligned";
    case FA_ERR_SCALE: return "FA_ERR_SCALE: scale is not finite";
    case FA_ERR_ALIAS: return "FA_ERR_ALIAS: output overlaps an input";
    case FA_ERR_NO_DEVICE: return "FA_ERR_NO_DEVICE: no usable HIP device";
    case FA_ERR_ARCH: return "FA_ERR_ARCH: device is not gfx950";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: workspace missing or too small";
  }
  return "unknown fa_status";
}

const char* flash_attn_last_error(void) { return g_last_error; }

int flash_attn_abi_version(void) { return FA_MI355X_ABI_VERSION; }

}  // extern "C"
