/*
 * fa_mi355x.h -- C ABI of the MI355X (gfx950) FlashAttention forward library.
 *
 * The library computes exact attention, O = softmax(scale * Q K^T) V, together
 * with the natural-log log-sum-exp of every score row, in one fused HIP kernel
 * that walks K and V tile by tile with an online softmax (running row maximum
 * and running sum, accumulator rescaled when the maximum grows), so the N x N
 * score matrix is never written to HBM.  Sources: "FlashAttention" (Chapter 15,
 * vizuara), sections "Standard vs Flash Attention" (the four steps: load tiles,
 * tile scores, online softmax, accumulate O and write it once) and "The Tiling
 * Strategy"; "FlashAttention, Playable", EP 03 (tiling) and EP 04 (online
 * softmax); "FlashAttention: Tiled & Fused", hero diagram (O written once,
 * running statistics kept on chip).
 *
 * Conventions shared by every entry point
 *   - All functions are extern "C", never throw, and report errors through
 *     fa_status.  No entry point allocates device memory or keeps a pointer
 *     after it returns; scratch memory, where a path needs it, is passed in.
 *   - Argument checks run before any HIP runtime call, so a host without a
 *     GPU can exercise every error path.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FA_MI355X_ABI_VERSION 7

typedef enum {
  FA_F32 = 0,   /* IEEE binary32 */
  FA_F16 = 1,   /* IEEE binary16 */
  FA_BF16 = 2   /* bfloat16 */
} fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,       /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,      /* B, H or N negative, or an index would overflow */
  FA_ERR_HEAD_DIM = 3,   /* d is not a supported head dimension (64, 128) */
  FA_ERR_DTYPE = 4,      /* dtype is not an fa_dtype value */
  FA_ERR_ALIGN = 5,      /* a pointer is not 16-byte aligned */
  FA_ERR_SCALE = 6,      /* scale is NaN or infinite */
  FA_ERR_ALIAS = 7,      /* o or lse overlaps an input or each other */
  FA_ERR_NO_DEVICE = 8,  /* no HIP device is usable */
  FA_ERR_ARCH = 9,       /* the current device is not gfx950 */
  FA_ERR_HIP = 10,       /* the HIP runtime reported an error (see last_error) */
  FA_ERR_WORKSPACE = 11  /* a needed workspace is NULL or smaller than required */
} fa_status;

/*
 * flash_attn_fwd -- exact attention forward pass for every (batch, head).
 *
 * For each b < B, h < H and query row i < N:
 *   s_ij   = scale * sum_c q[b,h,i,c] * k[b,h,j,c]      for visible keys j
 *   o[b,h,i,:] = sum_j softmax_j(s_ij) * v[b,h,j,:]
 *   lse[b,h,i] = ln(sum_j exp(s_ij))
 * Visible keys are j < N, and with causal != 0 only j <= i (lower-triangular
 * mask, diagonal included; the pages do not treat masking, so this is the
 * plain reading of a causal mask).
 *
 * Arguments
 *   q, k, v  device pointers, read only, contiguous row-major [B, H, N, d]
 *            arrays of `dtype` (element [b,h,n,c] at ((b*H + h)*N + n)*d + c).
 *   o        device pointer, contiguous [B, H, N, d] of `dtype`; fully
 *            overwritten (rounded to nearest even from fp32).
 *   lse      device pointer, contiguous [B, H, N] float32; fully overwritten.
 *   B, H, N  batch, heads and sequence length, each >= 0.  If any is 0 the
 *            call returns FA_OK once d, dtype and scale are checked, without
 *            looking at any pointer (they may be NULL) or touching the device.
 *   d        head dimension: 64 or 128.
 *   scale    finite float multiplying Q K^T (usually 1/sqrt(d)); negative and
 *            zero values are allowed.
 *   causal   0 = every key visible, nonzero = lower-triangular mask.
 *   dtype    element type of q, k, v and o.  FA_F16 and FA_BF16 run both
 *            products on MFMA with fp32 accumulation and round the softmax
 *            weights to `dtype` before the second product; FA_F32 keeps every
 *            step in fp32.
 *   stream   hipStream_t to enqueue on, passed as void*; NULL is the null
 *            stream of the current device.
 *
 * Ownership and synchronisation: the caller owns all five buffers, which must
 * live on the current HIP device and be 16-byte aligned.  o and lse must not
 * overlap each other or q, k, v.  The call enqueues one kernel and returns
 * without synchronising; results are valid once `stream` has completed.  It is
 * reentrant and keeps no state between calls apart from a per-device cache of
 * the architecture check and a thread-local error string.
 *
 * Errors: argument errors are returned before any HIP call (FA_ERR_NULL,
 * FA_ERR_SHAPE, FA_ERR_HEAD_DIM, FA_ERR_DTYPE, FA_ERR_ALIGN, FA_ERR_SCALE,
 * FA_ERR_ALIAS).  Then FA_ERR_NO_DEVICE or FA_ERR_ARCH if the current device
 * cannot run the gfx950 kernel, and FA_ERR_HIP if the launch fails; the HIP
 * error text is then available from flash_attn_last_error().  Nothing is
 * enqueued when an error is returned.
 */
fa_status flash_attn_fwd(const void* q, const void* k, const void* v,
                         void* o, float* lse,
                         int64_t B, int64_t H, int64_t N, int64_t d,
                         float scale, int causal,
                         fa_dtype dtype, void* stream);

/*
 * flash_attn_fwd_persistent -- flash_attn_fwd's computation (fp16 and bf16)
 * under a persistent schedule.
 *
 * Source: "FlashAttention" (Chapter 15, vizuara), "FlashAttention Evolution",
 * FA-4 card (persistent kernels); the computation is flash_attn_fwd's (same
 * pages).  Instead of one workgroup per 256-row query block, a fixed grid of
 * num_workgroups workgroups stays resident and each loops over the blocks:
 * causal blocks longest first, dealt to the workgroups in a snake order
 * (workgroup g takes block r*G + g in even rounds and r*G + G-1-g in odd
 * ones, G the grid size); unmasked blocks head-major, a contiguous range of
 * them per XCD and round, and a workgroup runs its unmasked blocks back to
 * back as one stream of key tiles (the next block's Q is loaded and the
 * finished block's O stored while tiles are in flight).  Each block is
 * computed exactly as flash_attn_fwd's 256-row kernel computes it, so o and
 * lse are bitwise equal to that kernel's (flash_attn_fwd itself takes another
 * schedule for causal d = 64 problems with few blocks, whose rounding can
 * differ in the last bit).  flash_attn_fwd uses this schedule, with one
 * workgroup per compute unit, for unmasked fp16 / bf16 problems with at least
 * two blocks per compute unit.
 *
 * Arguments as for flash_attn_fwd, plus
 *   num_workgroups  resident workgroups; 0 = one per compute unit of the
 *                   current device.  Clamped to the number of blocks,
 *                   B * H * ceil(N / 256).
 * dtype must be FA_F16 or FA_BF16 (FA_F32 returns FA_ERR_DTYPE).
 *
 * Errors as for flash_attn_fwd, plus FA_ERR_SHAPE for num_workgroups < 0.
 */
fa_status flash_attn_fwd_persistent(const void* q, const void* k, const void* v,
                                    void* o, float* lse,
                                    int64_t B, int64_t H, int64_t N, int64_t d,
                                    float scale, int causal, int num_workgroups,
                                    fa_dtype dtype, void* stream);

/*
 * flash_attn_fwd_kvcache -- attention of Nq new queries against a key/value
 * cache of Nk rows (decode), fp16 or bf16.
 *
 * Source: "FlashAttention: Tiled & Fused", related-diagram card "KV Cache: Why
 * Generation Speeds Up" (generation stores and reuses the keys and values of
 * earlier tokens) for the operation; the computation is the one of
 * flash_attn_fwd (same pages).  Reading where the pages are silent:
 * the Nq queries are the last Nq positions of the sequence whose Nk keys are
 * cached, so with causal != 0 query i sees the keys j <= i + (Nk - Nq); with
 * Nq == Nk that is flash_attn_fwd's mask.
 *
 * For each b < B, h < H and query row i < Nq:
 *   s_ij   = scale * sum_c q[b,h,i,c] * k[b,h,j,c]      for visible keys j < Nk
 *   o[b,h,i,:] = sum_j softmax_j(s_ij) * v[b,h,j,:]
 *   lse[b,h,i] = ln(sum_j exp(s_ij))
 *
 * Arguments
 *   q        device pointer, read only, contiguous [B, H, Nq, d] of `dtype`.
 *   k, v     device pointers, read only, contiguous [B, H, Nk, d] of `dtype`.
 *   o        device pointer, contiguous [B, H, Nq, d] of `dtype`; overwritten.
 *   lse      device pointer, contiguous [B, H, Nq] float32; overwritten.
 *   B, H, Nq, Nk  each >= 0; nothing is done when B, H or Nq is 0.  Nk must be
 *            >= 1, and >= Nq when causal.
 *   d        64 or 128.
 *   scale, causal  as for flash_attn_fwd.
 *   num_splits  number of key ranges computed by separate workgroups and then
 *            merged (each range's normalised output weighted by exp(its LSE -
 *            the largest LSE), the online-softmax rescale rule); <= 0 lets the
 *            library choose.  The count actually used is
 *            flash_attn_kvcache_splits(B, H, Nq, Nk, d, num_splits).
 *   workspace, workspace_bytes  device scratch owned by the caller, 16-byte
 *            aligned, at least flash_attn_kvcache_workspace_size(B, H, Nq, Nk,
 *            d, num_splits) bytes (0 when one split is used: then workspace
 *            may be NULL).  Its contents on entry do not matter; on return it
 *            holds partial results the caller may discard.  Calls that share
 *            a workspace must be ordered on one stream.
 *   dtype    FA_F16 or FA_BF16 (FA_F32 returns FA_ERR_DTYPE).
 *   stream   as for flash_attn_fwd.
 *
 * Enqueues one kernel (one split) or two (the ranges, then their merge) and
 * returns without synchronising.  o, lse and the workspace must not overlap
 * each other or q, k, v (FA_ERR_ALIAS).  Errors as for flash_attn_fwd, plus
 * FA_ERR_WORKSPACE when the workspace is NULL or too small.
 */
fa_status flash_attn_fwd_kvcache(const void* q, const void* k, const void* v,
                                 void* o, float* lse,
                                 int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                                 int64_t d, float scale, int causal,
                                 int num_splits, void* workspace,
                                 int64_t workspace_bytes,
                                 fa_dtype dtype, void* stream);

/* Bytes of device scratch the library holds on each GPU it runs on, for
 * flash_attn_fwd_kvcache_noalloc (held from its first call on that GPU
 * until the process ends). */
#define FA_MI355X_KVCACHE_SCRATCH_BYTES (16 * 1024 * 1024)

/*
 * flash_attn_fwd_kvcache_noalloc -- flash_attn_fwd_kvcache without a
 * workspace argument and without any allocation.
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * computation, arguments (less workspace and workspace_bytes), kernels,
 * key-split choice and results as flash_attn_fwd_kvcache: bit for bit equal
 * for the same num_splits.  The split partials go to a static device array of
 * the library (FA_MI355X_KVCACHE_SCRATCH_BYTES per GPU) instead of a caller's
 * workspace; its address on the current device is looked up once
 * (hipGetSymbolAddress) on the first call that needs it.  The call never
 * calls hipMalloc, hipFree or any allocating routine.
 *
 * Returns FA_ERR_WORKSPACE, before any HIP call, when the chosen splits need
 * more than FA_MI355X_KVCACHE_SCRATCH_BYTES
 * (flash_attn_kvcache_workspace_size() tells the size; pass fewer num_splits
 * or use flash_attn_fwd_kvcache).  Every call on one GPU shares that GPU's
 * array: calls that may overlap in time on one GPU (different streams, or
 * different host threads) race and give wrong results; order them on one
 * stream.  The stream must belong to the current device.  Other errors as for
 * flash_attn_fwd_kvcache.
 */
fa_status flash_attn_fwd_kvcache_noalloc(const void* q, const void* k,
                                         const void* v, void* o, float* lse,
                                         int64_t B, int64_t H, int64_t Nq,
                                         int64_t Nk, int64_t d, float scale,
                                         int causal, int num_splits,
                                         fa_dtype dtype, void* stream);

/*
 * flash_attn_fwd_fp8 -- the forward pass of flash_attn_fwd on 8-bit inputs.
 *
 * Source: "FlashAttention" (Chapter 15, vizuara), "FlashAttention Evolution"
 * (the later versions add FP8 support); the computation is flash_attn_fwd's.
 * Inputs are e4m3 codes (OCP "fn" variant: 1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits, no infinities, 0x7F/0xFF NaN) with one descale factor
 * per tensor: the value of element x of q is code(x) * q_descale, likewise for
 * k and v.  For each b, h and query row i < N:
 *   s_ij   = scale * sum_c qval[b,h,i,c] * kval[b,h,j,c]   for visible keys j
 *   o[b,h,i,:] = sum_j softmax_j(s_ij) * vval[b,h,j,:]      (bfloat16)
 *   lse[b,h,i] = ln(sum_j exp(s_ij))                          (float32)
 * with flash_attn_fwd's causal mask.  Both products run on the 8-bit matrix
 * unit; the softmax weights are rounded to e4m3 before the second product,
 * and the row sum adds the rounded weights.  Accuracy contract: per element,
 * |o - exact| <= sum_j max(w_j/16, 2^-10) |v_j - o_exact| / (sum_j w_j - sum_j
 * max(w_j/16, 2^-10)) (w_j = exp(s_ij - max_j s_ij)) plus the bfloat16
 * rounding of o; per row, |lse - exact| <= -ln(1 - that sum of terms / sum w).
 *
 * Arguments: q, k, v device pointers to contiguous [B, H, N, d] byte arrays;
 * o a contiguous [B, H, N, d] bfloat16 array; lse [B, H, N] float32; B, H,
 * N, d, scale, causal and stream as for flash_attn_fwd; q_descale,
 * k_descale, v_descale finite and > 0 (else FA_ERR_SCALE).  Same ownership,
 * alignment, overlap rules, synchronisation and errors as flash_attn_fwd.
 */
fa_status flash_attn_fwd_fp8(const void* q, const void* k, const void* v,
                             void* o, float* lse,
                             int64_t B, int64_t H, int64_t N, int64_t d,
                             float scale, int causal,
                             float q_descale, float k_descale, float v_descale,
                             void* stream);

/*
 * flash_attn_bwd -- gradients of flash_attn_fwd with respect to q, k and v.
 *
 * Source: the pages imply training ("FlashAttention: Tiled & Fused") without
 * giving the backward pass; it is the chain rule through flash_attn_fwd's
 * definition ("FlashAttention", Chapter 15, "Standard vs Flash Attention"),
 * tiled in the same way (the N x N matrices are recomputed tile by tile from
 * q, k and the saved lse, never stored).  With P = exp(s - lse) the forward's
 * softmax and do the gradient of the loss with respect to o:
 *   dv = P^T do,  dP = do v^T,  D_i = sum_c do[i,c] o[i,c],
 *   dS = P * (dP - D),  dq = scale * dS k,  dk = scale * dS^T q.
 *
 * Arguments: q, k, v, o, dout (do) device pointers to contiguous [B, H, N, d]
 * arrays of `dtype` (FA_F16 or FA_BF16), o and lse as flash_attn_fwd wrote
 * them (same scale and causal); dq, dk, dv contiguous [B, H, N, d] of
 * `dtype`, fully overwritten; workspace: device scratch owned by the caller,
 * 16-byte aligned, at least flash_attn_bwd_workspace_size(B, H, N) bytes (it
 * receives D and lse * log2(e) per row; its contents on entry do not
 * matter).  B, H, N, d, scale,
 * causal, stream as for flash_attn_fwd.  P and dS are rounded to `dtype`
 * before the products that use them (accuracy contract: the per-element
 * bound derived from those roundings and from o's).  Enqueues three kernels
 * and returns without synchronising; dq, dk, dv and the workspace must not
 * overlap the inputs or each other.  Errors as for flash_attn_fwd, plus
 * FA_ERR_WORKSPACE.
 */
fa_status flash_attn_bwd(const void* q, const void* k, const void* v,
                         const void* o, const void* dout, const float* lse,
                         void* dq, void* dk, void* dv,
                         int64_t B, int64_t H, int64_t N, int64_t d,
                         float scale, int causal,
                         void* workspace, int64_t workspace_bytes,
                         fa_dtype dtype, void* stream);

/* Workspace bytes flash_attn_bwd needs: B * H * N * 8 (0 for empty sizes, -1
 * if that overflows).  No HIP call. */
int64_t flash_attn_bwd_workspace_size(int64_t B, int64_t H, int64_t N);

/* Key ranges flash_attn_fwd_kvcache uses for these sizes and num_splits (1
 * for empty or invalid sizes).  No HIP call. */
int flash_attn_kvcache_splits(int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                              int64_t d, int num_splits);

/* Workspace bytes flash_attn_fwd_kvcache needs for these sizes and
 * num_splits: splits * B * H * Nq * (d + 1) * 4 when more than one split is
 * used, else 0; -1 if that size overflows.  No HIP call. */
int64_t flash_attn_kvcache_workspace_size(int64_t B, int64_t H, int64_t Nq,
                                          int64_t Nk, int64_t d,
                                          int num_splits);

/* Static, never-NULL description of a status code. */
const char* flash_attn_status_str(fa_status status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* flash_attn_last_error(void);

/* FA_MI355X_ABI_VERSION of the loaded library. */
int flash_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
