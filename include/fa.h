/*
 * fa.h -- C ABI of the MI355X (gfx950) exact-attention library, libfa.so.
 *
 * The operation. For every batch b, head h and query row i,
 *
 *     s_ij  = scale * <q_i, k_j>                    for j in J_i
 *     O_i   = sum_j softmax_j(s_i.) * v_j
 *     LSE_i = ln sum_{j in J_i} exp(s_ij)
 *
 * with J_i = {0..N-1}, or {0..i} when causal (top-left aligned, diagonal
 * kept). This is attention as a score product, a row softmax and a weighted
 * sum of value rows ("FlashAttention explainer" (aitangshan.cn), section 1;
 * "YOLO11 attention swapped for a FlashAttention-2-style implementation"
 * (discosf.com), sections 1.2 and 3.2), with the mask of future positions of
 * "FlashAttention explainer" section 7.1 and the per-row log-sum-exp that the
 * fused call of "YOLO models integrating Flash Attention" (rkmt.cn) returns.
 * The kernels compute it FlashAttention-2 style: Q tiled one block per
 * workgroup, K/V streamed in tiles, an online softmax with a running max and
 * sum, and only O and LSE written to HBM ("FlashAttention explainer"
 * sections 4.1-4.3 and 5.2).
 *
 * Conventions shared by every entry point:
 *  - Pointers named q, k, v, o, lse, do_, dq, dk, dv, cu_seqlens are DEVICE
 *    pointers. The caller allocates and owns every buffer; the library
 *    allocates nothing on any call and keeps no state beyond a per-device
 *    cache of device properties. Calls are thread-safe.
 *  - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *    the default stream). Kernel faults surface at the caller's next
 *    synchronisation, not as a return code.
 *  - Q/K/V/O elements are 16-bit floats of type `dtype` (fa_dtype); LSE is
 *    fp32, natural logarithm. Accumulation is fp32.
 *  - Every argument error is detected on the host BEFORE any HIP call and
 *    returned as a negative fa_status; nothing is enqueued then. A size of
 *    zero in B, H or N is a successful no-op (pointers may then be NULL).
 *  - Supported head dims d: 64, 96, 128, 256. Data pointers must be 16-byte
 *    aligned, LSE 4-byte aligned. Outputs must not overlap inputs.
 *  - Non-finite inputs are not checked; they propagate as NaN/Inf.
 */
#ifndef FA_H
#define FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = -1,        /* a required pointer is NULL                        */
  FA_ERR_DIM = -2,         /* negative size, or a size/stride product overflows */
  FA_ERR_UNSUPPORTED = -3, /* head dim or dtype not supported                   */
  FA_ERR_SCALE = -4,       /* scale is NaN or infinite                          */
  FA_ERR_ALIGN = -5,       /* pointer or row stride not 16-byte aligned         */
  FA_ERR_LAUNCH = -6,      /* the HIP launch itself failed                      */
  FA_ERR_ALIAS = -7,       /* an output overlaps an input, the other output or itself */
  FA_ERR_DEVICE = -8,      /* no usable gfx950 device is current                */
  FA_ERR_TOO_LARGE = -9    /* the problem exceeds fa_bwd_noalloc's static scratch */
} fa_status;

/*
 * fa_fwd -- attention forward on contiguous [B, H, N, d] tensors.
 *
 *   q, k, v : [B, H, N, d] row-major, dtype           (read)
 *   o       : [B, H, N, d] row-major, dtype           (written; fully overwritten)
 *   lse     : [B, H, N] fp32, natural log             (written; fully overwritten)
 *   scale   : multiplies q.k before the softmax; any finite value (0 gives
 *             uniform weights). The Python binding's default is 1/sqrt(d).
 *   causal  : nonzero keeps only keys j <= i.
 *
 * Returns FA_OK or a negative fa_status.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int N, int d, float scale, int causal,
           int dtype, void *stream);

/*
 * fa_fwd_strided -- the same forward with explicit element strides, for the
 * [B, N, H, d] layout and for a packed QKV tensor [B, N, 3, H, d] (pass
 * q = qkv, k = qkv + H*d, v = qkv + 2*H*d with row stride 3*H*d). These are
 * the layouts the pages' wrappers take ("YOLO models integrating Flash
 * Attention" and "Why the official YOLOv12 image is fast" (pwwt.cn),
 * section 5: packed-QKV calls; "YOLO11 ... FlashAttention-2" section 3.2:
 * batch, length, heads, head-dim inputs).
 *
 *   *_sb, *_sh, *_sr : strides in ELEMENTS of the batch, head and row axes of
 *                      q, k, v and o; the head-dim axis is contiguous. Row
 *                      and head strides must be multiples of 8 elements;
 *                      row strides at most 2^24 elements (FA_ERR_DIM beyond).
 *   lse     : [B, H, N] fp32 contiguous.
 * The address ranges of o and lse (from the base pointer to the last element
 * the strides reach) must not meet those of q, k or v, nor each other, and no
 * two rows of o may share an element (with o's axes of extent above 1 sorted
 * by stride, each stride must reach past what the smaller axes span; a row
 * spans d elements): FA_ERR_ALIAS otherwise. q, k and v may share memory, as
 * in a packed QKV tensor.
 */
int fa_fwd_strided(const void *q, const void *k, const void *v, void *o, float *lse,
                   int B, int H, int N, int d, float scale, int causal, int dtype,
                   int64_t q_sb, int64_t q_sh, int64_t q_sr,
                   int64_t k_sb, int64_t k_sh, int64_t k_sr,
                   int64_t v_sb, int64_t v_sh, int64_t v_sr,
                   int64_t o_sb, int64_t o_sh, int64_t o_sr,
                   void *stream);

/*
 * fa_fwd_varlen -- forward over a packed batch of variable-length sequences
 * (the cu_seqlens / max_seqlen form of the varlen flash call shown in "Why the
 * official YOLOv12 image is fast", section 5).
 *
 *   q, k, v, o : [T, H, d] row-major (T = total tokens), dtype
 *   cu_seqlens : int32 [B+1] on the device, cu[0] = 0, non-decreasing,
 *                cu[B] = T; sequence b owns rows cu[b] .. cu[b+1]-1.
 *                Its contents are NOT validated (they are on the device):
 *                a wrong table reads or writes out of bounds.
 *   max_seqlen : an upper bound of cu[b+1]-cu[b] over b (sizes the grid).
 *   lse        : [H, T] fp32.
 * Attention never crosses sequence boundaries; causal is per sequence.
 * H*d (the row stride) must be at most 2^24 (FA_ERR_DIM beyond).
 */
int fa_fwd_varlen(const void *q, const void *k, const void *v, void *o, float *lse,
                  const int32_t *cu_seqlens, int B, int T, int max_seqlen, int H, int d,
                  float scale, int causal, int dtype, void *stream);

/*
 * fa_bwd -- attention backward by recomputation ("FlashAttention explainer"
 * section 6.2, first strategy; "YOLO11 ... FlashAttention-2" section 2.3):
 * only Q, K, V, O, dO and the forward's LSE are read; S and P are rebuilt
 * tile by tile and never stored.
 *
 *   q, k, v, o, do_ : [B, H, N, d] row-major, dtype   (read)
 *   lse             : [B, H, N] fp32 from fa_fwd       (read)
 *   dq, dk, dv      : [B, H, N, d] row-major, dtype   (written)
 *   workspace       : device scratch of fa_bwd_workspace_bytes(B,H,N,d) bytes,
 *                     16-byte aligned, owned by the caller; contents on entry
 *                     are ignored. It holds the fp32 row terms D_i = <dO_i, O_i>.
 * Head dims 64, 96, 128 and 256. The kernels enqueued on `stream`: at d = 64
 * and 128, dQ (parallel over query blocks; it also forms D_i) then dK/dV
 * (parallel over key blocks), or, when there is at most one dQ block per
 * compute unit, D_i and then one grid holding both kernels' blocks; at d = 96
 * and 256, D_i, then dK/dV as two passes (dV, then dK), then dQ (d = 256 at
 * one wave per SIMD), the three again in one grid when there is at most one
 * block of each per compute unit. There are no atomics, so results are
 * deterministic.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *do_,
           const float *lse, void *dq, void *dk, void *dv, void *workspace,
           int B, int H, int N, int d, float scale, int causal, int dtype, void *stream);

/* Bytes of workspace fa_bwd needs for this problem (0 when any size is 0;
 * -1 on invalid sizes). Host-only; makes no HIP call. */
int64_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * fa_bwd_noalloc -- fa_bwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments and results as fa_bwd, without the
 * workspace. The row terms D_i live instead in a static device array of the
 * library (FA_BWD_NOALLOC_MAX_ROWS fp32 values, 16 MiB, held by each device
 * the library runs on until the process ends). The call makes no hipMalloc or
 * hipFree and calls no allocating library routine.
 *
 *   B * H * N must be at most FA_BWD_NOALLOC_MAX_ROWS (FA_ERR_TOO_LARGE
 *   beyond, checked before any HIP call).
 *
 * All calls on one device share that device's array, whose contents persist
 * from call to call (each call writes every D_i it reads before reading it).
 * Calls that overlap in time on one device -- on different streams, or from
 * different threads without ordering -- race on it and may return wrong
 * gradients; serialise them (one stream, or events between streams).
 */
#define FA_BWD_NOALLOC_MAX_ROWS 4194304
int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o, const void *do_,
                   const float *lse, void *dq, void *dk, void *dv,
                   int B, int H, int N, int d, float scale, int causal, int dtype, void *stream);

/*
 * fa_fwd_fa1_order -- the forward with the FlashAttention-1 loop order, kept
 * as an ablation: the outer loop walks K/V blocks and the inner loop walks Q
 * blocks, so the running O, m and l of every row are re-read and re-written
 * in HBM at each outer step ("FlashAttention explainer" section 5.1). Same
 * arguments and result as fa_fwd, plus:
 *   workspace : device scratch of fa_fwd_fa1_workspace_bytes(B,H,N,d) bytes
 *               (fp32 running O, m, l), 16-byte aligned, caller-owned.
 */
int fa_fwd_fa1_order(const void *q, const void *k, const void *v, void *o, float *lse,
                     void *workspace, int B, int H, int N, int d, float scale, int causal,
                     int dtype, void *stream);
int64_t fa_fwd_fa1_workspace_bytes(int B, int H, int N, int d);

/* Human-readable text for an fa_status code (static storage). */
const char *fa_strerror(int code);

/* Library ABI version: (major << 16) | minor. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
