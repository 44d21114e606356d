/*
 * mgqa.h - C ABI of the MI355X (gfx950) masked grouped-query attention library.
 *
 * Operation (task page "TPU v6e Masked GQA Kernel Optimization", sections
 * "What You Have", "What You Submit" and "Hard Constraints"): the attention
 * forward pass over decode, prefill and encoder shapes with GQA ratios 1:1 to
 * 16:1, an optional causal mask, an optional sliding window and an optional
 * logit softcap; output in the input precision and in Q's shape; same inputs
 * give the same output bits.  For every batch b, query head h, query row i:
 *
 *   O[b,h,i,:] = sum_j softmax_j( mask( softcap( Q[b,h,i,:].K[b,g,j,:] / sqrt(d) ) ) ) V[b,g,j,:]
 *
 * with these readings of points the page leaves open:
 *   - g = h / (Hq/Hkv): consecutive query heads share one K/V head;
 *   - scale 1/sqrt(d), d the head size passed in (no padding involved);
 *   - softcap c > 0: s -> c*tanh(s/c) on the scaled score, before the mask;
 *   - causal mask aligned bottom-right: row i sits at key position
 *     p = i + Lkv - Lq and sees keys j <= p;
 *   - window W > 0: keys with p - j < W (W keys including the diagonal); without
 *     the causal mask also j - p < W;
 *   - a causal mask or a window with Lq > Lkv is rejected (rows would be empty).
 *
 * Layout: all tensors are dense row-major, element offsets computed in 64 bit:
 *   q, out : [B][Hq ][Lq ][d]      k, v : [B][Hkv][Lkv][d]
 * Element type: bf16 for attn_fwd; bf16 or fp16 for attn_fwd_ex (out has the
 * input type).  Accumulation and softmax are fp32.  All tensor pointers are
 * device pointers, 16-byte aligned; d must be a multiple of 8 (16-byte rows).
 *
 * Ownership: the caller owns q, k, v, out and any workspace.  The library keeps
 * no pointer after a call returns; the buffers must stay valid until the work
 * queued on `stream` has finished.  q, k, v are read only; out must not overlap
 * them.  `stream` is a hipStream_t passed as void* (NULL: the null stream).
 * All work of one call is queued on that stream; calls return without waiting.
 *
 * Errors: every entry point returns 0 on success or a negative MGQA_ERR_* code.
 * Arguments are validated before any HIP call; on a validation error nothing
 * is queued.  Faults inside a kernel surface at the caller's next
 * synchronisation, as usual for HIP.  attn_error_string() gives the text.
 *
 * Determinism: the kernel choice, tiling and split plan depend on the shape
 * and options only, no float atomics are used and every reduction has a fixed
 * order, so identical inputs give bit-identical outputs on one device and build.
 */
#ifndef MGQA_H
#define MGQA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MGQA_OK             0
#define MGQA_ERR_NULL      -1  /* a required pointer is NULL                         */
#define MGQA_ERR_SHAPE     -2  /* a size <= 0, Hq % Hkv != 0 or Hq/Hkv > 16           */
#define MGQA_ERR_HEAD_DIM  -3  /* d not a multiple of 8 or d > 128                    */
#define MGQA_ERR_MASK      -4  /* window < 0, causal not 0/1, or mask with Lq > Lkv   */
#define MGQA_ERR_SOFTCAP   -5  /* softcap negative, NaN or infinite                   */
#define MGQA_ERR_ALIGN     -6  /* a tensor pointer not 16-byte aligned                */
#define MGQA_ERR_WORKSPACE -7  /* workspace missing or smaller than required          */
#define MGQA_ERR_HIP       -8  /* a HIP runtime call or kernel launch failed          */
#define MGQA_ERR_DTYPE     -9  /* dtype not MGQA_BF16 / MGQA_FP16                      */
#define MGQA_ERR_RANGE    -10  /* a size too large for the library's 32-bit indexing
                                  (Lkv*d or S*d above 2^30, Lq*Hq at or above 2^31,
                                  a tensor above 2^40 elements), or a cache length,
                                  ring start or append position outside the cache */
#define MGQA_ERR_UNSUPPORTED -11 /* a valid combination this library does not run      */

#define MGQA_BF16 0
#define MGQA_FP16 1
#define MGQA_F32  2  /* KV-cache storage only (kv_cache_append) */

/* Masked GQA attention forward, bf16 in and out.  window <= 0 means no window,
 * softcap <= 0 means no softcap, causal is 0 or 1.  Allocates its own
 * stream-ordered workspace when the split decode path needs one
 * (hipMallocAsync / hipFreeAsync on `stream`). */
int attn_fwd(const void* q, const void* k, const void* v, void* out,
             int B, int Hq, int Hkv, int Lq, int Lkv, int d,
             int causal, int window, float softcap, void* stream);

/* Bytes of workspace attn_fwd_ex needs for this shape (0 when the planned path
 * needs none).  Returns 0 as well for arguments attn_fwd_ex would reject. */
size_t attn_workspace_bytes(int B, int Hq, int Hkv, int Lq, int Lkv, int d,
                            int causal, int window);

/* Same operation with an explicit element type (MGQA_BF16 or MGQA_FP16) and a
 * caller-provided workspace of at least attn_workspace_bytes() bytes (may be
 * NULL when that is 0).  The workspace holds arrival counters in its first
 * 1024 bytes (the same bytes for every shape) and fp32 split partials after
 * them.  It must be zero-filled before its first use; every call that completes
 * leaves the counters at zero again, so one workspace can be reused by later
 * calls of any shape on the same stream without clearing.  Calls that run
 * concurrently (different streams) must use different workspaces. */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* out,
                int B, int Hq, int Hkv, int Lq, int Lkv, int d,
                int causal, int window, float softcap, int dtype,
                void* workspace, size_t workspace_bytes, void* stream);

/* Largest split workspace attn_fwd_noalloc serves from its device-resident
 * scratch (8 MiB per GPU). */
#define MGQA_NOALLOC_SCRATCH_BYTES (8u << 20)

/* attn_fwd_ex without any allocation and without a workspace argument, for
 * callers that cannot allocate device memory (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The split partials
 * and arrival counters live in a device array inside the library, one per GPU
 * (MGQA_NOALLOC_SCRATCH_BYTES, held until the process ends).  On the first call
 * that needs it on a device, the library looks up that GPU's copy and clears
 * its counter block with a kernel on `stream` (so the first such call on a
 * device must not be under graph capture); later calls need no clearing,
 * because every completed call leaves the counters at zero.  Plans whose
 * workspace (attn_workspace_bytes) exceeds MGQA_NOALLOC_SCRATCH_BYTES return
 * MGQA_ERR_WORKSPACE before any HIP call.  All calls on one GPU share the
 * scratch: calls that can overlap on one GPU (different streams, or several
 * host threads) race and must not be issued.  Same operation, dtypes, layouts,
 * output bits and other errors as attn_fwd_ex. */
int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                     int B, int Hq, int Hkv, int Lq, int Lkv, int d,
                     int causal, int window, float softcap, int dtype, void* stream);

/* Attention over the first `length` keys of a KV cache of S slots per
 * (batch, kv head): K/V rows of head (b, g) start at element (b*Hkv + g)*S*d
 * ([B][Hkv][S][d], the layout kv_cache_append writes with layout 1).  Same
 * operation, options, dtypes, workspace rules and errors as attn_fwd_ex with
 * Lkv = length (attn_workspace_bytes with Lkv = length gives the workspace).
 *
 * ring_start = -1: keys 0..length-1 are slots 0..length-1.
 * ring_start in [0, S): ring buffer; logical key j (0 <= j < length <= S) is
 * slot (ring_start + j) mod S, and the causal/window rules apply to logical
 * positions.  A sliding-window decode over a ring of S = W slots is the same
 * attention as a linear decode over the last W keys (the "ring or linear
 * windows" of the Metal attention pull request).  The ring form runs on the
 * decode path only (Hq/Hkv * Lq <= 16); otherwise MGQA_ERR_UNSUPPORTED. */
int attn_fwd_cache(const void* q, const void* k_cache, const void* v_cache, void* out,
                   int B, int Hq, int Hkv, int Lq, int S, int length, int ring_start, int d,
                   int causal, int window, float softcap, int dtype,
                   void* workspace, size_t workspace_bytes, void* stream);

/* One decode (or chunked-prefill) step over a KV cache with the cache update
 * folded in: the KV-cache update at a position of the TensorTonic page ("KV
 * Cache Update at a Position") followed by the attention of the task page
 * over the updated cache.  After the call the cache holds length =
 * position + Lq logical keys; logical key j lives in slot j (ring_start = -1,
 * linear cache) or in slot (ring_start + j) mod S (ring buffer, as in
 * attn_fwd_cache).  The Lq new rows are logical keys position ..
 * position+Lq-1, and the Lq query rows sit at those positions (the
 * bottom-right alignment).  For a linear cache this equals
 *   kv_cache_append(k_cache, v_cache, new_k, new_v, B, S, Hkv, d, Lq, position,
 *                   dtype, 1, NULL, stream);
 *   attn_fwd_cache(q, k_cache, v_cache, out, B, Hq, Hkv, Lq, S, position + Lq, -1,
 *                  d, causal, window, softcap, dtype, workspace, workspace_bytes, stream);
 * with the same output bits and the same cache contents afterwards; for a
 * ring, the same with the new rows written to their ring slots.
 *   q, out      : [B][Hq][Lq][d] of dtype.
 *   k/v_cache   : [B][Hkv][S][d] of dtype, updated in place: the new rows' slots
 *                 receive new_k / new_v rounded to dtype (nearest even); no
 *                 other slot is written.
 *   new_k/new_v : float32 [B][Hkv][Lq][d], 16-byte aligned, not overlapping the caches.
 * Requires 0 <= position <= S - Lq and -1 <= ring_start < S (else
 * MGQA_ERR_RANGE).  On the split-KV path (decode, multi-token decode) this is
 * one kernel launch that reads the new keys from new_k / new_v and writes them
 * to the caches itself; otherwise the update kernel runs first on the same
 * stream (linear caches only: a ring needs the decode path, Hq/Hkv * Lq <= 16,
 * else MGQA_ERR_UNSUPPORTED).  Workspace: attn_workspace_bytes with
 * Lkv = position + Lq.  Other arguments, errors and ownership as attn_fwd_ex. */
int attn_fwd_cache_append(const void* q, void* k_cache, void* v_cache, const float* new_k,
                          const float* new_v, void* out, int B, int Hq, int Hkv, int Lq, int S,
                          int position, int ring_start, int d, int causal, int window, float softcap,
                          int dtype, void* workspace, size_t workspace_bytes, void* stream);

/* KV-cache update at a position (TensorTonic, "KV Cache Update at a
 * Position"): for every batch row and head, slots position .. position+L-1 of
 * k_cache / v_cache receive the L new float32 vectors converted to the cache
 * type (round to nearest even); every other slot is left untouched.
 *   layout 0: caches [B][S][H][D], new vectors [B][L][H][D] (the page's layout)
 *   layout 1: caches [B][H][S][D], new vectors [B][H][L][D] (attn_fwd_cache's)
 * cache_dtype: MGQA_F32, MGQA_BF16 or MGQA_FP16.  Requires 0 <= position <= S-L
 * (else MGQA_ERR_RANGE).  If length_out (device int32) is not NULL, the kernel
 * writes position + L there.  Caches are updated in place on `stream`; new_k,
 * new_v must not overlap the caches.  D may be any positive size. */
int kv_cache_append(void* k_cache, void* v_cache, const float* new_k, const float* new_v,
                    int B, int S, int H, int D, int L, int position, int cache_dtype, int layout,
                    int* length_out, void* stream);

/* Plan the library would use for this shape, without touching the GPU.
 * info[0] path: 0 = prefill kernel (every wave sweeps the whole key band of
 *         its rows; 128-row workgroups for head sizes 104..128, 256-row
 *         otherwise),
 *         1 = split-KV kernel (decode, multi-token decode and
 *         short sequences: the waves of a workgroup, and possibly several
 *         workgroups, split the key band of its rows),
 *         2 = short-band kernel (three 16-row blocks over a key band of at
 *         most 768 keys, head size 49..96, e.g. the 729-token encoder: each
 *         of 8 waves takes its own contiguous keys; info[4] is the most keys
 *         one wave takes)
 * info[1] workgroups launched
 * info[2] query rows (head, position pairs) per workgroup
 * info[3] key splits per block of rows (1 on the prefill path); workgroups =
 *         blocks of rows x info[3] x info[8]
 * info[4] keys per tile
 * info[5] padded head size used for Q.K^T (multiple of 32)
 * info[6] padded head size used for P.V (multiple of 16)
 * info[7] workspace bytes
 * info[8] column slices: workgroups sharing one key range of a block of rows,
 *         each computing P.V for its share of the head size (1, or 2 when a
 *         single 16-row block has many key splits; split path only)
 * info[9..11] work items of the head-size-128 prefill kernel (0 otherwise).
 *         Per (batch row, kv head) there are n blocks of info[2]/G
 *         positions and info[1]/(B*Hkv) workgroups: the first
 *         ceil(info[10]/2) each run blocks info[10]-1-j and j one after the
 *         other (the short-band ramp under a causal mask, ends paired; one
 *         block when the two coincide), the next info[11] one whole block
 *         each (n-1 downwards), the rest one half block each (the next
 *         blocks downwards, two halves of info[2]/(2G) positions apiece).
 *         info[9] = ceil(info[10]/2).
 * Returns 0 or a validation error code (then info is untouched). */
int attn_plan(int B, int Hq, int Hkv, int Lq, int Lkv, int d,
              int causal, int window, float softcap, int dtype, long long info[12]);

/* Static text for an error code (never NULL). */
const char* attn_error_string(int code);

/* Library ABI version (major*100 + minor). */
int attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MGQA_H */
