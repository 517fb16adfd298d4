/*
 * rswa.h -- C ABI of librswa: Reference Sliding Window Attention (R-SWA) on
 * AMD Instinct MI355X (gfx950).
 *
 * R-SWA, as the pages define it: every query attends to the whole reference
 * segment P = {1..L_m} (vision tokens + prompt, encoded once and never
 * updated) plus the causal window D_n(t) of the n most recent output tokens
 *   WeThinkIn "Unlimited OCR Works：一篇读懂 R-SWA 如何把长文档 OCR 从 for-loop
 *   推向 one-shot", section 方法展开.3, Eqs. (1)-(4);
 * so the KV cache holds L_m + min(n, T) entries after T outputs (same page,
 * section 方法展开.4, Eq. (6)). The cache is a queue of capacity m + n whose
 * oldest output (position m+1) is evicted by each new token
 *   夜雨聆风 "多模态文档解析开源新进展:Unlimited OCR技术方案", section
 *   "为什么它能”无限”读下去？关键在 KV cache 恒定";
 * i.e. a fixed-capacity output KV buffer of width n on top of the reference
 * KV cache (yhxrc.cn news article, section "R-SWA 如何穩住長程解碼？").
 *
 * General rules for every call
 *  - All tensor pointers are DEVICE pointers owned by the caller. The library
 *    allocates no device memory (rswa_decode_attn_noalloc uses a static buffer
 *    reserved when the library loads) and no host memory except the handle of
 *    rswa_decode_graph_create; its only mutable global state is that static
 *    buffer and the per-device table of its addresses.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls
 *    only enqueue work on it and return; none synchronises except
 *    rswa_check_device_error.
 *  - Arguments are validated on the host before anything is enqueued. On an
 *    error the call returns a negative rswa_status_t and enqueues nothing.
 *    Errors from the HIP runtime at launch map to RSWA_ERR_HIP.
 *  - Facts only visible on the device (per-sequence lengths and counters) are
 *    checked by the kernels; a violation sets a bit in the cache's device
 *    error word (RSWA_DEVERR_*), skips the affected sequence and is read back
 *    by rswa_check_device_error.
 *  - Tensors of element type rswa_dtype_t; bf16 means IEEE bfloat16 bit
 *    patterns. All pointers must be 16-byte aligned.
 *  - Calls that use the same cache or the same workspace must be ordered (one
 *    stream, or events between streams): their device state (step, arrive,
 *    window slots, partial results) is read and written without locks.
 *  - Nothing is thrown across the ABI and nothing aborts.
 */
#ifndef RSWA_H
#define RSWA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RSWA_ABI_VERSION 9

#if defined(__GNUC__)
#define RSWA_API __attribute__((visibility("default")))
#else
#define RSWA_API
#endif

typedef enum {
  RSWA_OK = 0,
  RSWA_ERR_NULL = -1,        /* a required pointer is NULL                          */
  RSWA_ERR_SHAPE = -2,       /* a size/shape argument is out of range               */
  RSWA_ERR_UNSUPPORTED = -3, /* valid but not implemented (dtype, head_dim, mode)   */
  RSWA_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned                    */
  RSWA_ERR_CAPACITY = -5,    /* sizes would overflow the kernels' index arithmetic  */
  RSWA_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required          */
  RSWA_ERR_STATE = -7,       /* device-side state was found invalid                 */
  RSWA_ERR_HIP = -8          /* the HIP runtime reported an error                   */
} rswa_status_t;

typedef enum { RSWA_BF16 = 0, RSWA_FP32 = 1 } rswa_dtype_t;

/* Visibility of rows inside the reference prefix in the packed form. The pages
 * define N(t) for output tokens only; prefix rows are causal by default. */
typedef enum { RSWA_PREFIX_CAUSAL = 0, RSWA_PREFIX_FULL = 1 } rswa_prefix_mode_t;

/* Bits of the device error word. */
#define RSWA_DEVERR_REF_LEN 1   /* ref_len[b] < 0 or > max_ref_len                   */
#define RSWA_DEVERR_STEP 2      /* step[b] < 0, or step[b] would overflow int32      */
#define RSWA_DEVERR_EMPTY 4     /* decode with nothing visible (L_m = 0 and T = 0)   */
#define RSWA_DEVERR_ALIGN 8     /* seq_base[b] / ref_base[b] not 16-byte aligned     */
#define RSWA_DEVERR_PACK 16     /* prefill: cu_seqlens inconsistent for sequence b,
                                   or ref_len[b] larger than its rows                */

/*
 * KV cache descriptor (plain struct, caller-owned, passed by pointer).
 *
 * Sequence b owns one contiguous block in each of the pools k and v, starting
 * at ELEMENT offset seq_base[b], laid out [H][ref_len[b] + window][head_dim]:
 *   head h, slot s  ->  pool + seq_base[b] + ((int64)h*(ref_len[b]+window) + s)*head_dim
 * Slots 0 .. ref_len[b]-1 hold the reference segment (position p in slot p-1).
 * Output token T (T = 1, 2, ...) is written to slot
 *   ref_len[b] + ((T - 1) mod window)
 * which overwrites output T - window, the oldest one, exactly when the queue
 * of capacity L_m + n is full. This slot rule is part of the ABI: a caller may
 * build a cache state directly. After T outputs, slots [0, L_m + min(n, T))
 * are occupied and all of them are visible to the next query (attention does
 * not depend on key order).
 *
 * step[b] is T, the number of outputs appended so far. It lives on the device
 * so that decode steps need no host synchronisation.
 *
 * arrive (optional, ABI 6) is device int32 [B] of arrival counters that let a
 * fused decode step run as one launch (see rswa_decode_attn). It must hold
 * zeros before the first decode call; rswa_cache_init and rswa_prefill zero
 * it, and every decode call leaves it zero. NULL keeps the two-launch path.
 */
typedef struct rswa_cache {
  int32_t batch;        /* B >= 1                                                 */
  int32_t num_heads;    /* H >= 1; MHA: query heads == KV heads                   */
  int32_t head_dim;     /* d in {64, 128}                                         */
  int32_t window;       /* n >= 1 (the pages' default is 128)                     */
  int32_t max_ref_len;  /* host-side bound: 0 <= ref_len[b] <= max_ref_len        */
  int32_t dtype;        /* rswa_dtype_t of the pools and of q/out/k_new/v_new     */
  void *k;              /* device pool of keys                                    */
  void *v;              /* device pool of values                                  */
  const int64_t *seq_base; /* device [B], element offsets (multiple of 16 bytes)  */
  const int32_t *ref_len;  /* device [B], L_m per sequence                        */
  int32_t *step;           /* device [B], T per sequence                          */
  int32_t *error;          /* device, one int32 word of RSWA_DEVERR_* bits        */
  int32_t *arrive;         /* NULL, or device [B] arrival counters (see below)    */
} rswa_cache_t;

/* Library ABI version (RSWA_ABI_VERSION). */
RSWA_API int32_t rswa_abi_version(void);

/* Static string for a status code; never NULL. */
RSWA_API const char *rswa_status_str(int32_t status);

/*
 * Write the reference segment into the cache ("encoded once, never updated":
 * 夜雨聆风 page, same section as above) and reset step[b] = 0 (and arrive[b] = 0
 * when arrive is set) for every b.
 * k_ref, v_ref: device; sequence b's reference at element offset ref_base[b]
 * (device [B]), laid out [H][ref_len[b]][head_dim], same dtype as the cache.
 * When max_ref_len == 0 the three may be NULL. Does not touch the window slots.
 */
RSWA_API rswa_status_t rswa_cache_init(const rswa_cache_t *cache, const void *k_ref, const void *v_ref,
                              const int64_t *ref_base, void *stream);

/*
 * Append one output token per sequence (and evict the oldest output once the
 * window is full): for each b with active == NULL or active[b] != 0, write
 * k_new[b][h][:], v_new[b][h][:] into slot ref_len[b] + (step[b] mod window)
 * of every head h, then step[b] += 1. Bit-exact copy.
 * k_new, v_new: device [B][H][head_dim]; active: NULL or device uint8 [B].
 */
RSWA_API rswa_status_t rswa_append_kv(const rswa_cache_t *cache, const void *k_new, const void *v_new,
                             const uint8_t *active, void *stream);

/*
 * Workspace bytes needed by rswa_decode_attn with the library's split choice
 * (num_splits = 0) for a cache of `batch` sequences of `num_heads` heads of
 * dimension head_dim whose longest sequence holds max_len = max_ref_len +
 * window slots: the per-split partial softmax states of the fixed-capacity
 * cache (yhxrc page, "R-SWA 如何穩住長程解碼？"; 夜雨聆风 page, "为什么它能”无限”读下去？
 * 关键在 KV cache 恒定"). Equals rswa_decode_workspace_size(cache, 0) for a
 * descriptor with those sizes. Returns 0 for invalid sizes (batch or num_heads
 * < 1, head_dim not 64 or 128, max_len < 1, batch * num_heads >= 2^30).
 */
RSWA_API size_t rswa_workspace_size(int32_t batch, int32_t num_heads, int32_t head_dim,
                                    int32_t max_len);

/*
 * Workspace bytes needed by rswa_decode_attn for this cache descriptor and
 * split count (0 = the library's choice). Returns 0 for an invalid
 * descriptor. The workspace holds per-split partial softmax states.
 */
RSWA_API size_t rswa_decode_workspace_size(const rswa_cache_t *cache, int32_t num_splits);

/*
 * One decode step of attention for every sequence (WeThinkIn page, Eqs.
 * (1)-(4)): out[b][h] = softmax(scale * K_vis q[b][h]) V_vis over the visible
 * slots [0, L_m + min(n, T)) of sequence b, head h.
 *
 *  q, out       device [B][H][head_dim], cache dtype. bf16 output is rounded
 *               to nearest even from the fp32 result.
 *  k_new, v_new both NULL: attend over the cache as it is (T = step[b]).
 *               both non-NULL (device [B][H][head_dim]): fused append+attend.
 *               The new token is appended exactly as rswa_append_kv would do,
 *               then attended to (T = step[b] + 1), and step[b] is incremented.
 *               The evicted entry is never read.
 *  scale        softmax scale; 0 selects 1/sqrt(head_dim). Must be finite.
 *  num_splits   0 = the library's choice; otherwise the number of key chunks
 *               per (sequence, head) merged at the end (>= 1). The result does
 *               not depend on it beyond fp32 rounding.
 *  workspace    device, >= rswa_decode_workspace_size(cache, num_splits) bytes.
 *
 * Accumulation is fp32. Softmax runs in base 2 with log2(e) folded into the
 * scale.
 *
 * Launches: with more than one split, a split kernel and a merge kernel. With
 * one split the split kernel writes out itself (one launch); a fused call then
 * also needs cache->arrive (otherwise it keeps the merge launch): the H
 * workgroups of sequence b count their arrival in arrive[b], and the last one
 * publishes step[b] and sets arrive[b] back to 0. arrive must hold zeros before
 * the first call (rswa_cache_init zeroes it) and is zero again after every
 * call. The library picks one split when every sequence fits one chunk of a
 * batch that fills the GPU. With num_splits = 0 and a large step that does not
 * qualify (batch * heads * (max_ref_len + window) >= 2^22 slots, e.g. a ragged
 * batch), it instead cuts the visible slots of all (sequence, head) pairs,
 * counted on the device, into equal pieces, one per workgroup, and merges the
 * pieces' partial states per pair (a work-list kernel and a merge kernel).
 */
RSWA_API rswa_status_t rswa_decode_attn(const rswa_cache_t *cache, const void *q, void *out,
                               const void *k_new, const void *v_new, float scale,
                               int32_t num_splits, void *workspace, size_t workspace_bytes,
                               void *stream);

/*
 * rswa_decode_attn for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops or harnesses that forbid hipMalloc): the
 * same arguments, checks, kernels and results as rswa_decode_attn, but the
 * per-split partial states live in a library-owned static device buffer of
 * RSWA_NOALLOC_SCRATCH_BYTES (8 MiB) instead of a caller workspace. The call
 * allocates nothing; each GPU the library runs on holds its own buffer until
 * the process ends, and the first call on a device (that device current) looks
 * up its address. Nothing in the buffer needs to start at zero (every call
 * writes the partial states before it reads them).
 *  Returns RSWA_ERR_WORKSPACE when rswa_decode_workspace_size(cache,
 *  num_splits) exceeds RSWA_NOALLOC_SCRATCH_BYTES (e.g. 32 sequences x 16
 *  heads with 64 splits), without enqueuing anything.
 * All calls on one GPU share its buffer: calls that may overlap (different
 * streams, or a graph replay beside an eager call) race on it and must be
 * ordered by the caller.
 */
#define RSWA_NOALLOC_SCRATCH_BYTES (8u << 20)
RSWA_API rswa_status_t rswa_decode_attn_noalloc(const rswa_cache_t *cache, const void *q, void *out,
                                                const void *k_new, const void *v_new, float scale,
                                                int32_t num_splits, void *stream);

/*
 * Packed (teacher-forced) R-SWA forward over one sequence of seq_len tokens:
 * row i attends to key j iff j <= i and (j < ref_len or i - j < window); with
 * RSWA_PREFIX_FULL, rows i < ref_len instead attend to all j < ref_len. For a
 * row i >= ref_len this is N(t) of the WeThinkIn page's Eqs. (1)-(2) for the
 * query formed at position i. q, k, v, out: device [seq_len][num_heads][head_dim]
 * bf16 (row-major, heads interleaved). Only RSWA_BF16 and head_dim 128 are
 * implemented. QK^T and PV run on bf16 matrix cores with fp32 accumulation;
 * the probabilities are rounded to bf16 before the PV product.
 * lse: NULL, or device float [num_heads][seq_len] receiving each row's natural
 * log of the softmax normaliser, log sum_j exp(scale q_i.k_j) over the visible
 * keys (the input the backward pass needs). The sum runs over the same
 * bf16-rounded probabilities that enter PV, so lse is within about 2^-8 of the
 * exact value (bf16 keeps 8 significant bits).
 * scale: 0 selects 1/sqrt(head_dim); otherwise finite and > 0. The packed
 * kernels track each row's maximum of the unscaled scores and mask with -inf
 * before scaling, which needs a positive scale; a negative one is rejected
 * with RSWA_ERR_SHAPE here and in every other packed call (varlen, prefill and
 * both backward calls). The decode calls accept any finite scale.
 * Sizes: seq_len * num_heads * head_dim below 2^31 and num_heads below 2^16
 * (the kernels' offsets are 32-bit, their row offsets 24-bit products), else
 * RSWA_ERR_CAPACITY; the same limits hold for every other packed call (with
 * total_tokens, or the cache's heads for rswa_prefill).
 */
RSWA_API rswa_status_t rswa_masked_attn(const void *q, const void *k, const void *v, void *out,
                               float *lse, int32_t seq_len, int32_t ref_len, int32_t window,
                               int32_t num_heads, int32_t head_dim, int32_t dtype,
                               int32_t prefix_mode, float scale, void *stream);

/*
 * Packed forward over several samples per pack ("varlen"): sample s owns rows
 * [cu_seqlens[s], cu_seqlens[s+1]) of q, k, v, out (same [rows][H][head_dim]
 * bf16 layout as rswa_masked_attn, total_tokens rows in all) and has its own
 * reference length ref_lens[s]; inside a sample the visibility is exactly that
 * of rswa_masked_attn, and no row sees another sample's keys. The pages pack
 * 2-50-page samples into 32K sequences for training (WeThinkIn page, section
 * 实验与证据.1) without stating a cross-sample mask; this call takes the reading
 * that samples are independent.
 *  cu_seqlens   device int32 [num_seqs + 1], non-decreasing, cu_seqlens[0] >= 0,
 *               cu_seqlens[num_seqs] <= total_tokens.
 *  ref_lens     device int32 [num_seqs], 0 <= ref_lens[s] <= sample length.
 *  max_seq_len  host bound on every sample's length (sets the grid).
 *  lse          NULL, or device float [num_heads][total_tokens] (per pack row).
 * The device arrays are not read on the host: a sample that breaks these
 * rules (or is longer than max_seq_len) is skipped and its rows are not
 * written. Rows outside every sample are not written either.
 */
RSWA_API rswa_status_t rswa_masked_attn_varlen(const void *q, const void *k, const void *v, void *out,
                                      float *lse, const int32_t *cu_seqlens,
                                      const int32_t *ref_lens, int32_t num_seqs,
                                      int32_t total_tokens, int32_t max_seq_len, int32_t window,
                                      int32_t num_heads, int32_t head_dim, int32_t dtype,
                                      int32_t prefix_mode, float scale, void *stream);

/*
 * Prefill -> decode hand-off for every sequence of a cache: sample b of the
 * pack (rows [cu_seqlens[b], cu_seqlens[b+1]), cu_seqlens device int32
 * [batch + 1]) is sequence b's reference segment (ref_len[b] rows, the
 * cache's device value) followed by its first T0_b = rows - ref_len[b]
 * outputs (output t at row ref_len[b] + t - 1, the token whose query is q_t).
 * One call runs the packed forward of every sample (as rswa_masked_attn_varlen
 * with window = cache->window, out and lse as there) and leaves the cache as
 * rswa_cache_init followed by T0_b appends would: reference rows in slots
 * 0 .. ref_len[b]-1, the last min(window, T0_b) outputs in their ring slots
 * ref_len[b] + ((t-1) mod window), step[b] = T0_b, arrive[b] = 0 when
 * arrive is set (yhxrc and 夜雨聆风 pages;
 * WeThinkIn page, Eq. (6)). Decode then continues with output T0_b + 1.
 *  q, k, v, out  device [total_tokens][num_heads][head_dim], cache dtype; only
 *                RSWA_BF16 with head_dim 128 (the packed kernel's case). k and v
 *                must not overlap the cache pools.
 * One kernel launch: each forward workgroup also copies the cache-kept rows of
 * its own query block into the cache. A sequence whose sample does not fit
 * (RSWA_DEVERR_PACK) or whose cache metadata are invalid (RSWA_DEVERR_REF_LEN,
 * RSWA_DEVERR_ALIGN) is flagged in the error word and its cache block and step
 * are left untouched; the rows of every well-formed sample are still computed.
 */
RSWA_API rswa_status_t rswa_prefill(const rswa_cache_t *cache, const void *q, const void *k,
                           const void *v, void *out, float *lse, const int32_t *cu_seqlens,
                           int32_t total_tokens, int32_t max_seq_len, int32_t prefix_mode,
                           float scale, void *stream);

/*
 * Bytes of device workspace rswa_masked_attn_bwd needs for these sizes and
 * num_parts (0 = the library's choice, as in the call). 0 for invalid sizes
 * and for sizes the call rejects with RSWA_ERR_CAPACITY.
 */
RSWA_API size_t rswa_masked_bwd_workspace_size(int32_t seq_len, int32_t ref_len, int32_t num_heads,
                                               int32_t num_parts);

/*
 * Backward of rswa_masked_attn for the loss sum(dout * out): the gradients of
 * O_i = softmax(scale K_J q_i) V_J over the same visible sets J(i) (WeThinkIn
 * page, Eqs. (1)-(4), the packed reading described at rswa_masked_attn):
 *   dV_j = sum_i P_ij dO_i,  dS_ij = P_ij (dO_i . v_j - dO_i . O_i),
 *   dQ_i = scale sum_j dS_ij k_j,  dK_j = scale sum_i dS_ij q_i.
 * The softmax weights P are recomputed from lse.
 *
 *  q, k, v, out, dout  device [seq_len][num_heads][head_dim] bf16; out and lse
 *               are the forward's outputs for the same q, k, v, sizes, mode
 *               and scale (other values give gradients of nothing defined).
 *  lse          device float [num_heads][seq_len] from rswa_masked_attn.
 *  dq, dk, dv   device [seq_len][num_heads][head_dim] bf16, written whole
 *               (keys no row sees get zero). Must not alias the inputs.
 *  num_parts    0 = the library's choice; otherwise 1..64: the rows that
 *               see a reference-segment key are walked in this many runs
 *               whose fp32 partial sums are added in a fixed order (more
 *               runs spread long walks over more compute units). The
 *               result does not depend on it beyond fp32 rounding.
 *  workspace    device, 16-byte aligned, >= rswa_masked_bwd_workspace_size
 *               bytes for the same sizes and num_parts; its contents on entry
 *               do not matter.
 * Same restrictions as the forward (RSWA_BF16, head_dim 128). Matrix products
 * run on bf16 matrix cores with fp32 accumulation; P and dS are rounded to
 * bf16 as operands. The kernels use no atomics: repeated calls give
 * identical bits.
 */
RSWA_API rswa_status_t rswa_masked_attn_bwd(const void *q, const void *k, const void *v,
                                   const void *out, const void *dout, const float *lse,
                                   void *dq, void *dk, void *dv, int32_t seq_len,
                                   int32_t ref_len, int32_t window, int32_t num_heads,
                                   int32_t head_dim, int32_t dtype, int32_t prefix_mode,
                                   float scale, int32_t num_parts, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * Bytes of device workspace rswa_masked_attn_bwd_varlen needs for a pack of
 * total_tokens rows. 0 for invalid sizes and for sizes the call rejects with
 * RSWA_ERR_CAPACITY.
 */
RSWA_API size_t rswa_masked_bwd_varlen_workspace_size(int32_t total_tokens, int32_t num_heads);

/*
 * rswa_masked_attn_bwd over a pack of independent samples: the backward of
 * rswa_masked_attn_varlen for the loss sum(dout * out). Training runs on
 * samples of 1 to 50 pages up to a 32K-token length (WeThinkIn page, section
 * 实验与证据, 训练设置); a pack lets one call take a batch of them unpadded.
 * Each sample gets exactly the single-sequence gradients of its own rows.
 *  q, k, v, out, dout  device [total_tokens][num_heads][head_dim] bf16; out
 *               and lse come from rswa_masked_attn_varlen with the same
 *               cu_seqlens, ref_lens, sizes, window, mode and scale.
 *  lse          device float [num_heads][total_tokens] from that call.
 *  cu_seqlens, ref_lens, num_seqs, total_tokens, max_seq_len
 *               as for rswa_masked_attn_varlen (device int32 arrays).
 *  dq, dk, dv   device [total_tokens][num_heads][head_dim] bf16. Every row of
 *               every valid sample is written (keys no row sees get zero);
 *               rows outside every sample, and the rows of a sample whose
 *               metadata are invalid, are left as they were. Must not alias
 *               the inputs.
 *  workspace    device, 16-byte aligned, >= rswa_masked_bwd_varlen_workspace_size
 *               bytes; its contents on entry do not matter.
 * Same restrictions as rswa_masked_attn_bwd; no atomics, repeated calls give
 * identical bits, and a pack of one sample gives the bits of
 * rswa_masked_attn_bwd whenever that call runs in one part (seq_len up to
 * 8192 rows with num_parts 0).
 */
RSWA_API rswa_status_t rswa_masked_attn_bwd_varlen(
    const void *q, const void *k, const void *v, const void *out, const void *dout,
    const float *lse, void *dq, void *dk, void *dv, const int32_t *cu_seqlens,
    const int32_t *ref_lens, int32_t num_seqs, int32_t total_tokens, int32_t max_seq_len,
    int32_t window, int32_t num_heads, int32_t head_dim, int32_t dtype, int32_t prefix_mode,
    float scale, void *workspace, size_t workspace_bytes, void *stream);

/*
 * A decode step through several attention layers as one HIP graph. A decoder
 * replaces every attention layer with R-SWA (WeThinkIn page, 核心导读), so a
 * decode step is one rswa_decode_attn per layer, each with its own cache. These
 * calls record the num_layers calls once -- layer l:
 *   rswa_decode_attn(&caches[l], q[l], out[l], k_new ? k_new[l] : NULL,
 *                    v_new ? v_new[l] : NULL, scale, num_splits, workspace, ...)
 * in that order -- and replay them with one launch. The arrays are host arrays
 * read at creation; the device buffers they name are baked into the graph, so
 * a caller refreshes q/k_new/v_new in place between launches. Each replay runs
 * exactly what the eager calls would (same kernels, same step counters on the
 * device: fused calls advance step[b] on every replay). One workspace serves
 * every layer (the layers run in order); it must hold
 * max over l of rswa_decode_workspace_size(&caches[l], num_splits).
 *  create   validates every layer as rswa_decode_attn would (nothing is
 *           enqueued on failure), captures on an internal stream and
 *           instantiates; *graph receives an opaque handle (host memory plus
 *           HIP graph objects, freed by rswa_decode_graph_destroy).
 *  launch   enqueues one replay on `stream` (asynchronous).
 * The captured work holds no memset nodes, only the decode kernels. Replays
 * of one graph, and replays of graphs that share caches or workspace, must
 * not run concurrently.
 * Use it for several layers: one replay costs more host and launch time than
 * the one or two kernel launches of a single eager call (one layer of a
 * one-page step: 14 us replayed against 8 us eagerly; 12 layers: 87 us against
 * 96 us).
 */
typedef struct rswa_decode_graph rswa_decode_graph_t;

RSWA_API rswa_status_t rswa_decode_graph_create(const rswa_cache_t *caches, int32_t num_layers,
                                       const void *const *q, void *const *out,
                                       const void *const *k_new, const void *const *v_new,
                                       float scale, int32_t num_splits, void *workspace,
                                       size_t workspace_bytes, rswa_decode_graph_t **graph);
RSWA_API rswa_status_t rswa_decode_graph_launch(const rswa_decode_graph_t *graph, void *stream);
RSWA_API rswa_status_t rswa_decode_graph_destroy(rswa_decode_graph_t *graph);

/*
 * Measurement helper, not part of the attention path: streams `bytes` (a
 * multiple of 16) from device buffer `buf` with the decode kernel's access
 * pattern (16-byte non-temporal loads, 1 KB contiguous per wave instruction),
 * writing one value per workgroup to `sink` (device float [workgroups], 1024
 * entries when workgroups = 0, which picks 4 per CU) so that the loads are not
 * optimised away.
 * Timing it gives the achievable read rate that bounds rswa_decode_attn.
 */
RSWA_API rswa_status_t rswa_probe_stream_read(const void *buf, size_t bytes, float *sink,
                                     int32_t workgroups, void *stream);

/*
 * Measurement helper, not part of the attention path: `workgroups` workgroups
 * of 4 waves (0 picks 512, two waves per SIMD on 256 CUs) each run `iters`
 * rounds of 4 independent v_mfma_f32_32x32x16_bf16 products (the packed
 * kernels' instruction; 32768 FLOP each) and write one value per workgroup to
 * `sink` (device float [workgroups]). FLOP = workgroups * 4 waves * iters * 4 *
 * 32768; timing it gives the matrix-core rate the chip sustains at the clock it
 * holds under matrix load, the practical ceiling of the packed kernels.
 */
RSWA_API rswa_status_t rswa_probe_mfma(float *sink, int32_t workgroups, int32_t iters, void *stream);

/*
 * Measurement helper, not part of the attention path: per-CU rates of the units
 * the packed kernels lean on besides the matrix cores, in shader-clock cycles.
 * `workgroups` workgroups of 8 waves (0 picks 256: one per CU, which their
 * 96 KB of LDS enforces; two waves per SIMD, the packed forward's count) each
 * run `iters` rounds of one kind of instruction after a barrier and record the
 * cycles the rounds took (s_memtime on wave 0):
 *   RSWA_PROBE_LDS_B128 (0): 16 ds_read_b128 row-fragment reads per wave and
 *       round (16 KB), the forward's K-fragment pattern;
 *   RSWA_PROBE_LDS_TR16 (1): 32 ds_read_b64_tr_b16 transposing reads per wave and
 *       round (16 KB), the forward's V^T pattern;
 *   RSWA_PROBE_EXP (2): 8 independent v_exp_f32 per wave and round;
 *   RSWA_PROBE_FMA (3): 8 independent v_fma_f32 per wave and round.
 * out: device uint32 [2 * workgroups]: out[2 g] = cycles of workgroup g,
 * out[2 g + 1] = a fold of its results (kept so the work is not optimised away).
 * LDS bytes per clock per CU = 8 waves * iters * 16 KB / cycles;
 * cycles per wave instruction per SIMD = cycles / (2 waves * iters * 8).
 * Returns RSWA_ERR_SHAPE for workgroups < 0, iters < 1 or an unknown kind.
 */
enum {
  RSWA_PROBE_LDS_B128 = 0,
  RSWA_PROBE_LDS_TR16 = 1,
  RSWA_PROBE_EXP = 2,
  RSWA_PROBE_FMA = 3
};
RSWA_API rswa_status_t rswa_probe_cu(uint32_t *out, int32_t workgroups, int32_t iters, int32_t kind,
                                     void *stream);

/*
 * Measurement helper, not part of the attention path: facts of HIP device
 * `device` as the runtime reports them, so that a measurement record can state
 * the hardware it ran on. Writes min(count, RSWA_FACT_COUNT) host int64 values
 * to `out`, indexed by the RSWA_FACT_* constants: compute units, LDS bytes per
 * compute unit, L2 bytes (as reported; one XCD's share on a multi-XCD part),
 * peak shader clock (kHz), peak memory clock (kHz), memory bus width (bits),
 * global memory bytes, wavefront size. Host-synchronous; enqueues nothing.
 * Returns RSWA_ERR_NULL for a NULL out, RSWA_ERR_SHAPE for device < 0 or
 * count < 1, RSWA_ERR_HIP when the runtime cannot report the device.
 */
enum {
  RSWA_FACT_COMPUTE_UNITS = 0,
  RSWA_FACT_LDS_BYTES_PER_CU = 1,
  RSWA_FACT_L2_BYTES = 2,
  RSWA_FACT_CLOCK_KHZ = 3,
  RSWA_FACT_MEM_CLOCK_KHZ = 4,
  RSWA_FACT_MEM_BUS_BITS = 5,
  RSWA_FACT_GLOBAL_MEM_BYTES = 6,
  RSWA_FACT_WAVE_SIZE = 7,
  RSWA_FACT_COUNT = 8
};
RSWA_API rswa_status_t rswa_device_facts(int32_t device, int64_t *out, int32_t count);

/*
 * Synchronise `stream`, read the cache's device error word into *flags
 * (RSWA_DEVERR_* bits, 0 = none) and clear it. Returns RSWA_ERR_STATE when a
 * bit was set, RSWA_OK otherwise.
 */
RSWA_API rswa_status_t rswa_check_device_error(const rswa_cache_t *cache, int32_t *flags, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* RSWA_H */
