/*
 * kvcache.h - C ABI of the MI355X (gfx950) quantized, paged KV cache library.
 *
 * The library implements the decode hot path of a KV cache kept in
 * block-quantized pages, as described on the KV-offload pages:
 *
 *   - Strata page: the hotelren.com article "KV 沉进内存、显存减半：Strata 让
 *     12 GB 显卡跑满 262K 上下文", sections "KV 从显存搬进内存之后发生了什么"
 *     (authoritative KV in pinned host memory, a residency table with CLOCK
 *     second-chance eviction, zero-copy page-in of missing pages, identical
 *     results), "4-bit KV 缓存：先旋转，再压到 4-bit" (256-point Walsh-Hadamard
 *     rotation of Q, K and V, 4-bit q4_0 blocks, output restored by H) and
 *     "三种 KV 格式横向对比" (int8, q4_0, k8v4).
 *   - VRAM wiki page: anozoder.com wiki "qwen38-27b-quant-vram-2026", section
 *     "一、为什么 256K 上下文的显存这么吓人" (GQA shape: 24 query heads, 4 KV
 *     heads, head_dim 256).
 *   - KV-offload news page: rebasdaily.com topic page on Qwen3.8-Flash-Next KV
 *     offload, section "缓存为何不能直接搬走？" (every decoded token re-reads the
 *     whole KV of each full-attention layer).
 *
 * Conventions for every entry point:
 *   - Return 0 (KV_OK) or a negative KV_E* status. On a non-zero status
 *     nothing has been enqueued and kv_last_error() describes the problem
 *     (thread-local, valid until the next call on the same thread).
 *   - Device work is enqueued asynchronously on `stream` (a hipStream_t,
 *     NULL = the default stream). Argument checks happen on the host before
 *     anything is enqueued.
 *   - The library allocates no device or host memory; every buffer belongs
 *     to the caller and must stay alive until the enqueued work completes.
 *     (One exception: the fixed device array of kv_decode_attention_noalloc,
 *     part of the library's code object, not allocated by any call.)
 *   - Pointers named "device" must be device memory (or device-accessible
 *     pinned host memory); pointers named "host" are read on the host during
 *     the call. Device buffers must be 16-byte aligned (KV_EALIGN otherwise).
 *
 * Byte layout of a page (fixed by this library; the pages name pages, blocks
 * and slots but no layout): a page holds 256 consecutive tokens of one
 * sequence and one layer, for every KV head h in order, the K plane of head h
 * then its V plane. Plane sizes: int8 67,584 B, q4 and fp4 36,864 B, fp8
 * 66,048 B, so a page is 540,672 B (int8), 294,912 B (q4_0, fp4), 417,792 B
 * (k8v4) or 528,384 B (fp8) for 4 KV heads. fp4 records use the q4 byte layout
 * below (4-bit codes, 8 fp16 scales); fp8 records the int8 byte layout (one byte
 * per code) with one fp16 scale per token (one scale row in the V plane).
 *   K plane (token-major): 256 code rows (256 B int8 / 128 B q4) then 256 rows
 *     of fp16 scales (4 int8 groups of 64 / 8 q4 blocks of 32). In a code row,
 *     the bytes of the eight 32-element blocks are split into four slices and
 *     slice-major: q4 byte 32s+4j+w = code[32j+4s+w] | code[32j+16+4s+w] << 4,
 *     int8 byte 64s+8j+w = code[32j+8s+w] (s = 0..3, j = block 0..7).
 *   V plane (element-major): 256 code rows, one per head element, holding that
 *     element for the 256 tokens (int8: byte t = token t; q4: byte 16G+i =
 *     code[token 32G+i] | code[token 32G+16+i] << 4), then one row of 256 fp16
 *     scales per group (int8, 4 rows) or block (q4, 8 rows).
 *
 * Record rules (readings; the pages fix the byte sizes and the rotation):
 *   int8 per 64 elements: d = fp16_rne(max|x| / 127), c = clamp(round half
 *     away from zero(x / d), -127, 127), d == 0 gives c = 0; value c * d.
 *   q4_0 per 32 elements of y = H x: m = the y of largest |y| (first index on
 *     ties), d = fp16_rne(-m / 8), c = clamp(floor(y / d + 1/2) + 8, 0, 15),
 *     d == 0 gives c = 8; value (c - 8) * d. H[i][j] = (-1)^popcount(i&j)/16.
 *   k8v4: K as int8 (not rotated), V as rotated q4_0.
 *   fp4 per 32 elements of y = H x (a declared block-scaled 4-bit float format;
 *     smzdm roundup post.smzdm.com/p/ad79lwwz, section "一、先修正一笔老账", lists
 *     NVFP4 KV at the same 144 B per vector): a = max|y|; a == 0 gives d = 0 and
 *     c = 0; else d = 2^e, e = clamp(floor(log2 a) - 2, -23, 13) (stored as an
 *     exact fp16); c = the e2m1 grid index (values 0, .5, 1, 1.5, 2, 3, 4, 6) of
 *     |y| / d rounded to nearest, ties to the even index, saturating at 6, plus
 *     8 when y < 0 and the index is not 0; value +-grid[c & 7] * d.
 *   fp8 per vector, not rotated (a declared block-scaled 8-bit float format; the
 *     same roundup section lists FP8 KV at 516 B per position, 258 B per vector):
 *     d = fp16_rne(max|x| / 448), d == 0 gives c = 0; else c = the OCP E4M3 code
 *     (1 sign, 4 exponent bits of bias 7, 3 mantissa bits; 0x7F / 0xFF are NaN
 *     and never written) of |x| / d rounded to nearest, ties to the even code,
 *     beyond 448 to 448, with the sign bit when x < 0 and the magnitude is not
 *     0; value +-E4M3(c) * d.
 */
#ifndef KVCACHE_H
#define KVCACHE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define KV_OK            0
#define KV_EINVAL       (-1)  /* an argument is out of range or inconsistent      */
#define KV_EUNSUPPORTED (-2)  /* a shape this library does not implement          */
#define KV_EALIGN       (-3)  /* a device buffer is not 16-byte aligned           */
#define KV_ENOSLOTS     (-4)  /* a selection is larger than the slot pool         */
#define KV_EHIP         (-5)  /* the HIP runtime reported an error                */
#define KV_ESMALL       (-6)  /* a caller-provided buffer is too small            */

/* Device status bits OR-ed into a status word by kernels that find bad data
 * they cannot report synchronously (see kv_decode_attention). */
#define KV_STATUS_BAD_PAGE_ID     1  /* a block-table entry outside the pool: page skipped */
#define KV_STATUS_CONTEXT_CLAMPED 2  /* a context length above its bound: clamped            */

/* KV formats (Strata page, section "三种 KV 格式横向对比"). */
#define KV_FMT_INT8 0  /* K and V int8, per-64 fp16 scales, 264 B per vector        */
#define KV_FMT_Q4_0 1  /* K and V rotated by H, q4_0 blocks, 144 B per vector       */
#define KV_FMT_K8V4 2  /* K int8 (unrotated), V rotated q4_0: 408 B per KV head      */
#define KV_FMT_FP4  3  /* K and V rotated by H, e2m1 codes, 2^e block scales, 144 B   */
#define KV_FMT_FP8  4  /* K and V E4M3 codes, one fp16 scale per vector, 258 B       */

/* Shape of one layer's cache. Supported: head_dim == 256, page_tokens == 256,
 * n_kv_heads >= 1, n_q_heads a multiple of n_kv_heads with at most 8 query
 * heads per KV head. */
typedef struct kv_shape {
  int32_t n_q_heads;    /* e.g. 24 */
  int32_t n_kv_heads;   /* e.g. 4  */
  int32_t head_dim;     /* 256     */
  int32_t page_tokens;  /* 256     */
  int32_t format;       /* KV_FMT_* */
} kv_shape;

/* Thread-local text of the last non-zero status. Never NULL. */
const char* kv_last_error(void);

/* Library version as "major.minor.patch". */
const char* kv_version(void);

/* Bytes of one page for `shape` (int8 540672, q4_0 and fp4 294912, k8v4 417792,
 * fp8 528384 for 4 KV heads), or a negative status if the shape is invalid or
 * unsupported. */
int64_t kv_page_bytes(const kv_shape* shape);

/*
 * kv_append_quantize - quantize-on-append (Strata page, section "4-bit KV
 * 缓存：先旋转，再压到 4-bit": K and V are rotated and stored as q4_0 blocks as
 * they are written; section "三种 KV 格式横向对比" for int8 and k8v4; the fp4 and
 * fp8 records follow the rules above).
 *
 * Writes the records of tokens [start_pos, start_pos + n_tokens) of one
 * sequence into its pages: token p goes to page block_table[p / 256], row
 * p % 256. Every code and scale is bit-exact to the record rules above
 * (the rotation is computed exactly, in fp64).
 *
 *   k, v         device fp16 [n_tokens][n_kv_heads][256], token-major, finite
 *                (codes of a vector holding Inf or NaN are unspecified).
 *   block_table  device int32 [n_table]: physical page id of each logical
 *                page of the sequence; n_table * 256 >= start_pos + n_tokens.
 *   pool         device (or device-accessible pinned host) base of the page
 *                pool, n_pool_pages pages of kv_page_bytes() each. A page id
 *                outside [0, n_pool_pages) is skipped and, if `status` is not
 *                NULL, KV_STATUS_BAD_PAGE_ID is OR-ed into *status (device).
 *   status       device int32 or NULL.
 * Only the rows of the appended tokens change (a q4 V code byte shared with
 * another token keeps that token's nibble). Appends to the same page from
 * several calls must be ordered on one stream.
 */
int kv_append_quantize(const kv_shape* shape, const void* k, const void* v,
                       int64_t n_tokens, int64_t start_pos,
                       const int32_t* block_table, int32_t n_table,
                       void* pool, int64_t n_pool_pages,
                       int32_t* status, void* stream);

/*
 * kv_append_quantize with measurement events: identical work and checks, and the
 * append kernel is launched with hipExtLaunchKernelGGL so that `start_event` and
 * `stop_event` (hipEvent_t created by the caller, may be NULL) are recorded when the
 * kernel itself starts and ends on `stream` (its duration without the queueing gap in
 * front of it, as a kernel trace reports it). Nothing is recorded for n_tokens == 0.
 */
int kv_append_quantize_timed(const kv_shape* shape, const void* k, const void* v,
                             int64_t n_tokens, int64_t start_pos,
                             const int32_t* block_table, int32_t n_table,
                             void* pool, int64_t n_pool_pages,
                             int32_t* status, void* stream,
                             void* start_event, void* stop_event);

/*
 * kv_decode_workspace_bytes - bytes of workspace kv_decode_attention needs
 * for `batch` sequences of at most `max_context` tokens, with the given
 * pages_per_split (0 = the library's choice, as in kv_decode_attention).
 * Returns 0 for invalid arguments (see kv_last_error()).
 */
size_t kv_decode_workspace_bytes(const kv_shape* shape, int32_t batch,
                                 int64_t max_context, int32_t pages_per_split);

/*
 * kv_decode_attention - GQA decode attention over the paged, quantized
 * cache (KV-offload news page, section "缓存为何不能直接搬走？": a decode step
 * reads the whole KV of the layer; Strata page, section "4-bit KV 缓存：先旋转，
 * 再压到 4-bit": with rotated K the query is rotated by H first, and with
 * rotated V the output is multiplied by H).
 *
 * For each sequence b and query head h (KV head g = h / (n_q_heads /
 * n_kv_heads)), over its T = context_lens[b] tokens:
 *   q' = H q if K is rotated (q4_0, fp4) else q;  s_t = softmax_scale * <q', k^_t>;
 *   o' = sum_t softmax(s)_t v^_t;  out = H o' if V is rotated (q4_0, k8v4, fp4).
 * k^ and v^ are the dequantized records. T == 0 gives a zero output.
 * The work is split along the context ("split-K"): each split of
 * pages_per_split pages writes a partial (max, sum, weighted values) that a
 * second kernel combines with the log-sum-exp rule (partials of rotated V are
 * rotated back by the first kernel; H is linear, so this equals H o').
 * The arithmetic order depends only on logical token order, never on the
 * physical page ids, so results do not depend on where pages are placed.
 *
 *   q              device fp16 [batch][n_q_heads][256].
 *   pool           device base of n_pool_pages pages.
 *   block_tables   device int32 [batch][max_pages]; entries past the last
 *                  page of a sequence are not read.
 *   context_lens   device int32 [batch]; each must be <= max_context and
 *                  <= max_pages * 256 (larger values are clamped and flagged).
 *   max_context    host bound on every context length (sizes the split grid).
 *   softmax_scale  e.g. 1/16 = 1/sqrt(256).
 *   out            device fp32 [batch][n_q_heads][256].
 *   workspace      device, >= kv_decode_workspace_bytes() bytes. Its first
 *                  16 bytes must be zero before the first call (e.g. once,
 *                  right after allocation). The first int32 is a status word
 *                  into which the kernels OR KV_STATUS_* bits; the caller may
 *                  read and clear it. Bytes 4..11 are work counters that a
 *                  call leaves at zero again when it ends; calls that use one
 *                  workspace must therefore not overlap (same stream, or
 *                  ordered by events).
 *   pages_per_split  pages per split (>= 1), or 0 for the library's choice.
 */
int kv_decode_attention(const kv_shape* shape, const void* q, int32_t batch,
                        const void* pool, int64_t n_pool_pages,
                        const int32_t* block_tables, int32_t max_pages,
                        const int32_t* context_lens, int64_t max_context,
                        float softmax_scale, float* out,
                        void* workspace, size_t workspace_bytes,
                        int32_t pages_per_split, void* stream);

/*
 * kv_decode_attention_noalloc - kv_decode_attention for callers that cannot allocate
 * device memory: code being recorded into a HIP graph, tight serving loops, and
 * harnesses that forbid allocation. The same kernels and the same result, bit for
 * bit, as kv_decode_attention with the same arguments, but the split partials and
 * work counters live in a device array of the library (KV_NOALLOC_SCRATCH_BYTES per
 * GPU, held until the process ends) instead of a caller workspace. The call itself
 * allocates nothing.
 *
 *   status   device int32 or NULL: KV_STATUS_* bits are OR-ed into it (as into a
 *            workspace's status word); NULL = not reported.
 * Every other argument is that of kv_decode_attention. The array of the current
 * device (hipGetDevice, which must be the device of `stream`) is used; its address
 * is looked up on the first call on each device, which also enqueues a small
 * kernel that clears its header. Returns KV_ESMALL, enqueuing nothing, when the
 * partials would need more than KV_NOALLOC_SCRATCH_BYTES (that is, when
 * kv_decode_workspace_bytes for the same arguments exceeds it). All calls on one
 * GPU share the array and the last call's partials stay in it: calls that overlap
 * on one GPU (unordered streams, or other threads) race and give wrong results.
 */
#define KV_NOALLOC_SCRATCH_BYTES 16777216
int kv_decode_attention_noalloc(const kv_shape* shape, const void* q, int32_t batch,
                                const void* pool, int64_t n_pool_pages,
                                const int32_t* block_tables, int32_t max_pages,
                                const int32_t* context_lens, int64_t max_context,
                                float softmax_scale, float* out, int32_t* status,
                                int32_t pages_per_split, void* stream);

/*
 * kv_decode_mq_workspace_bytes - bytes of workspace kv_decode_attention_mq needs for
 * `batch` sequences of n_q queries each and at most `max_context` tokens, with the
 * given pages_per_split (0 = the library's choice): kv_decode_workspace_bytes for
 * batch * n_q sequences. Returns 0 for invalid arguments.
 */
size_t kv_decode_mq_workspace_bytes(const kv_shape* shape, int32_t batch, int32_t n_q,
                                    int64_t max_context, int32_t pages_per_split);

/*
 * kv_decode_attention_mq - causal attention of each sequence's n_q newest tokens
 * over the paged, quantized cache: the verification step of speculative decoding
 * (smzdm roundup, post.smzdm.com/p/ad79lwwz, section "二、一周跨卡实测": MTP
 * drafts of up to 3 tokens checked in one pass) and chunked prompt reading
 * (prefill rates in the same table; Strata page, section "三种 KV 格式横向对比":
 * prompt reading over the quantized formats).
 *
 * The n_q tokens must already be in the cache (kv_append_quantize of the chunk):
 * with T = context_lens[b], query j (0 <= j < n_q) of sequence b sits at position
 * T - n_q + j and attends to tokens 0 .. T - n_q + j, i.e. it is exactly
 * kv_decode_attention with context length T - n_q + j + 1 (0 if that is < 1,
 * which gives a zero output). n_q = 1 is kv_decode_attention.
 *
 *   q              device fp16 [batch][n_q][n_q_heads][256].
 *   out            device fp32 [batch][n_q][n_q_heads][256].
 *   workspace      as for kv_decode_attention, of at least
 *                  kv_decode_mq_workspace_bytes(shape, batch, n_q, max_context,
 *                  pages_per_split) bytes.
 *   pages_per_split  pages per split, or 0 for the library's choice for this call.
 * Every other argument is that of kv_decode_attention (block_tables and
 * context_lens have one row / entry per sequence). batch * n_q must be at most
 * 65535. Each query is a row of the decode path's split-K kernel (row b * n_q + j,
 * with the context its position allows); the rows of one sequence read the same
 * pages at about the same time, so repeated reads are mostly served by the caches.
 */
int kv_decode_attention_mq(const kv_shape* shape, const void* q, int32_t batch, int32_t n_q,
                           const void* pool, int64_t n_pool_pages,
                           const int32_t* block_tables, int32_t max_pages,
                           const int32_t* context_lens, int64_t max_context,
                           float softmax_scale, float* out,
                           void* workspace, size_t workspace_bytes,
                           int32_t pages_per_split, void* stream);

/*
 * The pages per split that pages_per_split = 0 selects, for `batch` sequences of at
 * most `max_context` tokens whose lengths add up to `total_context` (0: assume every
 * sequence at max_context). The split count is chosen so that the grid about fills
 * the GPU once; for a batch of very unequal lengths, passing its total here and the
 * result as pages_per_split keeps the GPU full where the default would not.
 * Returns >= 1, or 0 (kv_last_error) for an invalid shape or size.
 */
int32_t kv_decode_split_pages(const kv_shape* shape, int32_t batch, int64_t max_context,
                              int64_t total_context);

/*
 * The two phases of kv_decode_attention, for callers that schedule them
 * separately (e.g. to time or overlap them). Same arguments and checks as
 * kv_decode_attention; kv_decode_split enqueues only the split-K kernel
 * (partials into the workspace), kv_decode_combine only the log-sum-exp
 * combine (partials to `out`). Calling them in this order
 * on one stream with identical arguments is exactly kv_decode_attention.
 */
int kv_decode_split(const kv_shape* shape, const void* q, int32_t batch,
                    const void* pool, int64_t n_pool_pages,
                    const int32_t* block_tables, int32_t max_pages,
                    const int32_t* context_lens, int64_t max_context,
                    float softmax_scale, float* out,
                    void* workspace, size_t workspace_bytes,
                    int32_t pages_per_split, void* stream);
int kv_decode_combine(const kv_shape* shape, const void* q, int32_t batch,
                      const void* pool, int64_t n_pool_pages,
                      const int32_t* block_tables, int32_t max_pages,
                      const int32_t* context_lens, int64_t max_context,
                      float softmax_scale, float* out,
                      void* workspace, size_t workspace_bytes,
                      int32_t pages_per_split, void* stream);

/*
 * kv_decode_split with measurement events: identical work and checks, and the
 * kernel is launched with hipExtLaunchKernelGGL so that `start_event` and
 * `stop_event` (hipEvent_t created by the caller, may be NULL) are recorded
 * when the split-K kernel itself starts and ends on `stream`. The elapsed time
 * between them is the kernel's duration without the queueing gap in front of
 * it, which is what a kernel trace reports.
 */
int kv_decode_split_timed(const kv_shape* shape, const void* q, int32_t batch,
                          const void* pool, int64_t n_pool_pages,
                          const int32_t* block_tables, int32_t max_pages,
                          const int32_t* context_lens, int64_t max_context,
                          float softmax_scale, float* out,
                          void* workspace, size_t workspace_bytes,
                          int32_t pages_per_split, void* stream,
                          void* start_event, void* stop_event);

/*
 * kv_append_decode - one decode step of one layer: append one token per
 * sequence, then attend (Strata page, section "4-bit KV 缓存：先旋转，再压到
 * 4-bit": K and V are rotated and quantized as they are written; KV-offload
 * news page, section "缓存为何不能直接搬走？": the step then reads the whole
 * cache of the layer).
 *
 * Equivalent, byte for byte in the pool and bit for bit in `out`, to
 * kv_append_quantize of token T_b - 1 of every sequence b (T_b =
 * context_lens[b], its block table row) followed by kv_decode_attention with
 * the same arguments. The append is done inside the split-K kernel by the
 * workgroup whose split holds the token's page, before that page is read, so
 * the step takes two launches instead of three.
 *
 *   k_new, v_new   device fp16 [batch][n_kv_heads][256]: the token's K and V
 *                  (finite values).
 *   pool           device, writable (the token's row of its page is written).
 *   start_event, stop_event  hipEvent_t or NULL: recorded at the start and
 *                  end of the split-K kernel (as in kv_decode_split_timed).
 * Every other argument is that of kv_decode_attention. A sequence whose
 * context length is 0 or out of range appends nothing (the range case sets
 * KV_STATUS_CONTEXT_CLAMPED); a token page id outside the pool appends nothing
 * and sets KV_STATUS_BAD_PAGE_ID. Calls that share a workspace must not
 * overlap.
 */
int kv_append_decode(const kv_shape* shape, const void* k_new, const void* v_new,
                     const void* q, int32_t batch, void* pool, int64_t n_pool_pages,
                     const int32_t* block_tables, int32_t max_pages,
                     const int32_t* context_lens, int64_t max_context,
                     float softmax_scale, float* out, void* workspace,
                     size_t workspace_bytes, int32_t pages_per_split, void* stream,
                     void* start_event, void* stop_event);

/*
 * Residency table of one layer's device page slots (Strata page, section
 * "KV 从显存搬进内存之后发生了什么": a residency table with CLOCK second-chance
 * eviction). Plain host memory owned by the caller:
 *   slot_page[n_slots]  logical page held by each slot, -1 = empty
 *   page_slot[n_pages]  slot holding each logical page, -1 = not resident
 *   ref[n_slots]        second-chance reference bits
 *   hand                next slot the clock hand inspects
 */
typedef struct kv_residency {
  int32_t n_slots;
  int32_t n_pages;
  int32_t* slot_page;
  int32_t* page_slot;
  uint8_t* ref;
  int32_t hand;
} kv_residency;

/* Marks every slot empty, every page non-resident, clears the reference bits
 * and puts the hand at slot 0. */
int kv_residency_reset(kv_residency* table);

/*
 * kv_residency_select - one step of the CLOCK table (host only, no GPU).
 * For an ordered selection of n_sel distinct logical pages (n_sel <= n_slots,
 * else KV_ENOSLOTS): first every resident selected page gets ref = 1 and is
 * pinned for the step; then each missing page, in order, takes the slot the
 * hand finds (empty; else not pinned with ref = 0, clearing ref = 1 bits on
 * the way), is installed with ref = 1, pinned, the hand moved past it.
 *   out_slots   host int32 [n_sel]: the slot of every selected page, in order.
 *   miss_pages  host int32 [n_sel] (may be NULL): the missing pages in order,
 *   miss_slots  host int32 [n_sel] (may be NULL): the slot each went to,
 *   n_miss      host int32 (may be NULL): how many pages were missing.
 * On error the table is unchanged.
 */
int kv_residency_select(kv_residency* table, const int32_t* selection, int32_t n_sel,
                        int32_t* out_slots, int32_t* miss_pages, int32_t* miss_slots,
                        int32_t* n_miss);

/*
 * kv_gather_pages - page-in of one layer's selected pages (Strata page,
 * section "KV 从显存搬进内存之后发生了什么": before attention the selected
 * blocks are looked up in the residency table and missing pages are copied
 * zero-copy over PCIe from pinned host memory into device slots).
 *
 * Runs kv_residency_select on `table`, then enqueues one kernel that reads
 * every missing page directly from `host_pool` (pinned, device-accessible:
 * allocated with hipHostMalloc or torch pin_memory) and writes it to its slot
 * of `slot_pool`, and writes the slot of every selected page, in selection
 * order, to `out_block_table` (device int32 [n_sel]) - the block table that
 * kv_decode_attention then reads. Page bytes are copied verbatim, so
 * attention over gathered slots equals attention over the host pages.
 *
 *   host_pool        n_pages (= table->n_pages) pages of kv_page_bytes().
 *   slot_pool        device, table->n_slots pages.
 *   out_n_miss       host int32 or NULL.
 * The host pages must not change until the enqueued copy completes.
 */
int kv_gather_pages(const kv_shape* shape, kv_residency* table,
                    const int32_t* selection, int32_t n_sel,
                    const void* host_pool, void* slot_pool,
                    int32_t* out_block_table, int32_t* out_n_miss, void* stream);

/*
 * kv_gather_pages_layers - the page-in of several layers' selections in one
 * launch (each layer has its own residency table, pools and block table; the
 * Strata page's streaming step, section "KV 从显存搬进内存之后发生了什么", done
 * for a whole set of layers whose selections are known together).
 *
 * For each layer l: kv_residency_select on tables[l] with the n_sel pages at
 * selections[l * n_sel] (host int32); then one kernel copies every missing
 * page of every layer from host_pools[l] (pinned, device-accessible) to its
 * slot of slot_pools[l] (device), and writes each layer's slot block table to
 * out_block_tables[l * n_sel .. +n_sel) (device int32 [n_layers][n_sel]).
 * The result is that of kv_gather_pages called for each layer in turn.
 *   tables         host array of n_layers tables.
 *   host_pools, slot_pools  host arrays of n_layers pointers.
 *   out_n_miss     host int32 [n_layers] or NULL.
 * All arguments are checked before any table changes. The host pages must not
 * change until the enqueued copies complete.
 */
int kv_gather_pages_layers(const kv_shape* shape, int32_t n_layers, kv_residency* tables,
                           const int32_t* selections, int32_t n_sel,
                           const void* const* host_pools, void* const* slot_pools,
                           int32_t* out_block_tables, int32_t* out_n_miss, void* stream);

/*
 * kv_gather_pages_layers_timed - kv_gather_pages_layers, with `start_event` and
 * `stop_event` (hipEvent_t, each may be NULL) recorded by the copy launches
 * themselves: the start event at the start of the first copy kernel, the stop
 * event at the end of the last one. Their elapsed time is the time the copies
 * take on the GPU, without the host's CLOCK step or the launch in front of them
 * (a PCIe rate, as a kernel trace reports it). Nothing is recorded when
 * n_layers or n_sel is 0. Every other argument and all behaviour are those of
 * kv_gather_pages_layers.
 */
int kv_gather_pages_layers_timed(const kv_shape* shape, int32_t n_layers, kv_residency* tables,
                                 const int32_t* selections, int32_t n_sel,
                                 const void* const* host_pools, void* const* slot_pools,
                                 int32_t* out_block_tables, int32_t* out_n_miss, void* stream,
                                 void* start_event, void* stop_event);

/*
 * Page selection for streaming mode (KV-offload news page, section
 * "新招不是全搬，而是分层放": attention over a fixed budget of selected tokens,
 * whose selection rule the page does not give; this library declares the
 * plain rule below). The key sums are exact integers and each page
 * representative one rounding of an exact value, so the result does not
 * depend on summation order and is the same on every call.
 *
 * kv_page_key_sums - adds tokens [start_pos, start_pos + n_tokens) of one
 * sequence to its per-page key sums and rounds the page representatives:
 *   sums[p][g][e] += k[t][g][e] * 2^24 for every token t of logical page p
 *   reps[p][g][e]  = sums[p][g][e] / 2^32 rounded once to fp16 (nearest, ties
 *                    to even): the page's key sum over 256, for every page p
 *                    the call adds tokens to
 * (fp16 keys are integer multiples of 2^-24, so each term is an exact integer;
 * a page's sum stays below 2^48 and its representative within fp16 range).
 *   k       device fp16 [n_tokens][n_kv_heads][256] (the keys as appended).
 *   sums    device int64 [n_pages_cap][n_kv_heads][256], zero before the
 *           first token of each page is added. Atomic adds: the sums of calls
 *           that overlap are exact.
 *   reps    device fp16 [n_pages_cap][n_kv_heads][256]; each element is
 *           rounded from the sum the call's own add produced, so calls that
 *           add to the same page must be ordered (one stream) for the
 *           representatives to be those of the final sums.
 *
 * kv_select_pages - the pages one step attends, for n_sets independent sets
 * (layers, or sequences of equal page count) in one call. For set i:
 *   score[p] = sum over KV heads g and elements e of
 *              (sum over g's query heads h of q[i][h][e] * 2^24) * reps[i][p][g][e] * 2^24
 * (an exact 128-bit integer); the selection is the last page (p = n_pages - 1,
 * the newest tokens) and the k_sel - 1 other pages of largest score, ties to
 * the lower page index, written in ascending order to out_selection[i] (device
 * int32 [n_sets][k_sel]; the first min(k_sel, n_pages) entries); with
 * n_pages <= k_sel, every page. It reads 512 B per page and KV head.
 *   q          device fp16 [n_sets][n_q_heads][256] (each set's query).
 *   reps       device fp16 [n_sets][reps_pages][n_kv_heads][256], 16-B aligned,
 *              reps_pages >= n_pages (as kv_page_key_sums writes them).
 *   n_pages    pages of the context (<= 32768); k_sel in 1..256; at most 8 KV heads.
 *   workspace  device, >= kv_select_workspace_bytes(n_pages, n_sets) bytes, 16-B aligned.
 */
int kv_page_key_sums(const kv_shape* shape, const void* k, int64_t n_tokens, int64_t start_pos,
                     int64_t* sums, void* reps, int64_t n_pages_cap, void* stream);
size_t kv_select_workspace_bytes(int64_t n_pages, int32_t n_sets);
int kv_select_pages(const kv_shape* shape, const void* q, const void* reps, int64_t reps_pages,
                    int64_t n_pages, int32_t k_sel, int32_t n_sets, int32_t* out_selection,
                    void* workspace, size_t workspace_bytes, void* stream);

/* Host-side helpers of the record rules, exposed so the rounding can be
 * checked without a GPU. Not part of the hot path.
 *   kv_host_f64_to_f16: round a double to fp16 bits once, nearest-even.
 *   kv_host_encode_vector: record of one fp16 vector x[256] (raw fp16 bits)
 *     as the append kernel writes it: kind 0 = int8 (codes int8 x256,
 *     scales fp16 x4), kind 1 = q4 of H x (codes 0..15 x256, scales x8),
 *     kind 2 = fp4 of H x (codes 0..15 x256, power-of-two scales x8),
 *     kind 3 = fp8 (E4M3 codes x256, one scale). */
uint16_t kv_host_f64_to_f16(double x);
int kv_host_encode_vector(int32_t kind, const uint16_t* x, uint8_t* codes, uint16_t* scales);

#ifdef __cplusplus
}
#endif

#endif /* KVCACHE_H */
