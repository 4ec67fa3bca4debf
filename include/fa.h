/*
 * fa.h - fused exact attention forward and backward for AMD MI355X (gfx950).
 *
 * The library computes, for every batch b and query head hq,
 *
 *     O   = softmax(scale * Q K^T + mask) V
 *     lse = log(sum_j exp(scale * q_i . k_j))   over the visible keys j
 *
 * without ever writing the Nq x Nk score or probability matrices to memory.
 * The algorithm is the tiled online softmax ("FlashAttention Analysis",
 * ryotta.opik.net, section 3 "Tiling + Online Softmax"): a block of query
 * rows stays on chip while K/V blocks stream through it, a running row max
 * m and running sum l are kept, the partial output is rescaled by
 * exp(m_old - m_new) when the max grows, and O is divided by l once at the
 * end.  One fp32 logsumexp per query row is written for a
 * recomputation-based backward pass (FlashAttention version/GPU/training-
 * cost guide, tool.smithlab.co.kr, section on attention memory during
 * training).  The KV-split entry point is the Flash-Decoding form (same
 * "FlashAttention Analysis" page, "Flash-Decoding" paragraph): chunks of
 * the key axis are processed in parallel and merged by a log-sum-exp
 * reduction.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *   aligned, contiguous, head dimension fastest:
 *       q   [B, Hq,  Nq, d]  bf16
 *       k,v [B, Hkv, Nk, d]  bf16
 *       o   [B, Hq,  Nq, d]  bf16 (FA_OUT_BF16) or fp32 (FA_OUT_F32)
 *       lse [B, Hq,  Nq]     fp32, natural log
 * - Grouped-query attention: query head hq reads KV head hq / (Hq / Hkv);
 *   Hq must be a multiple of Hkv (Hkv == Hq is plain multi-head attention).
 *   The KV head count is passed instead of replicating K/V (cost guide,
 *   adoption checklist).
 * - causal != 0 hides key j from query i when j > i + (Nk - Nq): the mask is
 *   aligned at the last key, which is the usual lower triangle when
 *   Nq == Nk and lets a single query see every key.  A query row that sees
 *   no key at all (only possible when causal and Nq > Nk) gets O = 0 and
 *   lse = -inf.
 * - scale must be finite and >= 0 (1/sqrt(d) is the usual value).
 * - Head dimensions by entry point:
 *     fa_fwd, fa_fwd_noalloc, fa_fwd_window      32, 64, 96, 128, 256
 *     fa_fwd_varlen, fa_fwd_strided,
 *     fa_fwd_block_sparse, fa_fwd_colmask        32, 64, 96, 128
 *     fa_fwd_paged, fa_fwd_kvlen                 32, 64, 96, 128, 256
 *     fa_fwd_splitkv                             32, 64, 128, 256
 *     fa_bwd, fa_bwd_window                      64, 128
 *     fa_fwd_fp8                                 128
 *   32 and 96 run in the 64- and 128-column tiles of the prefill kernel
 *   with the columns past d masked, 256 in a prefill kernel of its own (one
 *   wave per SIMD); fa_fwd, fa_fwd_window, fa_fwd_paged and fa_fwd_kvlen
 *   take d = 96 only in the prefill form, and fa_fwd_paged takes d = 256
 *   only in the KV-split form.
 * - Every call is asynchronous: it validates its arguments on the host,
 *   enqueues kernels on `stream` and returns.  Results are valid once the
 *   stream has been synchronised; buffers must stay alive until then.
 * - Results are deterministic: repeated calls with the same arguments give
 *   bitwise identical outputs (fixed reduction orders, no float atomics).
 *
 * Errors
 * ------
 * Every entry point returns a status code.  All argument checks happen
 * before any HIP call, and nothing is written when a check fails.
 *   FA_ERR_INVALID_ARG  null or misaligned pointer, a size < 1, Hq not a
 *                       multiple of Hkv, scale not finite or negative, bad
 *                       out_dtype, workspace too small, num_splits < 1.
 *   FA_ERR_UNSUPPORTED  d not taken by the entry point (list above),
 *                       sizes beyond the 64-bit/grid limits or the 32-bit
 *                       per-head K/V range of the prefill form, or the
 *                       current device is not gfx950.
 *   FA_ERR_TOO_LARGE    (fa_fwd_noalloc only) the call needs more scratch
 *                       than the library's fixed scratch array holds.
 *   FA_ERR_HIP          a HIP runtime or launch error; the hipError_t is
 *                       available from fa_last_hip_error() on the same
 *                       thread.  Outputs are then undefined.
 * No C++ exception crosses this interface.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = 1,
  FA_ERR_UNSUPPORTED = 2,
  FA_ERR_HIP = 3,
  FA_ERR_TOO_LARGE = 4
};

enum { FA_OUT_BF16 = 0, FA_OUT_F32 = 1 };

/*
 * Attention forward.  Picks the execution form by shape: the tiled prefill
 * kernel (a workgroup per block of 256 query rows of one head) when there
 * are enough query rows to fill the GPU, otherwise the KV-split form with
 * fa_default_num_splits() chunks.  Both forms address one K or V head
 * with 32-bit byte offsets, so Nk * d * 2 must stay below 2^31
 * (FA_ERR_UNSUPPORTED otherwise; Nk < 8388608 at d = 128).  The KV-split
 * form needs an fp32 workspace (fa_splitkv_workspace_bytes).  The library
 * keeps one per (device, stream) for the later calls on that stream (calls
 * on one stream run in order), grown with hipFreeAsync / hipMallocAsync on
 * the stream when a call needs more, and held until the process ends;
 * under graph capture, or once 32 streams hold one, a call takes its own
 * with hipMallocAsync and returns it with hipFreeAsync on `stream`.
 * `stream` may be NULL (the null stream).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
           float scale, int out_dtype, hipStream_t stream);

/*
 * fa_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, choice of form, results and errors as fa_fwd, bit for
 * bit; it never calls hipMalloc, hipMallocAsync, hipFree or any allocating
 * routine.  When the KV-split form is chosen, its partials go to a
 * fixed-size scratch array inside the library (one per device, held until
 * the process ends), so:
 *   - a call whose partials need more than fa_noalloc_scratch_bytes()
 *     bytes (fa_splitkv_workspace_bytes at fa_default_num_splits chunks)
 *     returns FA_ERR_TOO_LARGE before any HIP call;
 *   - calls that overlap on one device (e.g. on two streams) share that
 *     array and race: serialise them.
 * The prefill form uses no scratch at all.
 */
int fa_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   int causal, float scale, int out_dtype, hipStream_t stream);

/* Size in bytes of the scratch array behind fa_fwd_noalloc (16 MiB). */
size_t fa_noalloc_scratch_bytes(void);

/*
 * KV-split (Flash-Decoding) forward with a caller-owned workspace.
 * The key axis is cut into `num_splits` chunks of whole 32-key blocks; each
 * (batch, KV head, chunk) computes unnormalised partial results for all
 * Hq/Hkv query heads of the group and all Nq queries, and a second kernel
 * merges the chunks in chunk order by the log-sum-exp rule.  Chunks that
 * hold no key (num_splits larger than the number of 32-key blocks) weigh
 * nothing.  `workspace` is a device buffer of at least
 * fa_splitkv_workspace_bytes(B, Hq, Nq, d, num_splits) bytes, 16-byte
 * aligned; its contents on entry do not matter and on return are scratch.
 * num_splits must be in [1, 4096].  Nk * d * 2 must stay below 2^31, as
 * for fa_fwd (FA_ERR_UNSUPPORTED otherwise).  d may be 32, 64, 128 or
 * 256.
 */
size_t fa_splitkv_workspace_bytes(int B, int Hq, int Nq, int d,
                                  int num_splits);

int fa_fwd_splitkv(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   int causal, float scale, int out_dtype, int num_splits,
                   void* workspace, size_t workspace_bytes,
                   hipStream_t stream);

/*
 * The number of chunks fa_fwd uses for the KV-split form at this shape, or
 * 0 when fa_fwd uses the prefill kernel instead.  Pure host arithmetic; no
 * HIP call.  Returns 0 for invalid sizes as well.
 */
int fa_default_num_splits(int B, int Hq, int Hkv, int Nq, int Nk, int d);

/*
 * Forward on FP8 inputs ("FlashAttention-2 (KO)", systems-analysis.info,
 * comparison with later versions: 8-bit floating point for extra speed;
 * "FlashAttention Analysis", ryotta.opik.net, evolution by generation:
 * FlashAttention-3's FP8 low-precision path).  Inputs are OCP FP8 E4M3
 * codes (1 byte each) with one fp32 descale factor per (batch, head); the
 * real inputs are code value * descale:
 *     q  [B, Hq,  Nq, d]      q_descale [B, Hq]    (DEVICE, fp32, > 0)
 *     k  [B, Hkv, Nk, d]      k_descale [B, Hkv]
 *     vt [B, Hkv, d, ldv]     v_descale [B, Hkv]   (V TRANSPOSED)
 *     o  [B, Hq,  Nq, d] bf16 or fp32, lse [B, Hq, Nq] fp32
 * ldv >= Nk is a multiple of 64; keys Nk .. ldv - 1 of vt are padding and
 * must hold finite codes (they get zero weight).  Mask, GQA mapping and
 * scale as for fa_fwd; d must be 128.  Both products run on the 8-bit
 * matrix cores: S = scale q k^T from the E4M3 codes, and P V with the
 * weights rounded to E4M3 (normalised by the fp32 sum of the unrounded
 * weights), so O carries the error of 8-bit weights (a relative 2^-4 per
 * weight) on top of the inputs' own quantisation; lse is computed in fp32
 * from the unrounded weights.  Errors as for fa_fwd; FA_ERR_INVALID_ARG
 * also for null or misaligned descale arrays or a bad ldv;
 * FA_ERR_UNSUPPORTED for d != 128.
 */
int fa_fwd_fp8(const void* q, const void* k, const void* vt,
               const float* q_descale, const float* k_descale,
               const float* v_descale, void* o, float* lse, int B, int Hq,
               int Hkv, int Nq, int Nk, int ldv, int d, int causal,
               float scale, int out_dtype, hipStream_t stream);

/*
 * Forward with a sliding-window mask (the training-cost guide,
 * tool.smithlab.co.kr, FAQ: sliding windows are among the mask features of
 * the fused kernels).  Query i, placed at c = i + Nk - Nq on the key axis
 * (the bottom-right alignment of the causal mask), sees key j only if
 *     c - window_left <= j <= c + window_right,
 * and, with `causal` set, j <= c as well.  A bound of -1 is no bound on
 * that side: (-1, -1) is fa_fwd without a mask, (-1, 0) or the causal flag
 * alone is fa_fwd causal, and those cases (and windows that hide nothing,
 * left >= Nk - 1 and right >= Nq - 1) are run by fa_fwd itself, KV split
 * included.  Otherwise the kernel fa_fwd would choose for the shape runs
 * with the band: the tiled prefill kernel, where K/V blocks outside every
 * row's window of a 256-row block are never read, or, when few query rows
 * share a KV head (decode), the KV-split form with its chunks cut from the
 * keys a row tile's window can reach (the last window_left + 1 keys for a
 * single query), its workspace taken from the stream-ordered pool.
 * Rows whose window holds no key get O = 0 and lse = -inf.  Layouts,
 * types, alignment, asynchrony and status codes as for fa_fwd;
 * FA_ERR_INVALID_ARG also for a bound below -1.
 */
int fa_fwd_window(const void* q, const void* k, const void* v, void* o,
                  float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                  int causal, int window_left, int window_right, float scale,
                  int out_dtype, hipStream_t stream);

/*
 * Block-sparse forward ("FlashAttention Analysis", ryotta.opik.net,
 * results of FlashAttention-1: extended with a block-sparse pattern, only
 * the blocks of a mask are computed).  block_mask (DEVICE, one byte per
 * block) marks blocks of 128 query rows x 64 keys: head hq of batch b uses
 * the bytes block_mask[b * mask_batch_stride + hq * mask_head_stride +
 * qb * nkb + kb] for query block qb = i / 128 and key block kb = j / 64,
 * nkb = ceil(Nk / 64), rows qb = 0 .. ceil(Nq / 128) - 1 (strides in
 * bytes, 0 to share a mask).  Key j is visible to query i only if that
 * byte is non-zero (and, with `causal`, j <= i + Nk - Nq).  Rows whose
 * blocks are all zero get O = 0, lse = -inf.  Layouts, types and status
 * codes as for fa_fwd (dense [B, H, N, d]; the prefill kernel always
 * runs, skipping zero blocks); FA_ERR_INVALID_ARG also for a null mask or
 * negative strides; FA_ERR_UNSUPPORTED when nkb > 8191.
 */
int fa_fwd_block_sparse(const void* q, const void* k, const void* v, void* o,
                        float* lse, const unsigned char* block_mask,
                        long long mask_batch_stride, long long mask_head_stride,
                        int B, int Hq, int Hkv, int Nq, int Nk, int d,
                        int causal, float scale, int out_dtype,
                        hipStream_t stream);

/*
 * Forward with a column-interval mask (prefill form).  "FlashAttention
 * Analysis" and the Korean overview ("FlashAttention-2 (KO)", closing
 * outlook) name FlashMask, an extension that expresses richer masks per key
 * column; the pages give no representation.  Reading taken: each key
 * column j of sequence b carries the query rows that may see it,
 *     col_bounds  int32 [B, Nk, 2] (DEVICE): rows lo = [b][j][0] ..
 *                 hi - 1 = [b][j][1] - 1 (an empty range hides the key),
 * shared by the sequence's heads and applied on top of the causal flag
 * (bottom-right alignment).  Document masks, prefix-LM masks and windows
 * are such intervals.  q, k, v, o, lse as for fa_fwd.  A first kernel
 * classifies every (256-row query block, 64-key block) once for all heads;
 * each workgroup then computes only the key blocks that some of its rows
 * may see, and a wave tests every key only where some key of a block is
 * hidden from some of its rows.  The classification (B * ceil(Nq / 256) *
 * ceil(Nk / 64) ints) lives in the same per-stream library workspace as
 * fa_fwd's KV-split partials, taken and grown the same way.  Bounds are
 * read on the device and used as given (rows outside [0, Nq) simply match
 * no row).  Errors as for fa_fwd;
 * FA_ERR_INVALID_ARG also for a null or not 8-byte aligned col_bounds;
 * FA_ERR_UNSUPPORTED when Nk exceeds 6655 blocks of 64 keys (425,920 keys).
 */
int fa_fwd_colmask(const void* q, const void* k, const void* v, void* o,
                   float* lse, const int* col_bounds, int B, int Hq, int Hkv,
                   int Nq, int Nk, int d, int causal, float scale,
                   int out_dtype, hipStream_t stream);

/*
 * Forward on strided tensors (views such as slices of a fused QKV
 * projection, [B, N, H, d] layouts, padded rows).  Each of q, k, v and o
 * is described by its element strides {batch, head, row} (a host array of
 * three), the head dimension contiguous: element (b, h, i, c) of q is
 * q[b * q_stride[0] + h * q_stride[1] + i * q_stride[2] + c].  Strides are
 * multiples of 8 (every row 16-byte aligned), row strides at least d; o's
 * strides must give each (b, h, i) its own d elements.  lse is dense
 * [B, Hq, Nq].  Semantics, masks (causal flag and window bounds as for
 * fa_fwd_window) and status codes as for fa_fwd_window; the tiled prefill
 * kernel always runs.  FA_ERR_INVALID_ARG also for a null stride array or
 * a bad stride; FA_ERR_UNSUPPORTED when one head of K or V spans 2^31
 * bytes or more ((Nk - 1) * row stride * 2 + 2d).
 */
int fa_fwd_strided(const void* q, const void* k, const void* v, void* o,
                   float* lse, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                   const long long* q_stride, const long long* k_stride,
                   const long long* v_stride, const long long* o_stride,
                   int causal, int window_left, int window_right, float scale,
                   int out_dtype, hipStream_t stream);

/*
 * Forward over a paged KV cache (decode, and chunks of queries over a
 * cache: chunked prefill).
 * "FlashAttention Analysis" (ryotta.opik.net), in its closing section on
 * where the method sits, notes that paged KV caches (PagedAttention, vLLM)
 * run the fused kernels inside; the layout below is that of common serving
 * engines.
 *     q        [B, Hq, Nq, d] bf16            o [B, Hq, Nq, d] (FA_OUT_*)
 *     k_cache, v_cache  [num_pages, page_size, Hkv, d] bf16
 *     page_table  int32 [B, max_pages_per_seq]   (DEVICE)
 *     seqlens_k   int32 [B]                      (DEVICE)
 *     lse      [B, Hq, Nq] fp32
 * Sequence b owns pages page_table[b][0], [1], ... in that order: its key
 * (value) row r is row r % page_size of page page_table[b][r / page_size],
 * and its keys are its first seqlens_k[b] rows.  Its Nq queries attend to
 * them as fa_fwd_window would (causal alignment at its own last key:
 * query i sits at c = i + seqlens_k[b] - Nq; window bounds -1 for none).
 * page_size must be a power of two, at least 32.  Offsets and page numbers
 * are read on the device; a length is clamped to [0, max_pages_per_seq *
 * page_size] and a page number to [0, num_pages), so bad tables give wrong
 * results but no access outside the caches.  A sequence with no keys gets
 * O = 0 and lse = -inf.  Two forms:
 *   - num_splits = 0 and fa_paged_num_splits(...) = 0: the tiled prefill
 *     kernel, each 64-key block read from its page.  Chosen when a KV head
 *     has many query rows (Nq * Hq / Hkv > 64, as fa_fwd decides) or
 *     d = 96, provided page_size >= 64, max_pages_per_seq <= 8192 and
 *     d <= 128.  `workspace` is not used (may be NULL).
 *   - otherwise the KV-split form (partial + merge kernels) with
 *     fa_paged_num_splits(...) chunks (num_splits = 0) or num_splits
 *     chunks (1 .. 4096, no chunk over 62 pages of 32-key blocks:
 *     ceil(max_pages_per_seq * page_size / 32 / num_splits) <= 62 *
 *     page_size / 32).  `workspace` (16-byte aligned, device) holds at
 *     least fa_splitkv_workspace_bytes(B, Hq, Nq, d, splits) bytes.
 * Errors as for fa_fwd; FA_ERR_INVALID_ARG also for null or misaligned
 * tables, a bad page_size, num_pages or max_pages_per_seq < 1, a bound
 * below -1, a bad split count or (KV-split form) a small workspace;
 * FA_ERR_UNSUPPORTED when max_pages_per_seq * page_size exceeds 2^30, or
 * for d = 96 where the prefill form does not apply (pages of 32 keys, more
 * than 8192 pages per sequence, num_splits > 0).
 *
 * fa_paged_num_splits returns the chunk count of the KV-split form for
 * num_splits = 0, or 0 when the prefill form runs (and for sizes that no
 * form takes).  Pure host arithmetic; no HIP call.
 */
int fa_paged_num_splits(int B, int Hq, int Hkv, int Nq, int d, int page_size,
                        int max_pages_per_seq);

int fa_fwd_paged(const void* q, const void* k_cache, const void* v_cache,
                 void* o, float* lse, const int* page_table,
                 const int* seqlens_k, int B, int Hq, int Hkv, int Nq, int d,
                 int num_pages, int page_size, int max_pages_per_seq,
                 int causal, int window_left, int window_right, float scale,
                 int out_dtype, int num_splits, void* workspace,
                 size_t workspace_bytes, hipStream_t stream);

/*
 * Variable-length decode (or query chunks) over a padded contiguous cache.
 * Serving engines keep the caches of a batch in one tensor padded to the
 * longest sequence
 * ("FlashAttention Analysis", ryotta.opik.net, closing section: the fused
 * kernels run inside paged and cached decoding; as for the paged cache,
 * each sequence attends to its own cache length).
 *     q        [B, Hq, Nq, d] bf16            o [B, Hq, Nq, d] (FA_OUT_*)
 *     k, v     [B, Hkv, Nk, d] bf16 (Nk: the padded length)
 *     seqlens_k int32 [B] (DEVICE)            lse [B, Hq, Nq] fp32
 * Sequence b's keys are its first seqlens_k[b] rows (clamped to [0, Nk] on
 * the device); the rows past them are never read.  Its Nq queries attend
 * to them as fa_fwd_window would (causal alignment at its own last key:
 * query i sits at c = i + seqlens_k[b] - Nq; window bounds -1 for none).  A
 * sequence with no keys gets O = 0 and lse = -inf.  Two forms:
 *   - num_splits = 0 and fa_default_num_splits(B, Hq, Hkv, Nq, Nk, d) = 0
 *     (many query rows per KV head, or d = 96): the tiled prefill kernel
 *     with each sequence's key count; `workspace` is not used (may be
 *     NULL).
 *   - otherwise the KV-split form (partial + merge kernels) with chunks
 *     cut from the padded length (chunks past a sequence's length weigh
 *     nothing): fa_default_num_splits(...) chunks for num_splits = 0,
 *     else num_splits (1 .. 4096); `workspace` (16-byte aligned, device)
 *     holds at least fa_splitkv_workspace_bytes(B, Hq, Nq, d, splits)
 *     bytes.
 * Errors as for fa_fwd_splitkv; FA_ERR_INVALID_ARG also for a null or
 * misaligned seqlens_k and a bound below -1; FA_ERR_UNSUPPORTED for d = 96
 * with num_splits > 0.
 */
int fa_fwd_kvlen(const void* q, const void* k, const void* v, void* o,
                 float* lse, const int* seqlens_k, int B, int Hq, int Hkv,
                 int Nq, int Nk, int d, int causal, int window_left,
                 int window_right, float scale, int out_dtype, int num_splits,
                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Forward over a packed batch of variable-length sequences (prefill form).
 * Sequence b has the query rows cu_seqlens_q[b] .. cu_seqlens_q[b + 1] - 1
 * and the key/value rows cu_seqlens_k[b] .. cu_seqlens_k[b + 1] - 1 of the
 * packed, token-major tensors
 *     q   [total_q, Hq,  d]  bf16        k, v [total_k, Hkv, d]  bf16
 *     o   [total_q, Hq,  d]  bf16 or fp32 (FA_OUT_*)
 *     lse [Hq, total_q]      fp32, natural log
 * and is attended to on its own: the result for it is fa_fwd on its rows
 * (GQA mapping, causal mask aligned at its own last key, scale as for
 * fa_fwd).  cu_seqlens_q and cu_seqlens_k are DEVICE arrays of B + 1 int32
 * offsets, non-decreasing from 0 to total_q (total_k); max_seqlen_q and
 * max_seqlen_k bound the per-sequence lengths.  Offsets are read on the
 * device: a length is clamped to its max_seqlen and to the packed tensor,
 * so bad offsets give wrong results but no access outside q, k, v, o, lse.
 * Rows of o and lse that belong to no sequence are not written.  Every
 * sequence runs on the tiled prefill kernel (workgroups of 256 query rows).
 * Errors as for fa_fwd; FA_ERR_INVALID_ARG also for null or misaligned
 * offset arrays and total_q or total_k < 1; FA_ERR_UNSUPPORTED also when
 * (max_seqlen_k - 1) * Hkv * d * 2 + 2d >= 2^31 (one sequence's K/V rows
 * of a head are addressed with 32-bit byte offsets).
 */
int fa_fwd_varlen(const void* q, const void* k, const void* v, void* o,
                  float* lse, const int* cu_seqlens_q, const int* cu_seqlens_k,
                  int B, int Hq, int Hkv, int total_q, int total_k,
                  int max_seqlen_q, int max_seqlen_k, int d, int causal,
                  float scale, int out_dtype, hipStream_t stream);

/*
 * Attention backward pass by recomputation ("FlashAttention Analysis",
 * ryotta.opik.net, section 4 "Recomputation"; the per-row logsumexp kept
 * for it: cost guide, section on attention memory during training).  Given
 * the forward inputs, the forward output `o` (bf16) and `lse` of fa_fwd
 * for the same arguments, and the incoming gradient `dout` (bf16, the
 * layout of o), computes
 *
 *     D_i = dout_i . o_i,   P = exp(scale q k^T - lse) on visible keys,
 *     dv = P^T dout,   ds = P (dout v^T - D),
 *     dq = scale ds k,   dk = scale ds^T q,
 *
 * the scores and probabilities recomputed tile by tile and never stored.
 * With grouped-query attention dk and dv of a KV head are the sums over the
 * Hq/Hkv query heads that read it.  Rows whose lse is -inf (no visible key)
 * contribute nothing.
 *   dq       [B, Hq,  Nq, d]   written, not accumulated into
 *   dk, dv   [B, Hkv, Nk, d]   written, not accumulated into
 * in bf16 (grad_dtype FA_OUT_BF16) or fp32 (FA_OUT_F32); all device
 * pointers, 16-byte aligned (lse 4-byte).  `workspace` is a device buffer of
 * at least fa_bwd_workspace_bytes(B, Hq, Nq) bytes (two fp32 per query
 * row), 16-byte aligned, scratch on return.  Three kernels are enqueued on
 * `stream`; each output element is written by exactly one workgroup (no
 * atomics), so results are deterministic.  Argument checks and status
 * codes as for fa_fwd (d 64 or 128 only); FA_ERR_INVALID_ARG also for a missing
 * or small workspace; FA_ERR_UNSUPPORTED also when one head of Q or K
 * spans 2^31 bytes or more ((N + 128) * d * 2 >= 2^31 for N = Nq or Nk).
 */
size_t fa_bwd_workspace_bytes(int B, int Hq, int Nq);

int fa_bwd(const void* q, const void* k, const void* v, const void* o,
           const float* lse, const void* dout, void* dq, void* dk, void* dv,
           int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal,
           float scale, int grad_dtype, void* workspace,
           size_t workspace_bytes, hipStream_t stream);

/*
 * Backward pass of fa_fwd_window: fa_bwd with the sliding-window mask of
 * fa_fwd_window (same window_left / window_right meaning; -1 is no bound
 * on that side), given the o and lse of fa_fwd_window for the same
 * arguments.  Entries outside a row's window have P = 0 and no gradient;
 * K/V blocks (query row steps) that no row (key) of a block can reach are
 * skipped.  Arguments, layouts, workspace and status codes as for fa_bwd;
 * FA_ERR_INVALID_ARG also for a bound below -1.  fa_bwd is this call with
 * both bounds -1.
 */
int fa_bwd_window(const void* q, const void* k, const void* v, const void* o,
                  const float* lse, const void* dout, void* dq, void* dk,
                  void* dv, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                  int causal, int window_left, int window_right, float scale,
                  int grad_dtype, void* workspace, size_t workspace_bytes,
                  hipStream_t stream);

/* Static, human-readable text for a status code. */
const char* fa_status_string(int status);

/* The hipError_t (as int) behind the last FA_ERR_HIP on this thread. */
int fa_last_hip_error(void);

/* Build identity: the SHA-256 (64 lowercase hex digits) of the sources and
 * compiler flags this library was built from, as a static string.  Loaders
 * compare it with the sources at hand and refuse or rebuild a stale
 * library.  The same digits follow the marker "FA_SOURCE_HASH=" in the
 * library file.  Never fails. */
const char* fa_source_hash(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
