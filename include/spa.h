/*
 * spa.h -- C ABI of libspa.so: split-K paged-attention decode and its
 * page-table / cu_seqlens metadata build, for AMD Instinct MI355X (gfx950).
 *
 * Every pointer argument is a DEVICE pointer (memory the caller allocated
 * with hipMalloc, or a PyTorch tensor's data pointer) unless stated
 * otherwise; every size is in elements unless stated otherwise.  The caller
 * owns every buffer, the workspace included; the library allocates nothing
 * and keeps no state between calls beyond a per-thread last-HIP-error code
 * and a read-only cache of device properties (compute units and LDS per
 * workgroup of each device, the kernels' static LDS), filled on first use
 * and used to size launches.  All calls are asynchronous on the
 * given stream, perform no host synchronisation and no memset, and may be
 * captured into a HIP graph.
 *
 * Error behaviour.  Arguments are checked on the host BEFORE anything is
 * launched: a rejected call returns a status and writes nothing.  A launch
 * failure returns SPA_ERR_HIP (spa_last_hip_error() gives the hipError_t).
 * Contract violations that only the device data could reveal -- a page id
 * outside [0, num_pages), a req_pool_indices entry outside the pool, a
 * seq_len outside [0, page_table_stride * page_size] -- give unspecified
 * results but no out-of-bounds access: the kernels guard these reads (see
 * each call).  Slot values inside req_to_token are not checked against
 * anything (they are only divided, or looked up in a map of known length).
 */
#ifndef SPA_H_
#define SPA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spa_status {
    SPA_OK = 0,
    SPA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad stride/alignment */
    SPA_ERR_UNSUPPORTED = 2,        /* shape/dtype outside the compiled set */
    SPA_ERR_WORKSPACE_TOO_SMALL = 3,
    SPA_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} spa_status;

typedef enum spa_kv_dtype {
    SPA_KV_BF16 = 0,   /* K/V pages hold bf16 values */
    SPA_KV_INT8 = 1,   /* K/V pages hold int8 codes; value = code * fp32 scale per (token, kv head) */
    SPA_KV_FP8 = 2     /* K/V pages hold OCP e4m3 codes (bias 7, largest finite 448, 0x7F/0xFF NaN);
                          value = e4m3(code) * fp32 scale per (token, kv head) */
} spa_kv_dtype;

/* flags for spa_paged_decode_attention (0 = the library chooses).  None of
 * them changes what is computed; the producer shape changes the rounding of
 * the in-workgroup combination, the merge placement changes nothing. */
#define SPA_DECODE_SEPARATE_MERGE 0x1u  /* merge as a second launch */
#define SPA_DECODE_FUSED_MERGE 0x2u     /* merge in the last split workgroup (one launch) */
#define SPA_DECODE_HEAD_GROUPED 0x4u    /* producer: 2 kv heads per workgroup (1-byte codes: 4 when
                                           num_kv_heads is a multiple of 4), waves walk all pages */
#define SPA_DECODE_PAGE_SPLIT 0x8u      /* producer: 1 kv head per workgroup, 4 waves share pages */

/* Human-readable name of a status code (static string, never NULL). */
const char *spa_status_string(spa_status status);

/* hipError_t of the last call on this host thread that returned SPA_ERR_HIP. */
int spa_last_hip_error(void);

/* ABI revision of this header; bumped on any change of a signature or of a
 * buffer layout (3: the workspace counter region moved to offset 0). */
int spa_abi_version(void);

/*
 * Page table, cache_seqlens and cu_seqlens_k in ONE launch.
 *
 * Defined by the fused CUDA-graph metadata update of sglang's TRTLLM MHA
 * backend ("trtllm_mha_graph_metadata.py": module docstring, kernel row and
 * cumsum branches, launcher), which replaces about 25 small host-dispatched
 * ops per graph replay.  For i < bs and p < max_seq_pages:
 *   cache_seqlens[i]  = seq_lens[i] + seqlen_offset                (int32)
 *   cu_seqlens_k[0]   = 0;  cu_seqlens_k[i+1] = sum_{i'<=i} cache_seqlens[i']  (int32, wraps)
 *   page_table[i*page_table_stride + p]
 *        = floor(req_to_token[req_pool_indices[i]*req_to_token_stride + p*page_size] / page_size)
 * using floor division (so slot -1 maps to page -1).  Columns
 * p >= max_seq_pages of page_table are not touched.
 *
 *   req_to_token      [pool_size, req_to_token_stride] int32, row-major
 *   req_pool_indices  [bs] int32, each in [0, pool_size)
 *   seq_lens          [bs] int32
 *   page_table        [bs, page_table_stride] int32 (output)
 *   cache_seqlens     [bs] int32 (output);  cu_seqlens_k [bs + 1] int32 (output)
 *
 * bs == 0 returns SPA_OK without launching (the source launcher's early
 * return).  Requires page_size >= 1, 0 <= max_seq_pages <= page_table_stride
 * and (max_seq_pages - 1) * page_size < req_to_token_stride.  Same launch
 * as spa_build_metadata with q_mode SPA_Q_MODE_NONE and no sliding-window
 * outputs.
 */
spa_status spa_build_page_table(const int32_t *req_to_token, int64_t req_to_token_stride,
                                int32_t pool_size, const int32_t *req_pool_indices,
                                const int32_t *seq_lens, int32_t bs, int32_t seqlen_offset,
                                int32_t page_size, int32_t max_seq_pages, int32_t *page_table,
                                int64_t page_table_stride, int32_t *cache_seqlens,
                                int32_t *cu_seqlens_k, hipStream_t stream);

/* cu_seqlens_q modes of spa_build_metadata (the source's Q_MODE values). */
#define SPA_Q_MODE_NONE 0      /* cu_seqlens_q is preset by the caller and not touched */
#define SPA_Q_MODE_CUMSUM 1    /* cu_seqlens_q[0] = 0, cu_seqlens_q[1+i] = qlens[0] + ... + qlens[i] */
#define SPA_Q_MODE_STRIDED 2   /* cu_seqlens_q[0] = 0, cu_seqlens_q[1+i] = (i + 1) * q_stride */

/*
 * The whole decode metadata update in ONE launch: everything
 * spa_build_page_table writes, plus three optional outputs (same sglang
 * source: docstring, the row branch's sliding-window part, the cumsum
 * branch's Q modes, the swa-out branch, the launcher's num_out_tokens).
 *
 *   cu_seqlens_q        [bs + 1] int32, per q_mode above (int32 arithmetic,
 *                       wraps); qlens [bs] int32 is read in CUMSUM mode only.
 *   swa_page_table      [bs, swa_page_table_stride] int32 or NULL.  For
 *                       p < max_seq_pages, with slot = the same req_to_token
 *                       entry page_table reads:
 *                         -1                               if slot < 0
 *                         -1                               if full_to_swa[slot] < 0
 *                         full_to_swa[slot] / page_size    otherwise
 *   swa_out_cache_loc   [swa_out_len] int64 or NULL.  With
 *                       num_out = min(swa_out_len, num_out_cache_loc), or 0
 *                       if out_cache_loc is NULL:
 *                         k < num_out:  -1 if out_cache_loc[k] < 0,
 *                                       else full_to_swa[out_cache_loc[k]]
 *                         otherwise:    0
 *   full_to_swa         [full_to_swa_len] int64 map from full-pool slots to
 *                       sliding-window slots (-1 = not resident), indexed by
 *                       every non-negative slot read above (the source sizes
 *                       it full_size + page_size + 1); may be NULL when
 *                       neither output reads it.  A slot at or past
 *                       full_to_swa_len is treated as unmapped (-1) instead
 *                       of being read.
 *
 * Device-side guards (not in the source, which reads whatever it is given):
 * a req_pool_indices entry outside [0, pool_size) leaves that row of
 * page_table and swa_page_table unwritten instead of reading outside
 * req_to_token.  Valid inputs never reach either guard.
 *
 * cu_seqlens_q[0] is written as 0 in the two computed modes, like
 * cu_seqlens_k[0].  bs == 0 returns SPA_OK and writes nothing, the zero
 * padding of swa_out_cache_loc included (the source launcher returns
 * first).  Alignment: int32 arrays 4 bytes, int64 arrays 8 bytes.
 * SPA_ERR_INVALID_ARGUMENT for an unknown q_mode, a missing array the
 * chosen outputs need, swa_page_table_stride < max_seq_pages, or negative
 * lengths; the checks of spa_build_page_table apply too.
 */
spa_status spa_build_metadata(
    const int32_t *req_to_token, int64_t req_to_token_stride, int32_t pool_size,
    const int32_t *req_pool_indices, const int32_t *seq_lens, int32_t bs, int32_t seqlen_offset,
    int32_t page_size, int32_t max_seq_pages, int32_t *page_table, int64_t page_table_stride,
    int32_t *cache_seqlens, int32_t *cu_seqlens_k, int32_t q_mode, const int32_t *qlens,
    int32_t q_stride, int32_t *cu_seqlens_q, const int64_t *full_to_swa,
    int64_t full_to_swa_len, int32_t *swa_page_table, int64_t swa_page_table_stride,
    const int64_t *out_cache_loc, int64_t num_out_cache_loc, int64_t *swa_out_cache_loc,
    int64_t swa_out_len, hipStream_t stream);

/*
 * Bytes of workspace spa_paged_decode_attention needs.  Layout (every
 * region 256-byte aligned): a counter region of 65536 bytes at offset 0 --
 * its first batch * num_kv_heads int32 are the arrival counters of a fused
 * call, one per (batch row, kv head) -- then the per-split partial state
 * (fp32 accumulator [B, Hq, S, D], fp32 max and sum [B, Hq, S]).  The
 * counter region has this one size for every shape, and the multi-token
 * workspace (spa_verify_workspace_bytes) starts with the same region, so no
 * call of either kind writes partial state where any call's counters live.
 * 0 for invalid sizes.
 */
size_t spa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t num_splits);

/*
 * Zero a workspace with a fill kernel (capture-safe; no hipMemset).  A new
 * workspace must be zeroed once before its first use (at least its first
 * 65536 bytes, the counter region); every successful attention call leaves
 * the counters at zero again, so no reset is needed between calls -- also
 * when one workspace, large enough for each, serves calls of different
 * shapes and both the one-token and the multi-token decode.  bytes must be
 * a multiple of 4.
 */
spa_status spa_workspace_reset(void *workspace, size_t bytes, hipStream_t stream);

/*
 * Split-K paged-attention decode: one query token per request attends over
 * its seq_lens[b] cached tokens, which live in fixed-size pages named by
 * page_table (lmdeploy PR "use PDL for paged attention", Summary and Changes:
 * a split-K producer writes per-split scratch, a reducer merges it).
 *
 *   q           [batch, num_q_heads, head_dim] bf16, contiguous, 16-byte aligned
 *   k_pages,
 *   v_pages     [num_pages, page_size, num_kv_heads, head_dim], bf16, int8
 *               codes or e4m3 codes, contiguous, 16-byte aligned; token t of request b is
 *               row (page_table[b*page_table_stride + t/page_size], t % page_size)
 *   k_scales,
 *   v_scales    [num_pages, page_size, num_kv_heads] fp32 (SPA_KV_INT8 and
 *               SPA_KV_FP8; ignored and may be NULL for bf16)
 *   page_table  [batch, page_table_stride] int32 physical page ids; an id
 *               outside [0, num_pages) is read as a page of zeros
 *   seq_lens    [batch] int32, each in [0, page_table_stride * page_size]
 *               (a length outside is clamped into that range)
 *   out         [batch, num_q_heads, head_dim] bf16 (output)
 *   lse         [batch, num_q_heads] fp32 (output, may be NULL):
 *               ln(sum_t exp(s_t)) with s_t = scale * q . k_t
 *
 * Query head h reads kv head h / (num_q_heads / num_kv_heads).  Request b's
 * ceil(L/page_size) pages are cut into num_splits splits of
 * ceil(pages/num_splits) pages each (trailing splits may be empty).  Each
 * split computes (max, sum, unnormalised accumulator); the splits are merged
 * by log-sum-exp in split order, either inside the producer launch by the
 * last split workgroup to arrive, or by a second launch -- same arithmetic,
 * bit-identical output.  With flags == 0 the library picks the producer
 * shape from batch, num_kv_heads, num_splits, kv_dtype and
 * page_table_stride (the same sizes always give the same choice, so results
 * are reproducible) and the merge placement that is faster for it; a bf16
 * head-grouped workgroup may also take several consecutive splits, sized
 * from the device's compute units (the per-split arithmetic, and so the
 * result, is unchanged).  L == 0 gives out = 0 and
 * lse = -inf.  Contradictory flags (both merges, both producers) are
 * SPA_ERR_INVALID_ARGUMENT.
 *
 * Supported: head_dim 128, page_size 64, num_q_heads == 4 * num_kv_heads,
 * kv_dtype bf16, int8 or fp8, 1 <= num_splits <= 1024
 * (SPA_DECODE_HEAD_GROUPED also needs an even num_kv_heads); otherwise
 * SPA_ERR_UNSUPPORTED.  The fused merge needs batch * num_kv_heads <= 16384
 * (the counter region): above that the default plan merges in a second
 * launch and SPA_DECODE_FUSED_MERGE is SPA_ERR_UNSUPPORTED.  workspace: spa_decode_workspace_bytes(...) bytes,
 * 16-byte aligned, zeroed before first use (see spa_workspace_reset);
 * concurrent calls must not share a workspace.  batch == 0 returns SPA_OK
 * without launching.
 */
spa_status spa_paged_decode_attention(const void *q, const void *k_pages, const void *v_pages,
                                      const float *k_scales, const float *v_scales,
                                      const int32_t *page_table, int64_t page_table_stride,
                                      const int32_t *seq_lens, int32_t batch,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t page_size, int32_t num_pages,
                                      int32_t num_splits, float scale, spa_kv_dtype kv_dtype,
                                      uint32_t flags, void *workspace, size_t workspace_bytes,
                                      void *out, float *lse, hipStream_t stream);

/*
 * spa_paged_decode_attention without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, checks, launches
 * and results (bit for bit) as spa_paged_decode_attention with a workspace
 * of spa_decode_workspace_bytes(...) bytes; it calls no allocating routine.
 *
 * Its workspace is a 32 MiB (33554432-byte) array of device memory inside
 * the library, one per GPU, held until the process ends; the first call on
 * a device looks up that device's copy and clears its counter region with a
 * fill kernel on `stream` (fused merges leave it zeroed again).  A call whose
 * spa_decode_workspace_bytes(...) exceeds 32 MiB returns
 * SPA_ERR_WORKSPACE_TOO_SMALL and launches nothing (batch 32 with 16 splits
 * at 32 query heads needs about 8.5 MB).  Every call on one GPU uses the
 * same array: calls that may overlap in time on one GPU (different streams
 * without ordering between them, or different host threads) race on it and
 * must be serialised by the caller.
 */
spa_status spa_paged_decode_attention_noalloc(
    const void *q, const void *k_pages, const void *v_pages, const float *k_scales,
    const float *v_scales, const int32_t *page_table, int64_t page_table_stride,
    const int32_t *seq_lens, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size, int32_t num_pages, int32_t num_splits, float scale,
    spa_kv_dtype kv_dtype, uint32_t flags, void *out, float *lse, hipStream_t stream);

/*
 * The launch plan spa_paged_decode_attention takes with flags == 0 for these
 * sizes: one producer flag (SPA_DECODE_HEAD_GROUPED or SPA_DECODE_PAGE_SPLIT)
 * or'ed with one merge flag (SPA_DECODE_FUSED_MERGE or
 * SPA_DECODE_SEPARATE_MERGE).  Passing the result back as flags gives the
 * same launches.  The flags depend on batch, num_kv_heads, num_splits,
 * kv_dtype and page_table_stride (head grouped, with an even num_kv_heads,
 * from 1024 request x kv head x split triples; for bf16 also from 256 when a
 * split holds at most 8 pages, ceil(page_table_stride / num_splits), and
 * from 128 when it holds at most 2; merge fused for up to 8 page-split or 4
 * head-grouped splits).  Within the plan, the splits a bf16 or fp8
 * head-grouped workgroup walks (fp8: at most 2) also depend on
 * page_table_stride, the current device's
 * compute units and, when the walked grid is about one round of resident
 * workgroups, per call on seq_lens (a walk is then taken only when the
 * longest request has at most 6/5 of the mean number of pages).  0 for sizes
 * spa_paged_decode_attention would reject as invalid or unsupported.
 */
uint32_t spa_decode_default_flags(int32_t batch, int32_t num_kv_heads, int32_t num_splits,
                                  spa_kv_dtype kv_dtype, int64_t page_table_stride);

/*
 * The producer pass of split-K decode alone (lmdeploy PR "use PDL for paged
 * attention", Changes: the split-K producer writes per-split scratch that a
 * reducer reads): the same per-split state spa_paged_decode_attention forms
 * before its merge, written to caller buffers in the layout spa_split_merge
 * reads.  spa_paged_decode_partials followed by spa_split_merge on the same
 * stream gives bit for bit the output of spa_paged_decode_attention with the
 * same producer flag and SPA_DECODE_SEPARATE_MERGE.  It is also the
 * per-device step of a context split across devices: each device forms the
 * states of its own splits, and one merge combines them after the exchange.
 *
 * For request b, query head h and split j (pages cut as in
 * spa_paged_decode_attention), over the split's tokens t:
 *   partial_max[b,h,j]   = m_j = max_t s_t               (natural-log units)
 *   partial_sum[b,h,j]   = sum_t exp(s_t - m_j)
 *   partial_acc[b,h,j,:] = sum_t exp(s_t - m_j) v_t      (not divided by the sum)
 * and (-inf, 0, 0) for a split with no tokens.
 *
 *   partial_acc [batch, num_q_heads, num_splits, head_dim] fp32, 16-byte aligned (output)
 *   partial_max, partial_sum [batch, num_q_heads, num_splits] fp32 (outputs)
 *   other arguments as in spa_paged_decode_attention.
 *
 * flags: 0 (the producer spa_paged_decode_attention would choose), or
 * SPA_DECODE_HEAD_GROUPED or SPA_DECODE_PAGE_SPLIT; a merge flag is
 * SPA_ERR_INVALID_ARGUMENT.  No workspace: the partial buffers are the
 * scratch, owned by the caller, and need no zeroing.  Supported set and
 * errors as in spa_paged_decode_attention; batch == 0 returns SPA_OK
 * without launching.
 */
spa_status spa_paged_decode_partials(const void *q, const void *k_pages, const void *v_pages,
                                     const float *k_scales, const float *v_scales,
                                     const int32_t *page_table, int64_t page_table_stride,
                                     const int32_t *seq_lens, int32_t batch,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t page_size, int32_t num_pages,
                                     int32_t num_splits, float scale, spa_kv_dtype kv_dtype,
                                     uint32_t flags, float *partial_acc, float *partial_max,
                                     float *partial_sum, hipStream_t stream);

/*
 * Bytes of workspace spa_paged_verify_attention needs: the 65536-byte
 * counter region of the decode workspace (unused here, never written), then
 * the per-split state of every (query row, head) (fp32 accumulator
 * [total_q, Hq, S, D], fp32 max and sum [total_q, Hq, S]), 256-byte aligned
 * regions.  0 for invalid sizes.
 */
size_t spa_verify_workspace_bytes(int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t num_splits);

/*
 * Multi-token query decode (target verify / draft extend): several query
 * tokens per request, causal among themselves, over the paged KV cache --
 * the step whose cu_seqlens_q the sglang fused metadata update builds
 * (module docstring; cumsum branch, Q modes 1 and 2).
 *
 * Request b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (n_b of
 * them, 0 <= n_b <= max_q_len) and seq_lens[b] = L_b cached tokens, whose
 * last n_b are the query tokens' own (a speculative-decoding step with k
 * draft tokens verifies n_b = k + 1 rows).  Query token i (row cu_seqlens_q[b] +
 * i) attends tokens 0 .. L_b - n_b + i:
 *   out[row, h, :] = softmax_t(s_t) . v_t,  lse[row, h] = ln sum_t exp(s_t),
 *   s_t = scale * q[row, h, :] . k_t,  query head h reads kv head h / 4;
 * a row that sees no token gets out = 0 and lse = -inf.  Split-K as in
 * spa_paged_decode_attention (same page partition, split states merged in
 * split order by a second launch; with bf16 KV a workgroup may take several
 * consecutive splits, which leaves the result unchanged).
 *
 *   q           [total_q, num_q_heads, head_dim] bf16, contiguous, 16-byte aligned
 *   cu_seqlens_q [batch + 1] int32 (device), non-decreasing, cu[0] >= 0,
 *               cu[batch] <= total_q (the metadata build writes it)
 *   out         [total_q, num_q_heads, head_dim] bf16 (output, 16-byte aligned)
 *   lse         [total_q, num_q_heads] fp32 (output, may be NULL)
 *   other arguments as in spa_paged_decode_attention.
 *
 * max_q_len (host side, 1..64) bounds n_b: one workgroup takes up to 8 query
 * tokens of a request (4 when max_q_len <= 4) and reads the request's K and
 * V once for all of them; a larger max_q_len cuts each request's rows into
 * chunks of 8, each reading K and V again.  A request whose device data
 * holds more rows than max_q_len has its first max_q_len rows computed with
 * the causal limits of all n_b rows, and the rest written as out = 0,
 * lse = -inf.
 *
 * Supported: max_q_len 1..64, head_dim 128, page_size 64, num_q_heads == 4 *
 * num_kv_heads with num_kv_heads even, bf16 / int8 / fp8 KV, 1 <= num_splits
 * <= 1024; otherwise SPA_ERR_UNSUPPORTED.  Rows not covered by cu_seqlens_q,
 * and the rows of a request whose span leaves [0, total_q), are left
 * unspecified (never written outside the output).  The workspace needs no
 * zeroing.  batch == 0 or total_q == 0 returns SPA_OK without launching.
 */
spa_status spa_paged_verify_attention(const void *q, const void *k_pages, const void *v_pages,
                                      const float *k_scales, const float *v_scales,
                                      const int32_t *page_table, int64_t page_table_stride,
                                      const int32_t *seq_lens, const int32_t *cu_seqlens_q,
                                      int32_t batch, int32_t total_q, int32_t max_q_len,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t page_size, int32_t num_pages,
                                      int32_t num_splits, float scale, spa_kv_dtype kv_dtype,
                                      void *workspace, size_t workspace_bytes, void *out,
                                      float *lse, hipStream_t stream);

/*
 * Log-sum-exp merge of per-split partial softmax state (the reducer of the
 * lmdeploy split-K decode).  For each (b, h), with j = 0..num_splits-1 in order:
 *   M = max_j m_j;  w_j = exp(m_j - M), or 0 where m_j = -inf (an empty split)
 *   out[b,h,:] = sum_j w_j acc_j / sum_j w_j l_j   (bf16, round to nearest even)
 *   lse[b,h]   = M + ln(sum_j w_j l_j)
 * and out = 0, lse = -inf where sum_j w_j l_j == 0.
 *
 *   partial_acc [batch, num_q_heads, num_splits, head_dim] fp32, unnormalised
 *   partial_max [batch, num_q_heads, num_splits] fp32, natural-log units of s
 *   partial_sum [batch, num_q_heads, num_splits] fp32
 *   out         [batch, num_q_heads, head_dim] bf16;  lse [batch, num_q_heads] fp32 (may be NULL)
 *
 * Any head_dim in [1, 4096] and num_splits in [1, 1024]; batch == 0 is a no-op.
 */
spa_status spa_split_merge(const float *partial_acc, const float *partial_max,
                           const float *partial_sum, int32_t batch, int32_t num_q_heads,
                           int32_t head_dim, int32_t num_splits, void *out, float *lse,
                           hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SPA_H_ */
