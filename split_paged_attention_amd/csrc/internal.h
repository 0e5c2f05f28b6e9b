// Internal declarations shared by the C-ABI layer (api.cpp) and the kernel
// translation units.  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace spa {

// Compiled shape set of the decode kernels.
constexpr int kHeadDim = 128;
constexpr int kPageSize = 64;
constexpr int kGroup = 4;       // query heads per kv head
// Per-wave timeline of the decode producer (diagnostics build, SPA_TIMELINE):
// slot numbers of include/spa_timeline.h.
enum TimelineSlot : int {
    kTlEntry = 0, kTlLength = 1, kTlFirstPageId = 2, kTlFirstScores = 3, kTlPagesDone = 4,
    kTlStatesIssued = 5, kTlStatesInMemory = 6, kTlArrived = 7, kTlMergeDone = 8, kTlEnd = 9,
    kTlWhat = 10, kTlPages = 11
};
constexpr int kTimelineSlots = 16;
constexpr size_t kTimelineWaves = 65536;
// Multi-token decode: query tokens per request the host may declare
// (max_q_len); one workgroup takes up to 8 of them, more are cut into chunks.
constexpr int kMaxVerifyQueryLen = 64;

// Workspace layout of the decode and multi-token decode calls (byte
// offsets, each region 256-aligned).  The counter region comes first and has
// one size for every shape and entry point, so no call writes partial state
// where any call's counters live: a workspace shared by calls of different
// shapes, or by one-token and multi-token calls, keeps its counters at zero.
constexpr size_t kCounterRegionBytes = 65536;
constexpr int64_t kMaxCounterGroups = (int64_t)(kCounterRegionBytes / sizeof(int32_t));
struct WorkspaceLayout {
    size_t cnt_off, acc_off, max_off, sum_off, total;
};
WorkspaceLayout workspace_layout(int64_t batch, int64_t hq, int64_t hkv, int64_t head_dim,
                                 int64_t splits);

struct DecodeParams {
    const void *q;             // [B, Hq, D] bf16
    const void *k_pages;       // [num_pages, P, Hkv, D]
    const void *v_pages;
    const float *k_scales;     // [num_pages, P, Hkv] (int8 only)
    const float *v_scales;
    const int32_t *page_table; // [B, pt_stride]
    int64_t pt_stride;
    const int32_t *seq_lens;   // [B]
    int32_t batch, hq, hkv, splits;
    int32_t split_walk;        // head-grouped bf16 / e4m3: splits per workgroup (divides splits)
    int32_t walk_checked;      // 1: walk only if the batch's page counts are balanced (grid
                               // of a workgroup per split); 0: always (grid cut to match)
    int32_t num_pages;         // pool size: page ids outside [0, num_pages) load nothing
    float qk_scale_log2;       // scale * log2(e)
    float *part_acc;           // [B, Hq, S, D]
    float *part_max;           // [B, Hq, S], natural-log units
    float *part_sum;           // [B, Hq, S]
    int32_t *counters;         // [B, Hkv]
    uint16_t *out;             // [B, Hq, D] bf16 ([total_q, Hq, D] multi-token)
    float *lse;                // [B, Hq] or nullptr
    // multi-token decode only: query rows of request b are
    // cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of total_q
    const int32_t *cu_seqlens_q;
    int32_t total_q;
    int32_t max_q_len;         // query rows computed per request (more get the empty state)
    int32_t q_chunks;          // query-token chunks per request (grid dimension)
};

// cu_seqlens_q handling of the metadata build.
constexpr int32_t kQModeNone = 0;      // preset by the caller, untouched
constexpr int32_t kQModeCumsum = 1;    // cu_seqlens_q[1 + i] = qlens[0] + ... + qlens[i]
constexpr int32_t kQModeStrided = 2;   // cu_seqlens_q[1 + i] = (i + 1) * q_stride

struct MetadataParams {
    const int32_t *req_to_token;     // [pool, req_to_token_stride]
    int64_t req_to_token_stride;
    int32_t pool_size;               // rows of req_to_token
    const int32_t *req_pool_indices; // [bs]
    const int32_t *seq_lens;         // [bs]
    int32_t bs, seqlen_offset, page_size, max_seq_pages;
    int32_t *page_table;             // [bs, page_table_stride]
    int64_t page_table_stride;
    int32_t *cache_seqlens;          // [bs]
    int32_t *cu_seqlens_k;           // [bs + 1]
    int32_t q_mode, q_stride;
    const int32_t *qlens;            // [bs] (cumsum mode)
    int32_t *cu_seqlens_q;           // [bs + 1] (cumsum / strided mode)
    const int64_t *full_to_swa;      // slot -> sliding-window slot, or nullptr
    int64_t full_to_swa_len;         // slots at or past it count as unmapped
    int32_t *swa_page_table;         // [bs, swa_page_table_stride] or nullptr
    int64_t swa_page_table_stride;
    const int64_t *out_cache_loc;    // [>= num_out]
    int64_t num_out;                 // translated prefix of swa_out_cache_loc
    int64_t *swa_out_cache_loc;      // [swa_out_len] or nullptr
    int64_t swa_out_len;
};

// Workgroups the metadata launch needs (bs rows, one scan, the swa-out tiles).
int64_t metadata_grid(int32_t bs, int64_t swa_out_len);

// Launchers: return hipSuccess or the launch error.
hipError_t launch_build_metadata(const MetadataParams &p, hipStream_t stream);

// Producer workgroup shape (same arithmetic per split, different rounding of
// the in-workgroup combination, so one shape always uses one mode).
enum class DecodeMode { kPageSplit, kHeadGrouped };
DecodeMode default_mode(int batch, int hkv, int splits, int kv_type, int64_t pt_stride);
// Splits one head-grouped workgroup walks (bf16 only; 1 for 1-byte codes),
// and the device's LDS limit per workgroup.
int split_walk_for(const DecodeParams &p, bool quant, int nw);
// 1 if a walk of `walk` splits over a grid of split_wgs workgroups (one per
// split) is taken only for a batch with balanced page counts, 0 if always.
int walk_checked_for(int64_t split_wgs, int walk);
size_t max_lds_per_block();
bool mode_supported(DecodeMode mode, int hkv);

// kv_type: kKvBf16, kKvInt8 or kKvFp8 pages.  fused: merge in the last
// split workgroup; otherwise a separate merge launch follows the producer.
constexpr int kKvBf16 = 0, kKvInt8 = 1, kKvFp8 = 2;
hipError_t launch_decode(const DecodeParams &p, int kv_type, DecodeMode mode, bool fused,
                         hipStream_t stream);
// The producer alone (separate-merge form): split states to p.part_*.
hipError_t launch_decode_producer(const DecodeParams &p, int kv_type, DecodeMode mode,
                                  hipStream_t stream);

// Multi-token decode producer (2 kv heads per workgroup, 4 or 8 query tokens
// of a request per workgroup, more in chunks) + split merge over total_q * hq
// rows; partial state rows are query rows.
int verify_tokens_per_workgroup(int max_q_len);
hipError_t launch_verify(const DecodeParams &p, int kv_type, int max_q_len, hipStream_t stream);
bool verify_supported(int hkv);

hipError_t launch_split_merge(const float *acc, const float *mx, const float *sum,
                              int32_t rows, int32_t head_dim, int32_t splits, uint16_t *out,
                              float *lse, hipStream_t stream);

hipError_t launch_fill_zero(void *ptr, size_t words, hipStream_t stream);

}  // namespace spa
