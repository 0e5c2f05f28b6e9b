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

// Workspace layout for a decode call (byte offsets, each region 256-aligned).
struct WorkspaceLayout {
    size_t acc_off, max_off, sum_off, cnt_off, total;
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
    float qk_scale_log2;       // scale * log2(e)
    float *part_acc;           // [B, Hq, S, D]
    float *part_max;           // [B, Hq, S], natural-log units
    float *part_sum;           // [B, Hq, S]
    int32_t *counters;         // [B, Hkv]
    uint16_t *out;             // [B, Hq, D] bf16
    float *lse;                // [B, Hq] or nullptr
};

// Launchers: return hipSuccess or the launch error.
hipError_t launch_build_page_table(const int32_t *req_to_token, int64_t req_to_token_stride,
                                   const int32_t *req_pool_indices, const int32_t *seq_lens,
                                   int32_t bs, int32_t seqlen_offset, int32_t page_size,
                                   int32_t max_seq_pages, int32_t *page_table,
                                   int64_t page_table_stride, int32_t *cache_seqlens,
                                   int32_t *cu_seqlens_k, hipStream_t stream);

// Producer workgroup shape (same arithmetic per split, different rounding of
// the in-workgroup combination, so one shape always uses one mode).
enum class DecodeMode { kPageSplit, kHeadGrouped };
DecodeMode default_mode(int batch, int hkv, int splits);
bool mode_supported(DecodeMode mode, int hkv);

// kv_int8: 0 = bf16 pages, 1 = int8 pages.  fused: merge in the last split
// workgroup; otherwise a separate merge launch follows the producer.
hipError_t launch_decode(const DecodeParams &p, int kv_int8, DecodeMode mode, bool fused,
                         hipStream_t stream);

hipError_t launch_split_merge(const float *acc, const float *mx, const float *sum,
                              int32_t rows, int32_t head_dim, int32_t splits, uint16_t *out,
                              float *lse, hipStream_t stream);

hipError_t launch_fill_zero(void *ptr, size_t words, hipStream_t stream);

}  // namespace spa
