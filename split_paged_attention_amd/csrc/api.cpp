// C ABI of libspa.so: host-side argument checks, workspace layout and
// dispatch to the kernels.  Every check runs before any HIP call, so a
// rejected call launches nothing and writes nothing.
#include <math.h>

#include <mutex>

#include "../../include/spa.h"
#include "internal.h"

namespace spa {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WorkspaceLayout workspace_layout(int64_t batch, int64_t hq, int64_t hkv, int64_t head_dim,
                                 int64_t splits) {
    (void)hkv;   // the counter region has one size for every shape
    WorkspaceLayout w{};
    const size_t rows = (size_t)batch * (size_t)hq * (size_t)splits;
    w.cnt_off = 0;
    w.acc_off = kCounterRegionBytes;
    w.max_off = align256(w.acc_off + rows * (size_t)head_dim * sizeof(float));
    w.sum_off = align256(w.max_off + rows * sizeof(float));
    w.total = align256(w.sum_off + rows * sizeof(float));
    return w;
}

}  // namespace spa

namespace {

thread_local int g_last_hip_error = 0;

spa_status hip_status(hipError_t e) {
    if (e == hipSuccess) return SPA_OK;
    g_last_hip_error = (int)e;
    return SPA_ERR_HIP;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int kv_type_of(spa_kv_dtype d) {
    return d == SPA_KV_INT8 ? spa::kKvInt8 : d == SPA_KV_FP8 ? spa::kKvFp8 : spa::kKvBf16;
}

// Device memory of spa_paged_decode_attention_noalloc: one decode
// workspace (counter region, then partial state) per GPU, held until the
// process ends.  In host code `scratch` is a stand-in for the symbol, not a
// device address: kernels and fills get the address hipGetSymbolAddress
// returns for the current device.
constexpr size_t kScratchBytes = (size_t)32 << 20;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on the current device.  The first call on a
// device looks it up and clears its counter region with the fill kernel on
// `stream` (the fused merge needs zeroed counters and leaves them zeroed).
spa_status scratch_of_current_device(void **ptr, hipStream_t stream) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxDevices) return SPA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        if (p == nullptr) return SPA_ERR_HIP;
        e = spa::launch_fill_zero(p, spa::kCounterRegionBytes / sizeof(uint32_t), stream);
        if (e != hipSuccess) return hip_status(e);
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SPA_OK;
}

// Launch plan of a decode call: KV type, producer shape, merge placement.
struct DecodePlan {
    int kv_type;
    spa::DecodeMode mode;
    bool fused;
};

// The plan flags == 0 selects.  Merge (measured over the same sweep as the
// producer choice): fused into the producer launch for page-split grids of
// up to 8 splits and head-grouped grids of up to 4; a second launch for more
// splits, where the last arrival's merge of all of them sits on the
// critical path of grids whose splits finish together.
DecodePlan default_plan(int32_t batch, int32_t hkv, int32_t splits, int kv_type,
                        int64_t pt_stride) {
    DecodePlan plan{};
    plan.kv_type = kv_type;
    plan.mode = spa::default_mode(batch, hkv, splits, kv_type, pt_stride);
    const int fused_max_splits = plan.mode == spa::DecodeMode::kPageSplit ? 8 : 4;
    plan.fused = splits <= fused_max_splits && (int64_t)batch * hkv <= spa::kMaxCounterGroups;
    return plan;
}

// Checks shared by the one-token decode entry points (everything but the
// outputs and scratch) and the parameters and plan they lead to.
// producer_only: a merge flag is an error (the caller merges).
spa_status decode_setup(const void *q, const void *k_pages, const void *v_pages,
                        const float *k_scales, const float *v_scales, const int32_t *page_table,
                        int64_t page_table_stride, const int32_t *seq_lens, int32_t batch,
                        int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        int32_t page_size, int32_t num_pages, int32_t num_splits, float scale,
                        spa_kv_dtype kv_dtype, uint32_t flags, bool producer_only,
                        spa::DecodeParams *p, DecodePlan *plan) {
    if (batch < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 || page_size < 1 ||
        num_pages < 1 || num_splits < 1 || page_table_stride < 1)
        return SPA_ERR_INVALID_ARGUMENT;
    if (num_q_heads % num_kv_heads != 0) return SPA_ERR_INVALID_ARGUMENT;
    if (kv_dtype != SPA_KV_BF16 && kv_dtype != SPA_KV_INT8 && kv_dtype != SPA_KV_FP8)
        return SPA_ERR_INVALID_ARGUMENT;
    const bool quant = kv_dtype != SPA_KV_BF16;
    const uint32_t merge_flags = SPA_DECODE_SEPARATE_MERGE | SPA_DECODE_FUSED_MERGE;
    const uint32_t known = merge_flags | SPA_DECODE_HEAD_GROUPED | SPA_DECODE_PAGE_SPLIT;
    if ((flags & ~known) != 0) return SPA_ERR_INVALID_ARGUMENT;
    if (producer_only && (flags & merge_flags) != 0) return SPA_ERR_INVALID_ARGUMENT;
    if ((flags & SPA_DECODE_SEPARATE_MERGE) && (flags & SPA_DECODE_FUSED_MERGE))
        return SPA_ERR_INVALID_ARGUMENT;
    if ((flags & SPA_DECODE_HEAD_GROUPED) && (flags & SPA_DECODE_PAGE_SPLIT))
        return SPA_ERR_INVALID_ARGUMENT;
    if (!isfinite(scale)) return SPA_ERR_INVALID_ARGUMENT;
    if (head_dim != spa::kHeadDim || page_size != spa::kPageSize ||
        num_q_heads != spa::kGroup * num_kv_heads || num_splits > 1024)
        return SPA_ERR_UNSUPPORTED;
    // grid = batch * kv_heads * splits workgroups must fit a 32-bit grid
    if ((int64_t)batch * num_kv_heads * num_splits > (int64_t)INT32_MAX)
        return SPA_ERR_UNSUPPORTED;
    *plan = default_plan(batch, num_kv_heads, num_splits, kv_type_of(kv_dtype), page_table_stride);
    if (flags & SPA_DECODE_HEAD_GROUPED) plan->mode = spa::DecodeMode::kHeadGrouped;
    if (flags & SPA_DECODE_PAGE_SPLIT) plan->mode = spa::DecodeMode::kPageSplit;
    if (flags & SPA_DECODE_SEPARATE_MERGE) plan->fused = false;
    if (flags & SPA_DECODE_FUSED_MERGE) plan->fused = true;
    if (producer_only) plan->fused = false;
    // the fused merge needs one arrival counter per (request, kv head)
    if (plan->fused && (int64_t)batch * num_kv_heads > spa::kMaxCounterGroups) {
        if (flags & SPA_DECODE_FUSED_MERGE) return SPA_ERR_UNSUPPORTED;
        plan->fused = false;
    }
    if (batch == 0) return SPA_OK;
    if (!spa::mode_supported(plan->mode, num_kv_heads)) return SPA_ERR_UNSUPPORTED;
    if (!q || !k_pages || !v_pages || !page_table || !seq_lens) return SPA_ERR_INVALID_ARGUMENT;
    if (quant && (!k_scales || !v_scales)) return SPA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
        !aligned(page_table, 4) || !aligned(seq_lens, 4) ||
        (quant && (!aligned(k_scales, 4) || !aligned(v_scales, 4))))
        return SPA_ERR_INVALID_ARGUMENT;
    p->q = q;
    p->k_pages = k_pages;
    p->v_pages = v_pages;
    p->k_scales = k_scales;
    p->v_scales = v_scales;
    p->page_table = page_table;
    p->pt_stride = page_table_stride;
    p->seq_lens = seq_lens;
    p->batch = batch;
    p->hq = num_q_heads;
    p->hkv = num_kv_heads;
    p->splits = num_splits;
    p->num_pages = num_pages;
    p->qk_scale_log2 = scale * 1.4426950408889634f;
    return SPA_OK;
}

// The decode launches of a checked call on a workspace of layout w.
spa_status run_decode(spa::DecodeParams &p, const DecodePlan &plan, const spa::WorkspaceLayout &w,
                      void *workspace, void *out, float *lse, hipStream_t stream) {
    char *ws = static_cast<char *>(workspace);
    p.part_acc = reinterpret_cast<float *>(ws + w.acc_off);
    p.part_max = reinterpret_cast<float *>(ws + w.max_off);
    p.part_sum = reinterpret_cast<float *>(ws + w.sum_off);
    p.counters = reinterpret_cast<int32_t *>(ws + w.cnt_off);
    p.out = static_cast<uint16_t *>(out);
    p.lse = lse;
    return hip_status(spa::launch_decode(p, plan.kv_type, plan.mode, plan.fused, stream));
}

}  // namespace

extern "C" {

const char *spa_status_string(spa_status status) {
    switch (status) {
        case SPA_OK: return "SPA_OK";
        case SPA_ERR_INVALID_ARGUMENT: return "SPA_ERR_INVALID_ARGUMENT";
        case SPA_ERR_UNSUPPORTED: return "SPA_ERR_UNSUPPORTED";
        case SPA_ERR_WORKSPACE_TOO_SMALL: return "SPA_ERR_WORKSPACE_TOO_SMALL";
        case SPA_ERR_HIP: return "SPA_ERR_HIP";
    }
    return "SPA_ERR_UNKNOWN";
}

int spa_last_hip_error(void) { return g_last_hip_error; }

int spa_abi_version(void) { return 3; }

spa_status spa_build_metadata(
    const int32_t *req_to_token, int64_t req_to_token_stride, int32_t pool_size,
    const int32_t *req_pool_indices, const int32_t *seq_lens, int32_t bs, int32_t seqlen_offset,
    int32_t page_size, int32_t max_seq_pages, int32_t *page_table, int64_t page_table_stride,
    int32_t *cache_seqlens, int32_t *cu_seqlens_k, int32_t q_mode, const int32_t *qlens,
    int32_t q_stride, int32_t *cu_seqlens_q, const int64_t *full_to_swa,
    int64_t full_to_swa_len, int32_t *swa_page_table, int64_t swa_page_table_stride,
    const int64_t *out_cache_loc, int64_t num_out_cache_loc, int64_t *swa_out_cache_loc,
    int64_t swa_out_len, hipStream_t stream) {
    const int64_t min_stride = max_seq_pages > 1 ? max_seq_pages : 1;
    if (bs < 0 || page_size < 1 || max_seq_pages < 0 || pool_size < 1 ||
        page_table_stride < min_stride || req_to_token_stride < 1)
        return SPA_ERR_INVALID_ARGUMENT;
    if (max_seq_pages > 0 && (int64_t)(max_seq_pages - 1) * page_size >= req_to_token_stride)
        return SPA_ERR_INVALID_ARGUMENT;
    if (q_mode != spa::kQModeNone && q_mode != spa::kQModeCumsum &&
        q_mode != spa::kQModeStrided)
        return SPA_ERR_INVALID_ARGUMENT;
    if (swa_page_table && swa_page_table_stride < min_stride) return SPA_ERR_INVALID_ARGUMENT;
    if (full_to_swa && full_to_swa_len < 0) return SPA_ERR_INVALID_ARGUMENT;
    if (swa_out_cache_loc && (swa_out_len < 0 || num_out_cache_loc < 0))
        return SPA_ERR_INVALID_ARGUMENT;
    int64_t num_out = 0;
    if (swa_out_cache_loc && out_cache_loc)
        num_out = num_out_cache_loc < swa_out_len ? num_out_cache_loc : swa_out_len;
    const int64_t out_len = swa_out_cache_loc ? swa_out_len : 0;
    const int64_t max_groups = (int64_t)(UINT32_MAX / 256);   // work-items fit in 32 bits
    if (out_len > max_groups * 1024 || spa::metadata_grid(bs, out_len) > max_groups)
        return SPA_ERR_INVALID_ARGUMENT;
    if (bs == 0) return SPA_OK;
    if (!req_to_token || !req_pool_indices || !seq_lens || !page_table || !cache_seqlens ||
        !cu_seqlens_k)
        return SPA_ERR_INVALID_ARGUMENT;
    if (q_mode != spa::kQModeNone && !cu_seqlens_q) return SPA_ERR_INVALID_ARGUMENT;
    if (q_mode == spa::kQModeCumsum && !qlens) return SPA_ERR_INVALID_ARGUMENT;
    if ((swa_page_table || num_out > 0) && !full_to_swa) return SPA_ERR_INVALID_ARGUMENT;
    if (!aligned(req_to_token, 4) || !aligned(req_pool_indices, 4) || !aligned(seq_lens, 4) ||
        !aligned(page_table, 4) || !aligned(cache_seqlens, 4) || !aligned(cu_seqlens_k, 4) ||
        !aligned(qlens, 4) || !aligned(cu_seqlens_q, 4) || !aligned(full_to_swa, 8) ||
        !aligned(swa_page_table, 4) || !aligned(out_cache_loc, 8) ||
        !aligned(swa_out_cache_loc, 8))
        return SPA_ERR_INVALID_ARGUMENT;
    spa::MetadataParams p{};
    p.req_to_token = req_to_token;
    p.req_to_token_stride = req_to_token_stride;
    p.pool_size = pool_size;
    p.req_pool_indices = req_pool_indices;
    p.seq_lens = seq_lens;
    p.bs = bs;
    p.seqlen_offset = seqlen_offset;
    p.page_size = page_size;
    p.max_seq_pages = max_seq_pages;
    p.page_table = page_table;
    p.page_table_stride = page_table_stride;
    p.cache_seqlens = cache_seqlens;
    p.cu_seqlens_k = cu_seqlens_k;
    p.q_mode = q_mode;
    p.q_stride = q_stride;
    p.qlens = qlens;
    p.cu_seqlens_q = cu_seqlens_q;
    p.full_to_swa = full_to_swa;
    p.full_to_swa_len = full_to_swa ? full_to_swa_len : 0;
    p.swa_page_table = swa_page_table;
    p.swa_page_table_stride = swa_page_table_stride;
    p.out_cache_loc = num_out > 0 ? out_cache_loc : nullptr;
    p.num_out = num_out;
    p.swa_out_cache_loc = swa_out_cache_loc;
    p.swa_out_len = out_len;
    return hip_status(spa::launch_build_metadata(p, stream));
}

spa_status spa_build_page_table(const int32_t *req_to_token, int64_t req_to_token_stride,
                                int32_t pool_size, const int32_t *req_pool_indices,
                                const int32_t *seq_lens, int32_t bs, int32_t seqlen_offset,
                                int32_t page_size, int32_t max_seq_pages, int32_t *page_table,
                                int64_t page_table_stride, int32_t *cache_seqlens,
                                int32_t *cu_seqlens_k, hipStream_t stream) {
    return spa_build_metadata(req_to_token, req_to_token_stride, pool_size, req_pool_indices,
                              seq_lens, bs, seqlen_offset, page_size, max_seq_pages, page_table,
                              page_table_stride, cache_seqlens, cu_seqlens_k, spa::kQModeNone,
                              nullptr, 0, nullptr, nullptr, 0, nullptr, 0, nullptr, 0, nullptr, 0,
                              stream);
}

size_t spa_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t num_splits) {
    if (batch < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 || num_splits < 1)
        return 0;
    return spa::workspace_layout(batch, num_q_heads, num_kv_heads, head_dim, num_splits).total;
}

spa_status spa_workspace_reset(void *workspace, size_t bytes, hipStream_t stream) {
    if (bytes == 0) return SPA_OK;
    if (!workspace || bytes % 4 != 0 || !aligned(workspace, 4)) return SPA_ERR_INVALID_ARGUMENT;
    return hip_status(spa::launch_fill_zero(workspace, bytes / 4, stream));
}

spa_status spa_paged_decode_attention(const void *q, const void *k_pages, const void *v_pages,
                                      const float *k_scales, const float *v_scales,
                                      const int32_t *page_table, int64_t page_table_stride,
                                      const int32_t *seq_lens, int32_t batch,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t page_size, int32_t num_pages,
                                      int32_t num_splits, float scale, spa_kv_dtype kv_dtype,
                                      uint32_t flags, void *workspace, size_t workspace_bytes,
                                      void *out, float *lse, hipStream_t stream) {
    spa::DecodeParams p{};
    DecodePlan plan{};
    spa_status st = decode_setup(q, k_pages, v_pages, k_scales, v_scales, page_table,
                                 page_table_stride, seq_lens, batch, num_q_heads, num_kv_heads,
                                 head_dim, page_size, num_pages, num_splits, scale, kv_dtype,
                                 flags, /*producer_only=*/false, &p, &plan);
    if (st != SPA_OK || batch == 0) return st;
    if (!out || !workspace) return SPA_ERR_INVALID_ARGUMENT;
    if (!aligned(workspace, 16) || !aligned(out, 2) || (lse && !aligned(lse, 4)))
        return SPA_ERR_INVALID_ARGUMENT;
    const spa::WorkspaceLayout w =
        spa::workspace_layout(batch, num_q_heads, num_kv_heads, head_dim, num_splits);
    if (workspace_bytes < w.total) return SPA_ERR_WORKSPACE_TOO_SMALL;
    return run_decode(p, plan, w, workspace, out, lse, stream);
}

spa_status spa_paged_decode_attention_noalloc(
    const void *q, const void *k_pages, const void *v_pages, const float *k_scales,
    const float *v_scales, const int32_t *page_table, int64_t page_table_stride,
    const int32_t *seq_lens, int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
    int32_t head_dim, int32_t page_size, int32_t num_pages, int32_t num_splits, float scale,
    spa_kv_dtype kv_dtype, uint32_t flags, void *out, float *lse, hipStream_t stream) {
    spa::DecodeParams p{};
    DecodePlan plan{};
    spa_status st = decode_setup(q, k_pages, v_pages, k_scales, v_scales, page_table,
                                 page_table_stride, seq_lens, batch, num_q_heads, num_kv_heads,
                                 head_dim, page_size, num_pages, num_splits, scale, kv_dtype,
                                 flags, /*producer_only=*/false, &p, &plan);
    if (st != SPA_OK || batch == 0) return st;
    if (!out) return SPA_ERR_INVALID_ARGUMENT;
    if (!aligned(out, 2) || (lse && !aligned(lse, 4))) return SPA_ERR_INVALID_ARGUMENT;
    const spa::WorkspaceLayout w =
        spa::workspace_layout(batch, num_q_heads, num_kv_heads, head_dim, num_splits);
    if (w.total > kScratchBytes) return SPA_ERR_WORKSPACE_TOO_SMALL;
    void *ws = nullptr;
    st = scratch_of_current_device(&ws, stream);
    if (st != SPA_OK) return st;
    return run_decode(p, plan, w, ws, out, lse, stream);
}

uint32_t spa_decode_default_flags(int32_t batch, int32_t num_kv_heads, int32_t num_splits,
                                  spa_kv_dtype kv_dtype, int64_t page_table_stride) {
    if (batch < 0 || num_kv_heads < 1 || num_splits < 1 || num_splits > 1024 ||
        page_table_stride < 1 || (int64_t)batch * num_kv_heads * num_splits > (int64_t)INT32_MAX)
        return 0u;
    if (kv_dtype != SPA_KV_BF16 && kv_dtype != SPA_KV_INT8 && kv_dtype != SPA_KV_FP8) return 0u;
    const DecodePlan plan = default_plan(batch, num_kv_heads, num_splits, kv_type_of(kv_dtype),
                                         page_table_stride);
    return (plan.mode == spa::DecodeMode::kHeadGrouped ? SPA_DECODE_HEAD_GROUPED
                                                       : SPA_DECODE_PAGE_SPLIT) |
           (plan.fused ? SPA_DECODE_FUSED_MERGE : SPA_DECODE_SEPARATE_MERGE);
}

spa_status spa_paged_decode_partials(const void *q, const void *k_pages, const void *v_pages,
                                     const float *k_scales, const float *v_scales,
                                     const int32_t *page_table, int64_t page_table_stride,
                                     const int32_t *seq_lens, int32_t batch,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t page_size, int32_t num_pages,
                                     int32_t num_splits, float scale, spa_kv_dtype kv_dtype,
                                     uint32_t flags, float *partial_acc, float *partial_max,
                                     float *partial_sum, hipStream_t stream) {
    spa::DecodeParams p{};
    DecodePlan plan{};
    spa_status st = decode_setup(q, k_pages, v_pages, k_scales, v_scales, page_table,
                                 page_table_stride, seq_lens, batch, num_q_heads, num_kv_heads,
                                 head_dim, page_size, num_pages, num_splits, scale, kv_dtype,
                                 flags, /*producer_only=*/true, &p, &plan);
    if (st != SPA_OK || batch == 0) return st;
    if (!partial_acc || !partial_max || !partial_sum) return SPA_ERR_INVALID_ARGUMENT;
    if (!aligned(partial_acc, 16) || !aligned(partial_max, 4) || !aligned(partial_sum, 4))
        return SPA_ERR_INVALID_ARGUMENT;
    p.part_acc = partial_acc;
    p.part_max = partial_max;
    p.part_sum = partial_sum;
    return hip_status(spa::launch_decode_producer(p, plan.kv_type, plan.mode, stream));
}

size_t spa_verify_workspace_bytes(int32_t total_q, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t num_splits) {
    if (total_q < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 || num_splits < 1)
        return 0;
    return spa::workspace_layout(total_q, num_q_heads, num_kv_heads, head_dim, num_splits).total;
}

spa_status spa_paged_verify_attention(const void *q, const void *k_pages, const void *v_pages,
                                      const float *k_scales, const float *v_scales,
                                      const int32_t *page_table, int64_t page_table_stride,
                                      const int32_t *seq_lens, const int32_t *cu_seqlens_q,
                                      int32_t batch, int32_t total_q, int32_t max_q_len,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, int32_t page_size, int32_t num_pages,
                                      int32_t num_splits, float scale, spa_kv_dtype kv_dtype,
                                      void *workspace, size_t workspace_bytes, void *out,
                                      float *lse, hipStream_t stream) {
    if (batch < 0 || total_q < 0 || num_q_heads < 1 || num_kv_heads < 1 || head_dim < 1 ||
        page_size < 1 || num_pages < 1 || num_splits < 1 || page_table_stride < 1 ||
        max_q_len < 1)
        return SPA_ERR_INVALID_ARGUMENT;
    if (num_q_heads % num_kv_heads != 0) return SPA_ERR_INVALID_ARGUMENT;
    if (kv_dtype != SPA_KV_BF16 && kv_dtype != SPA_KV_INT8 && kv_dtype != SPA_KV_FP8)
        return SPA_ERR_INVALID_ARGUMENT;
    const bool quant = kv_dtype != SPA_KV_BF16;
    if (!isfinite(scale)) return SPA_ERR_INVALID_ARGUMENT;
    if (head_dim != spa::kHeadDim || page_size != spa::kPageSize ||
        num_q_heads != spa::kGroup * num_kv_heads || num_splits > 1024 ||
        max_q_len > spa::kMaxVerifyQueryLen || !spa::verify_supported(num_kv_heads))
        return SPA_ERR_UNSUPPORTED;
    const int64_t qt = spa::verify_tokens_per_workgroup(max_q_len);
    const int64_t chunks = (max_q_len + qt - 1) / qt;
    if ((int64_t)batch * num_kv_heads * num_splits * chunks > (int64_t)INT32_MAX ||
        (int64_t)total_q * num_q_heads > (int64_t)INT32_MAX)
        return SPA_ERR_UNSUPPORTED;
    if (batch == 0 || total_q == 0) return SPA_OK;
    if (!q || !k_pages || !v_pages || !page_table || !seq_lens || !cu_seqlens_q || !out ||
        !workspace)
        return SPA_ERR_INVALID_ARGUMENT;
    if (quant && (!k_scales || !v_scales)) return SPA_ERR_INVALID_ARGUMENT;
    if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
        !aligned(workspace, 16) || !aligned(out, 16) || !aligned(page_table, 4) ||
        !aligned(seq_lens, 4) || !aligned(cu_seqlens_q, 4) || (lse && !aligned(lse, 4)) ||
        (quant && (!aligned(k_scales, 4) || !aligned(v_scales, 4))))
        return SPA_ERR_INVALID_ARGUMENT;
    const spa::WorkspaceLayout w =
        spa::workspace_layout(total_q, num_q_heads, num_kv_heads, head_dim, num_splits);
    if (workspace_bytes < w.total) return SPA_ERR_WORKSPACE_TOO_SMALL;

    char *ws = static_cast<char *>(workspace);
    spa::DecodeParams p{};
    p.q = q;
    p.k_pages = k_pages;
    p.v_pages = v_pages;
    p.k_scales = k_scales;
    p.v_scales = v_scales;
    p.page_table = page_table;
    p.pt_stride = page_table_stride;
    p.seq_lens = seq_lens;
    p.batch = batch;
    p.hq = num_q_heads;
    p.hkv = num_kv_heads;
    p.splits = num_splits;
    p.num_pages = num_pages;
    p.qk_scale_log2 = scale * 1.4426950408889634f;
    p.part_acc = reinterpret_cast<float *>(ws + w.acc_off);
    p.part_max = reinterpret_cast<float *>(ws + w.max_off);
    p.part_sum = reinterpret_cast<float *>(ws + w.sum_off);
    p.counters = nullptr;
    p.out = static_cast<uint16_t *>(out);
    p.lse = lse;
    p.cu_seqlens_q = cu_seqlens_q;
    p.total_q = total_q;
    return hip_status(spa::launch_verify(p, kv_type_of(kv_dtype), max_q_len, stream));
}

spa_status spa_split_merge(const float *partial_acc, const float *partial_max,
                           const float *partial_sum, int32_t batch, int32_t num_q_heads,
                           int32_t head_dim, int32_t num_splits, void *out, float *lse,
                           hipStream_t stream) {
    if (batch < 0 || num_q_heads < 1 || head_dim < 1 || head_dim > 4096 || num_splits < 1 ||
        num_splits > 1024)
        return SPA_ERR_INVALID_ARGUMENT;
    if ((int64_t)batch * num_q_heads > (int64_t)INT32_MAX) return SPA_ERR_UNSUPPORTED;
    if (batch == 0) return SPA_OK;
    if (!partial_acc || !partial_max || !partial_sum || !out) return SPA_ERR_INVALID_ARGUMENT;
    if (!aligned(partial_acc, 4) || !aligned(partial_max, 4) || !aligned(partial_sum, 4) ||
        !aligned(out, 2) || (lse && !aligned(lse, 4)))
        return SPA_ERR_INVALID_ARGUMENT;
    return hip_status(spa::launch_split_merge(partial_acc, partial_max, partial_sum,
                                              batch * num_q_heads, head_dim, num_splits,
                                              static_cast<uint16_t *>(out), lse, stream));
}

}  // extern "C"
