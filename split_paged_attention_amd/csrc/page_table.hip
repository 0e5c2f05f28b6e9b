// Page table + cache_seqlens + cu_seqlens_k in one launch.
//
// Definition: sglang "trtllm_mha_graph_metadata.py" (module docstring; the
// kernel's per-row branch and its single-program cumsum branch; the
// launcher's early return for an empty batch and its grid of bs + 1
// programs).  Workgroup i < bs rewrites page-table row i and
// cache_seqlens[i]; workgroup bs scans seq_lens + seqlen_offset into
// cu_seqlens_k.  The work is a few KB of strided int32 gathers: the cost
// that matters is the single launch replacing many host-dispatched ops.
#include "internal.h"

namespace spa {
namespace {

constexpr int kThreads = 256;

// floor(a / b) for b > 0, also for negative a (slot -1 -> page -1).
__device__ __forceinline__ int32_t floor_div_pos(int32_t a, int32_t b) {
    int32_t q = a / b;
    return (a % b != 0 && a < 0) ? q - 1 : q;
}

__device__ __forceinline__ int32_t add_wrap(int32_t a, int32_t b) {
    return (int32_t)((uint32_t)a + (uint32_t)b);
}

__global__ __launch_bounds__(kThreads) void build_page_table_kernel(
    const int32_t *__restrict__ req_to_token, int64_t req_to_token_stride,
    const int32_t *__restrict__ req_pool_indices, const int32_t *__restrict__ seq_lens,
    int32_t bs, int32_t seqlen_offset, int32_t page_size, int32_t max_seq_pages,
    int32_t *__restrict__ page_table, int64_t page_table_stride,
    int32_t *__restrict__ cache_seqlens, int32_t *__restrict__ cu_seqlens_k) {
    const int tid = threadIdx.x;
    const int i = blockIdx.x;
    if (i < bs) {
        const int64_t row = (int64_t)req_pool_indices[i];
        if (tid == 0) cache_seqlens[i] = add_wrap(seq_lens[i], seqlen_offset);
        const int32_t *src = req_to_token + row * req_to_token_stride;
        int32_t *dst = page_table + (int64_t)i * page_table_stride;
        for (int p = tid; p < max_seq_pages; p += kThreads)
            dst[p] = floor_div_pos(src[(int64_t)p * page_size], page_size);
        return;
    }
    // Inclusive scan of cache_seqlens over bs entries, kThreads at a time.
    __shared__ int32_t buf[kThreads];
    __shared__ int32_t carry_s;
    if (tid == 0) {
        carry_s = 0;
        cu_seqlens_k[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < bs; base += kThreads) {
        const int idx = base + tid;
        int32_t v = idx < bs ? add_wrap(seq_lens[idx], seqlen_offset) : 0;
        buf[tid] = v;
        __syncthreads();
        for (int off = 1; off < kThreads; off <<= 1) {
            int32_t add = tid >= off ? buf[tid - off] : 0;
            __syncthreads();
            v = add_wrap(v, add);
            buf[tid] = v;
            __syncthreads();
        }
        const int32_t carry = carry_s;
        if (idx < bs) cu_seqlens_k[idx + 1] = add_wrap(carry, v);
        __syncthreads();
        if (tid == kThreads - 1) carry_s = add_wrap(carry, v);
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_build_page_table(const int32_t *req_to_token, int64_t req_to_token_stride,
                                   const int32_t *req_pool_indices, const int32_t *seq_lens,
                                   int32_t bs, int32_t seqlen_offset, int32_t page_size,
                                   int32_t max_seq_pages, int32_t *page_table,
                                   int64_t page_table_stride, int32_t *cache_seqlens,
                                   int32_t *cu_seqlens_k, hipStream_t stream) {
    hipLaunchKernelGGL(build_page_table_kernel, dim3(bs + 1), dim3(kThreads), 0, stream,
                       req_to_token, req_to_token_stride, req_pool_indices, seq_lens, bs,
                       seqlen_offset, page_size, max_seq_pages, page_table, page_table_stride,
                       cache_seqlens, cu_seqlens_k);
    return hipGetLastError();
}

}  // namespace spa
