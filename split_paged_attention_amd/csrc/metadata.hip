// Decode metadata in one launch: page table, cache_seqlens, cu_seqlens_k and
// the optional cu_seqlens_q, sliding-window page table and swa_out_cache_loc.
//
// Definition: sglang "trtllm_mha_graph_metadata.py" (module docstring; the
// kernel's per-row branch with its sliding-window part, its single-program
// cumsum branch with the two computed cu_seqlens_q modes, its swa-out branch;
// the launcher's early return for an empty batch, its num_out_tokens and its
// grid).  Workgroup i < bs rewrites page-table row i (and the sliding-window
// row, from the same req_to_token load) and cache_seqlens[i]; workgroup bs
// scans cache_seqlens (and qlens) into cu_seqlens_k (and cu_seqlens_q); the
// workgroups after it translate and zero-pad swa_out_cache_loc, kOutTile
// entries each.  All of it is a few KB of int32/int64 gathers: what matters
// is the single launch in place of many host-dispatched ops, so the kernel is
// built for latency (one dependent load chain per workgroup, wave-level
// scans with a single barrier per 256 entries).
#include "internal.h"

namespace spa {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kOutPerThread = 4;

// floor(a / b) for b > 0, also for negative a (slot -1 -> page -1).
__device__ __forceinline__ int32_t floor_div_pos(int32_t a, int32_t b) {
    int32_t q = a / b;
    return (a % b != 0 && a < 0) ? q - 1 : q;
}

__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t up = (uint32_t)__shfl_up((int)v, off, 64);
        if (lane >= off) v += up;
    }
    return v;
}

// Inclusive scan (mod 2^32) of n values given by load(i), written to
// dst[1 + i] as int32, with dst[0] = 0.  One workgroup; wave sums go through
// LDS, so each 256-entry block costs one barrier pair.
template <typename Load>
__device__ void block_scan_to(int32_t *__restrict__ dst, int32_t n, Load load,
                              uint32_t *wave_sums) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (tid == 0) dst[0] = 0;
    uint32_t carry = 0;
    for (int32_t base = 0; base < n; base += kThreads) {
        const int32_t i = base + tid;
        const uint32_t v = wave_inclusive_scan(i < n ? load(i) : 0u);
        if (lane == 63) wave_sums[wave] = v;
        __syncthreads();
        uint32_t before = carry, total = carry;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t s = wave_sums[w];
            if (w < wave) before += s;
            total += s;
        }
        if (i < n) dst[1 + i] = (int32_t)(before + v);
        carry = total;
        __syncthreads();   // wave_sums is rewritten by the next block
    }
}

__global__ __launch_bounds__(kThreads) void build_metadata_kernel(MetadataParams p) {
    const int tid = threadIdx.x;
    const int64_t wg = blockIdx.x;
    if (wg < p.bs) {
        const int32_t i = (int32_t)wg;
        const int32_t row_id = p.req_pool_indices[i];
        if (tid == 0)
            p.cache_seqlens[i] = (int32_t)((uint32_t)p.seq_lens[i] + (uint32_t)p.seqlen_offset);
        // A pool index outside the pool leaves the row's tables untouched
        // rather than reading outside req_to_token.
        if ((uint32_t)row_id >= (uint32_t)p.pool_size) return;
        const int64_t row = row_id;
        const int32_t *src = p.req_to_token + row * p.req_to_token_stride;
        int32_t *dst = p.page_table + (int64_t)i * p.page_table_stride;
        int32_t *swa_dst = p.swa_page_table
                               ? p.swa_page_table + (int64_t)i * p.swa_page_table_stride
                               : nullptr;
        for (int32_t c = tid; c < p.max_seq_pages; c += kThreads) {
            const int32_t token = src[(int64_t)c * p.page_size];
            dst[c] = floor_div_pos(token, p.page_size);
            if (swa_dst) {
                // The map is read only at slots inside it; any negative
                // mapped slot becomes the -1 sentinel.
                const int64_t s = token >= 0 && token < p.full_to_swa_len ? p.full_to_swa[token]
                                                                           : -1;
                swa_dst[c] = s < 0 ? -1 : (int32_t)(s / p.page_size);
            }
        }
        return;
    }
    if (wg == p.bs) {
        __shared__ uint32_t wave_sums[kWaves];
        const int32_t *sl = p.seq_lens;
        const uint32_t off = (uint32_t)p.seqlen_offset;
        block_scan_to(p.cu_seqlens_k, p.bs, [=](int32_t i) { return (uint32_t)sl[i] + off; },
                      wave_sums);
        if (p.q_mode == kQModeCumsum) {
            const int32_t *ql = p.qlens;
            block_scan_to(p.cu_seqlens_q, p.bs, [=](int32_t i) { return (uint32_t)ql[i]; },
                          wave_sums);
        } else if (p.q_mode == kQModeStrided) {
            if (tid == 0) p.cu_seqlens_q[0] = 0;
            for (int32_t i = tid; i < p.bs; i += kThreads)
                p.cu_seqlens_q[1 + i] = (int32_t)((uint32_t)(i + 1) * (uint32_t)p.q_stride);
        }
        return;
    }
    // swa_out_cache_loc: translate the first num_out entries, zero the rest.
    const int64_t base = (wg - p.bs - 1) * (int64_t)(kThreads * kOutPerThread);
#pragma unroll
    for (int r = 0; r < kOutPerThread; ++r) {
        const int64_t k = base + r * kThreads + tid;
        if (k >= p.swa_out_len) break;
        int64_t v = 0;
        if (k < p.num_out) {
            const int64_t loc = p.out_cache_loc[k];
            v = loc < 0 || loc >= p.full_to_swa_len ? -1 : p.full_to_swa[loc];
        }
        p.swa_out_cache_loc[k] = v;
    }
}

}  // namespace

int64_t metadata_grid(int32_t bs, int64_t swa_out_len) {
    const int64_t tile = kThreads * kOutPerThread;
    return (int64_t)bs + 1 + (swa_out_len + tile - 1) / tile;
}

hipError_t launch_build_metadata(const MetadataParams &p, hipStream_t stream) {
    const int64_t grid = metadata_grid(p.bs, p.swa_out_cache_loc ? p.swa_out_len : 0);
    hipLaunchKernelGGL(build_metadata_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       p);
    return hipGetLastError();
}

}  // namespace spa
