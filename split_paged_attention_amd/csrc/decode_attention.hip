// Split-K paged-attention decode for gfx950 (CDNA4).
//
// What is computed (lmdeploy PR "use PDL for paged attention", Summary and
// Changes): for every request one query token attends over its cached tokens,
// which sit in 64-token pages named by a page table.  A producer cuts each
// request's pages into num_splits splits and writes per-split partial
// softmax state -- running max m, running sum l and an unnormalised output
// accumulator -- and a reducer merges the splits by log-sum-exp.  The pages
// close the producer -> reducer launch gap with CUDA programmatic dependent
// launch; gfx950 has no such launch attribute, so here the merge runs inside
// the producer launch: every split workgroup publishes its partial state with
// write-through (system-scope) stores, bumps an arrival counter for its
// (request, kv head) with a memory-side atomic, and the workgroup that
// arrives last reads all splits back from memory, merges them in split order
// and resets the counter.  No L2 writeback fence is needed, and the protocol
// does not depend on which XCD a workgroup runs on.  A separate merge kernel with the same
// per-element arithmetic serves the two-launch mode and the public merge call.
//
// Work decomposition: one workgroup per (request b, kv head, split j); its
// NW waves take the split's pages round robin (page = 64 tokens = one tile)
// and are merged in LDS at the end.  Per tile and wave:
//   * QK^T on the matrix cores: v_mfma_f32_16x16x32_bf16 with the 4 query
//     heads of the GQA group as the A rows (each head repeated in 4 rows) and
//     16 tokens as the B columns; the B operand is loaded straight from HBM,
//     lane (n, g) reading 16 bytes of token n's key (16 rows x 64 contiguous
//     bytes per load instruction).  Every lane then holds the 4 heads' scores
//     of one token.  The K tile is read once for all 4 heads.
//   * online softmax in base 2 (scale * log2 e folded into one multiply),
//     max across the 16 lanes of a row with DPP;
//   * int8 KV: key codes become exact f16 values for the f16 matrix cores
//     (query scaled by a per-head power of two), value codes exact f16
//     1152 + code for v_dot2_f32_f16, the bias removed once per split;
//   * fp8 (e4m3) KV: the same f16 matrix cores and f16 dot products; the
//     hardware converter turns codes into exact f16 values (keys at scale 1,
//     values at scale 1/256, the 256 going into the value scale);
//   * P.V, head-grouped bf16 and int8: on the matrix cores, the page's
//     values staged token-major in LDS (bf16: in the key tile, which QK^T
//     has consumed) and turned into B operands by transposed LDS reads, the
//     probabilities token-major beside them as A operands.  bf16
//     probabilities go in two bf16 terms, hi + lo: each term's products with
//     bf16 values are exact in fp32, so P.V carries them to 2^-17.
//   * P.V, page-split producer and head-grouped e4m3: on the vector ALUs,
//     v_dot2 over pairs of tokens: lane (r, c) owns dims 8c..8c+7 of tokens
//     4i + r (so one V load instruction reads 4 whole 256-byte rows), pairs
//     tokens t and t + 16 in one dot2, and gets the packed probabilities of
//     its tokens from a 512-byte per-wave LDS buffer (bf16: the hi and lo
//     terms, two dot2 each).
// The path is HBM-bound (about 4 flop per KV byte for bf16), so the design
// goal is bytes in flight and a single pass over K and V.
#include "internal.h"
#include "kernel_common.h"

namespace spa {

#ifdef SPA_TIMELINE
// Diagnostics build only: the per-wave timeline (include/spa_timeline.h).
__device__ uint64_t timeline_buf[kTimelineWaves * kTimelineSlots];
#define SPA_TL_VAL(k, v)                                                    \
    do {                                                                    \
        if (tl_on) timeline_buf[tl_row + (k)] = (uint64_t)(v);              \
    } while (0)
#define SPA_TL(k) SPA_TL_VAL(k, __builtin_amdgcn_s_memrealtime())
#else
#define SPA_TL_VAL(k, v) \
    do {                 \
    } while (0)
#define SPA_TL(k) SPA_TL_VAL(k, 0)
#endif

namespace {

// ---------------------------------------------------------------------------
// The log-sum-exp merge.  Both merge paths (the fused tail and the separate
// kernel) apply exactly the same per-element operations, in split order
// j = 0..S-1, so they give the same bits:
//   M = max_j m_j;  for each non-empty j: w = 2^((m_j - M) log2 e),
//   l = fma(w, l_j, l),  o = fma(w, acc_j, o);  out = bf16(o / l), lse = M + ln l.
// Loads are issued CH splits at a time so that their latencies overlap.
constexpr int kMergeChunk = 8;            // fused tail (VEC outputs per thread)
constexpr int kMergeChunkSeparate = 16;   // merge kernel (one output per thread)

template <int VEC>
__device__ __forceinline__ void merge_step(float mj, float lj, const float (&aj)[VEC], float M,
                                           float &l, float (&o)[VEC]) {
    if (mj == kNegInf) return;   // empty split: weight 0
    const float w = exp2_fast((mj - M) * kLog2e);
    l = __builtin_fmaf(w, lj, l);
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[v] = __builtin_fmaf(w, aj[v], o[v]);
}

template <int VEC>
__device__ __forceinline__ void merge_finish(float M, float l, const float (&o)[VEC],
                                             uint16_t *out, float *lse, bool write_lse) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) out[v] = to_bf16_bits(l > 0.f ? o[v] / l : 0.f);
    if (write_lse) *lse = l > 0.f ? M + __builtin_amdgcn_logf(l) * kLn2 : kNegInf;
}

// One output element of row (b, h), plain loads (separate merge kernel),
// CH splits per batch of loads.
template <int CH>
__device__ __forceinline__ void merge_element(const float *__restrict__ acc,
                                              const float *__restrict__ mx,
                                              const float *__restrict__ sum, int splits,
                                              int head_dim, int64_t row, int d,
                                              uint16_t *__restrict__ out,
                                              float *__restrict__ lse) {
    const float *mrow = mx + row * splits;
    const float *lrow = sum + row * splits;
    const float *arow = acc + row * splits * (int64_t)head_dim + d;
    float M = kNegInf;
    // With at most CH splits one batch of loads holds all of them, and M
    // comes from it (one memory round trip instead of two).
    const bool one_pass = splits <= CH;
    if (!one_pass) {
        for (int j0 = 0; j0 < splits; j0 += CH) {
            float mv[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u) mv[u] = mrow[min(j0 + u, splits - 1)];
#pragma unroll
            for (int u = 0; u < CH; ++u) M = fmaxf(M, mv[u]);
        }
    }
    float l = 0.f, o[1] = {0.f};
    for (int j0 = 0; j0 < splits; j0 += CH) {
        float mv[CH], lv[CH], av[CH][1];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int j = min(j0 + u, splits - 1);
            mv[u] = mrow[j];
            lv[u] = lrow[j];
            av[u][0] = arow[(int64_t)j * head_dim];
        }
        if (one_pass) {
#pragma unroll
            for (int u = 0; u < CH; ++u) M = fmaxf(M, mv[u]);
        }
#pragma unroll
        for (int u = 0; u < CH; ++u)
            if (j0 + u < splits) merge_step<1>(mv[u], lv[u], av[u], M, l, o);
    }
    merge_finish<1>(M, l, o, out + row * head_dim + d, lse != nullptr ? lse + row : nullptr,
                    lse != nullptr && d == 0);
}

// VEC consecutive elements of one row, reading state that other workgroups
// published in this launch: system-scope (cache-bypassing) buffer loads
// through descriptors based at this group's first row (rows of one group
// are contiguous).  m/l descriptor: [rows][S]; acc descriptor: [rows][S][D].
template <int VEC>
__device__ __forceinline__ void merge_vec_sys(__amdgpu_buffer_rsrc_t racc,
                                              __amdgpu_buffer_rsrc_t rmax,
                                              __amdgpu_buffer_rsrc_t rsum, int splits,
                                              int head_dim, int hl, int d0, uint16_t *out,
                                              float *lse, bool write_lse) {
    static_assert(VEC == 2 || VEC == 4 || VEC == 8, "vector width");
    constexpr int CH = kMergeChunk;
    const int mrow = hl * splits * 4;                       // byte offsets
    const int arow = (hl * splits * head_dim + d0) * 4;
    auto ldf = [&](__amdgpu_buffer_rsrc_t r, int off) { return buf_ldf<kSysCoherent>(r, off, 0); };
    float M = kNegInf;
    const bool one_pass = splits <= CH;   // as in merge_element
    if (!one_pass) {
        for (int j0 = 0; j0 < splits; j0 += CH) {
            float mv[CH];
#pragma unroll
            for (int u = 0; u < CH; ++u) mv[u] = ldf(rmax, mrow + 4 * min(j0 + u, splits - 1));
#pragma unroll
            for (int u = 0; u < CH; ++u) M = fmaxf(M, mv[u]);
        }
    }
    float l = 0.f, o[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) o[v] = 0.f;
    for (int j0 = 0; j0 < splits; j0 += CH) {
        float mv[CH], lv[CH], av[CH][VEC];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int j = min(j0 + u, splits - 1);
            mv[u] = ldf(rmax, mrow + 4 * j);
            lv[u] = ldf(rsum, mrow + 4 * j);
            const int off = arow + j * head_dim * 4;
            if constexpr (VEC == 2) {
                const uint2 w = buf_ld8<kSysCoherent>(racc, off, 0);
                av[u][0] = __uint_as_float(w.x);
                av[u][1] = __uint_as_float(w.y);
            } else {
#pragma unroll
                for (int q4 = 0; q4 < VEC / 4; ++q4) {
                    const uint4 w = buf_ld16<kSysCoherent>(racc, off + 16 * q4, 0);
                    av[u][4 * q4 + 0] = __uint_as_float(w.x);
                    av[u][4 * q4 + 1] = __uint_as_float(w.y);
                    av[u][4 * q4 + 2] = __uint_as_float(w.z);
                    av[u][4 * q4 + 3] = __uint_as_float(w.w);
                }
            }
        }
        if (one_pass) {
#pragma unroll
            for (int u = 0; u < CH; ++u) M = fmaxf(M, mv[u]);
        }
#pragma unroll
        for (int u = 0; u < CH; ++u)
            if (j0 + u < splits) merge_step<VEC>(mv[u], lv[u], av[u], M, l, o);
    }
    merge_finish<VEC>(M, l, o, out, lse, write_lse);
}

// Store that is written through to memory (system scope): visible to every
// XCD once the issuing wave's store counter drains, with no L2 writeback.
__device__ __forceinline__ void st_sys(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------------------
// Producer (+ fused merge).
// HG = false: a workgroup is one (request, kv head, split); its NW waves take
//             the split's pages round robin and are merged through LDS.
// HG = true:  a workgroup is one (request, block of NW kv heads, split); wave w
//             is kv head block*NW + w and walks all the split's pages, so the
//             NW waves read the same token rows of the same pages together.
// KV: 0 = bf16 pages, 1 = int8 codes, 2 = e4m3 codes (1 and 2 with fp32
// scales per token and kv head).
// One stashed split state: 4 heads x D accumulators, then 4 maxima and 4 sums.
constexpr int kStashFloats = kGroup * kHeadDim + 2 * kGroup;

template <int KV, int NW, bool FUSED, bool HG>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(KV != 0 && HG ? 3 : 2)))
void decode_kernel(DecodeParams p,
                                                        const int32_t *__restrict__ page_table,
                                                        const int32_t *__restrict__ seq_lens) {
    constexpr int D = kHeadDim, P = kPageSize;
    constexpr bool QUANT = KV != 0;        // 1-byte codes + scales, f16 arithmetic
    constexpr bool I8 = KV == 1;
    // Head-grouped: K rows staged through LDS (see ktile); the page-split
    // producer of small grids loads K straight into operand registers, one
    // LDS round trip shorter per page.
    constexpr bool KSTAGE = HG;
    // K/V are read once, so they stream past the caches (non-temporal
    // loads: a plain paged read of the same layout runs 12% faster so, and
    // the producer 3% (bf16) to 12% (1-byte codes) at batch 32 / 8K).
    constexpr int KV_POLICY = kStreaming;
    const int lane = threadIdx.x & 63;
    // wave index is uniform per wave; say so, so that page ids, buffer
    // descriptors and loop bounds live in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#ifdef SPA_TIMELINE
    const size_t tl_wave = (size_t)blockIdx.x * NW + wave;
    const bool tl_on = lane == 0 && tl_wave < kTimelineWaves;
    const size_t tl_row = tl_wave * kTimelineSlots;
#endif
    SPA_TL(kTlEntry);
    const int n = lane & 15, g = lane >> 4;     // QK layout: token n of a 16-block, k-chunk g
    const int vr = lane >> 4, vc = lane & 15;   // PV layout: token phase r, dims 8c..8c+7

    // blockIdx -> (group = request rank * groups per request + kv block,
    // split j).  Dispatch is round robin over the 8 XCDs, so ids congruent
    // mod 8 share an XCD and its L2.  For 1-byte codes with a batch that is
    // a multiple of 8, every kv block and split of a request run on one XCD,
    // which then reads whole token rows of its requests' pages (and their
    // interleaved per-head scales, fetched once instead of once per kv
    // block) through one L2 (measured: 7% faster for int8 and fp8 at batch
    // 32 / 8K, 2% slower for bf16); the longest-first ranks are dealt to the
    // XCDs in serpentine order (ragged int8 batch: 71.5 -> 64.7 us against
    // round robin).  Otherwise the S splits of a group share an XCD.
    const int S = p.splits;
    // Lane i holds request i's length (the walk choice and, for batches of
    // up to 64, the request ranking below read it).
    const int Li = lane < p.batch ? seq_lens[lane] : INT32_MIN;
    // A head-grouped bf16 or e4m3 workgroup may walk `walk` consecutive
    // splits (S a multiple of it), one page pipeline across the split boundaries, the
    // states of all but its last split kept in LDS until the walk ends: grids
    // larger than the GPU's resident workgroups then run in one round, and
    // the later splits skip the workgroup start (request ranking, page-id
    // and first-page latency).  Each split's arithmetic is unchanged.  With
    // the fused merge a group's S splits arrive as its S / walk workgroups.
    // When the walked grid is about one round of resident workgroups, the
    // walk is taken only for a batch whose requests have about the same
    // number of pages (pages_balanced): in a ragged batch the longest
    // requests' walks would trail the rest (batch 32, 16 splits, graph
    // replay, walking 8 against one split per workgroup: lengths U[1, 8K]
    // 142.5 / 105.0 us, U[2K, 8K] 148.2 / 119.8, U[6K, 8K] 161.1 / 168.7,
    // all 8K 175.7 / 186.0).  The grid then has a workgroup per split, and
    // when the batch walks, those past the walked grid exit at once.  A
    // walked grid of several rounds always walks (walk_checked = 0, grid
    // cut): the dispatcher evens out the workgroups' lengths.
    int walk = 1;
    if constexpr (HG && !I8) {
        if (p.split_walk > 1 &&
            (!p.walk_checked || pages_balanced(seq_lens, p.batch, Li, p.pt_stride * P, P, lane)))
            walk = p.split_walk;
    }
    const int SG = S / walk;                        // split groups per kv group
    const int kv_per_grp = HG ? NW : 1;             // kv heads per workgroup
    const int grp_per_b = p.hkv / kv_per_grp;
    const int ngroups = p.batch * grp_per_b;
    if ((int64_t)blockIdx.x >= (int64_t)ngroups * SG) return;
    int grp, j;
    {
        const int bid = blockIdx.x;
        const int xcd = bid & 7, slot = bid >> 3;
        if (QUANT && (p.batch & 7) == 0) {
            j = slot % SG;
            const int rest = slot / SG;
            // ranks dealt to the XCDs in serpentine order (0..7, then 7..0,
            // ...), so each XCD's share of a ragged batch sums to about the
            // same length
            const int row = rest / grp_per_b;
            const int rank = row * 8 + ((row & 1) ? 7 - xcd : xcd);
            grp = rank * grp_per_b + rest % grp_per_b;
        } else if ((ngroups & 7) == 0) {
            grp = (slot / SG) * 8 + xcd;
            j = slot % SG;
        } else {
            grp = bid / SG;
            j = bid % SG;
        }
        j *= walk;                                  // first split of this workgroup
    }
    // Requests are taken longest first (rank r = r-th longest, ties by
    // index), so that in a ragged batch the long splits start early instead
    // of trailing behind the short ones.  Batches of more than 64 requests
    // keep their natural order.
    const int r = grp / grp_per_b;
    const int kvblock = grp - r * grp_per_b;
    int b, L;
    if (p.batch == 1) {   // nothing to rank: the query load need not wait for seq_lens
        b = 0;
        L = seq_lens[0];
    } else if (p.batch <= 64) {
        // (equal lengths skip the ranking: rank r is request r; batch 32 /
        // 8K producer 162.2 -> 161.0 us bf16, 95.9 -> 94.7 us fp8)
        b = r;
        if (__ballot(lane < p.batch && Li != __builtin_amdgcn_readfirstlane(Li)) != 0) {
            int rank = 0;
            for (int k = 0; k < p.batch; ++k) {
                const int Lk = __builtin_amdgcn_readlane(Li, k);
                rank += (Lk > Li) || (Lk == Li && k < lane);
            }
            const unsigned long long hit = __ballot(lane < p.batch && rank == r);
            b = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
        }
        L = __builtin_amdgcn_readlane(Li, b);
    } else {
        b = r;
        L = seq_lens[b];
    }
    // A length the page-table row cannot cover is cut to the row, so the
    // page-id loads stay inside it.
    L = (int)min((int64_t)max(L, 0), p.pt_stride * P);
    SPA_TL(kTlLength);
    const int kvh = kvblock * kv_per_grp + (HG ? wave : 0);
    const int pages = (L + P - 1) / P;
    const int pps = (pages + S - 1) / S;
    const int pg0 = min(j * pps, pages);
    const int pg1 = min(j * pps + walk * pps, pages);   // end of this workgroup's pages
    int jcur = j;                                        // split being accumulated
    int split_end = min(pg0 + pps, pages);               // its end page
    // Head-grouped walks: states of completed splits before the last, per
    // wave (walk - 1) x kStashFloats floats of dynamic LDS.
    extern __shared__ __attribute__((aligned(16))) float stash[];
    int nstash = 0;
    const int row_stride = p.hkv * D;           // elements between consecutive token rows

    // A operand: row i of the MFMA is query head (kvh*4 + (i & 3)).  The
    // contraction may visit the 128 dims in any order as long as A and B
    // agree: bf16 k-chunk g of MFMA c covers dims 32c + 8g .. +8 (a 16-byte
    // key load per chunk); 1-byte codes use dims 64(c/2) + 16g + 8(c%2) .. +8,
    // so that one 16-byte key load per lane feeds two MFMAs.
    bf16x8_t qa[4];
    {
        const uint16_t *qp = reinterpret_cast<const uint16_t *>(p.q) +
                             ((int64_t)b * p.hq + kvh * kGroup + (n & 3)) * D;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int d0 = QUANT ? 64 * (c >> 1) + 16 * g + 8 * (c & 1) : 32 * c + 8 * g;
            qa[c] = *reinterpret_cast<const bf16x8_t *>(qp + d0);
        }
    }
    // int8 KV: the scores use the f16 matrix cores with exact f16 key codes,
    // so the query goes to f16 too, each head scaled by a power of two that
    // puts its largest |q| in [2^14, 2^15) (exact: a bf16 value has 8
    // significant bits); qinv[h] undoes the scaling on the scores.
    f16x8_t qa16[4];
    float qinv[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (QUANT) {
        float amax = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)qa[c][e]));
        amax = max_xor32(max_xor16(amax));   // lane n: head n & 3, all 128 dims
        const int sh = amax > 0.f ? 15 - __builtin_amdgcn_frexp_expf(amax) : 0;
        const float up = __builtin_ldexpf(1.f, sh);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int e = 0; e < 8; ++e) qa16[c][e] = (_Float16)((float)qa[c][e] * up);
#pragma unroll
        for (int h = 0; h < 4; ++h)
            qinv[h] = __builtin_ldexpf(1.f, -__builtin_amdgcn_readlane(sh, h));
    }
    float qscale[4];   // score factor per head, times the key scale of a token
#pragma unroll
    for (int h = 0; h < 4; ++h) qscale[h] = p.qk_scale_log2 * qinv[h];

    float m[4], lpart[4], acc[4][8], psum[4];
    // Matrix-core P.V state (head-grouped int8 codes): oacc[T] is the
    // 16 x 16 output tile of dims 16T .. 16T + 15, rows 4g + h = head h (the
    // four row groups hold the same values), column j = dim 16T + j; for
    // int8, pacc has the sums of P' (value codes carry a bias of 1152).
    f32x4_t oacc[8], pacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 8; ++t) oacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        m[h] = kNegInf;
        lpart[h] = 0.f;
        psum[h] = 0.f;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;
    }

    // Head-grouped int8 codes and bf16 run P.V on the matrix cores (see
    // below); e4m3 codes and the page-split producer on the vector ALU.
    constexpr bool MXPV = I8 && HG;
    constexpr bool BFPV = !QUANT;                        // bf16, both producers
    constexpr bool VPV = !MXPV && !BFPV;                 // vector-ALU P.V
    __shared__ uint32_t pbuf[VPV ? NW : 1][8][4][4];      // [wave][pair u][phase r][head]
    __shared__ float sm_m[NW][4], sm_l[NW][4];
    __shared__ float sm_acc[HG ? 1 : NW][4][HG ? 1 : D];   // page split: waves' states
    // Head-grouped: the page's K rows, staged per wave: loaded as whole rows
    // (bf16: 4 rows of 256 bytes per load instruction, which memory serves
    // about 6% faster than 16 rows x 64 bytes; 1-byte codes: 8 rows of 128
    // bytes) and read back in the matrix-core operand layout; rows padded by
    // 16 bytes so the 16 token rows of an operand read fall in different LDS
    // banks.
    // Staged 1-byte codes skip the registers: buffer loads write the rows
    // straight into the tile (16 bytes per lane, lane-linear in LDS), which
    // frees the 32 registers a page of K would hold and lets 3 waves share a
    // SIMD.  The rows are then unpadded; instead 16-byte chunk h of row r sits
    // at chunk h ^ (r & 7), so the 16 rows of an operand read still spread
    // over the banks.
    constexpr bool KDMA = QUANT && KSTAGE;
    constexpr int KROWB = KDMA ? D : D * (QUANT ? 1 : 2) + 16;   // bytes per staged row
    __shared__ __attribute__((aligned(16))) uint8_t ktile[KSTAGE ? NW : 1][KSTAGE ? P : 1][KROWB];
    // Matrix-core P.V, per wave: the page's probabilities token-major, 4
    // heads per 8-byte row (int8: P' in f16, value scale folded in; bf16:
    // hi and lo terms); and the values (int8: half a page of codes, 32 token
    // rows of 128 bytes, padded by 16 so that the 8 rows of a transposed read
    // fall in distinct banks; bf16: the whole page in the key tile).
    // Transposed reads turn both into operands whose contraction runs over
    // tokens.
    constexpr int VROWB = D + 16;
    __shared__ __attribute__((aligned(16))) uint16_t ptile[MXPV || BFPV ? NW : 1][MXPV || BFPV ? P : 1][4];
    // bf16: the probabilities' low terms (p = hi + lo to 16 significant bits;
    // both terms' products with bf16 values are exact in fp32, so P.V
    // carries p to 2^-17 instead of the 2^-9 of one bf16 term, which can
    // cost 0.007 on an output of a few tokens)
    __shared__ __attribute__((aligned(16))) uint16_t ptile_lo[BFPV ? NW : 1][BFPV ? P : 1][4];
    // bf16 page split (no key tile): half a page of values at a time, rows
    // as the key tile's
    constexpr int VROWB16 = 2 * D + 16;
    __shared__ __attribute__((aligned(16))) uint8_t vtile16[BFPV && !HG ? NW : 1][BFPV && !HG ? P / 2 : 1][VROWB16];
    __shared__ __attribute__((aligned(16))) uint8_t vtile[MXPV ? NW : 1][MXPV ? P / 2 : 1][MXPV ? VROWB : 1];
    __shared__ int sm_last;

    const int32_t *pt_row = page_table + (int64_t)b * p.pt_stride;

    // Tile registers.  K in MFMA B layout: lane (n, g) holds token 16t + n,
    // dims 32c + 8g .. +8.  V in P.V layout: lane (r, c) holds token 4i + r,
    // dims 8c .. 8c+7.  One page = 64 tokens per tile.
    //
    // Loads go through a buffer resource per (page, kv head) whose range ends
    // after the page's last valid token row: rows past the context read as 0
    // without touching memory (so V needs no masking), and a zero range turns
    // the prefetch past the split's last page into a no-op.
    constexpr int ES = QUANT ? 1 : 2;                     // bytes per element
    const int row_bytes = row_stride * ES;
    const int k_lane = (n * row_stride + (QUANT ? 16 : 8) * g) * ES;   // byte offsets in a page
    const int v_lane = (vr * row_stride + 8 * vc) * ES;
    // staged 1-byte K: lane l loads 16 bytes of token row l / 8 of each 8-row
    // block, at byte 16 (l % 8)
    const int k8_row = lane >> 3;
    // direct-to-LDS 1-byte K: lane l writes tile bytes 16 l .. of an 8-row
    // block, i.e. row l / 8, chunk l % 8, which holds the row's chunk
    // (l % 8) ^ (l / 8)
    const int k8_dma = k8_row * row_bytes + (((lane & 7) ^ k8_row) << 4);
    // A loop iteration handles one page of this wave's page sequence (two
    // pages per iteration for 1-byte codes measured slower: 256 registers).
    uint4 kr[4][4];          // bf16 K (staged: kr[i/4][i%4] = token 4i + vr, dims 8vc ..)
    uint4 vr16[16];          // bf16 V
    uint4 kr8[4][2];         // int8 / e4m3 K codes: [t][c/2], 16 per lane
                             // (staged: kr8[i/2][i%2] = token 8i + l/8, bytes 16 (l%8) ..)
    uint2 vr8[16];           // int8 / e4m3 V codes
    // Scales of a page: lane l holds token l's (one load per page and
    // tensor); lane (n, g) fetches token 16t + n's with a lane permute when
    // it needs it.  e4m3 value scales are stored times 256.
    float ksc_tok, vsc_tok, vsc_next;
    const int s_lane64 = lane * p.hkv * 4;
    auto rsrc = [&](const void *base, int64_t page, int64_t elem_per_page, int64_t elem_off,
                    int esize, int nbytes) {
        const char *ptr = static_cast<const char *>(base) + (page * elem_per_page + elem_off) * esize;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(ptr), (short)0, nbytes,
                                                 kBufferWord3);
    };
    auto load_k_scales = [&](int64_t page, int valid_rows) {
        const auto rs = rsrc(p.k_scales, page, (int64_t)P * p.hkv, kvh, 4, valid_rows * p.hkv * 4);
        ksc_tok = buf_ldf(rs, s_lane64, 0);
    };
    // K codes (and, unstaged, the key scales: staged K is requested before
    // the current page's scores use the current scales)
    // (rows 16 t0 .. 16 t1 - 1 of the page: staged K goes out in two halves)
    auto load_k = [&](int64_t page, int valid_rows, int t0 = 0, int t1 = 4) {
        const auto r = rsrc(p.k_pages, page, (int64_t)P * row_stride, (int64_t)kvh * D, ES,
                            valid_rows * row_bytes);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if (t < t0 || t >= t1) continue;
            if constexpr (KSTAGE && !QUANT) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    kr[t][c] = buf_ld16<KV_POLICY>(r, v_lane, 4 * (4 * t + c) * row_bytes);
            } else if constexpr (KSTAGE) {
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2) {
                    const int blk = 2 * t + c2;          // rows 8 blk .. 8 blk + 7
                    buf_ld16_lds<KV_POLICY>(r, &ktile[wave][8 * blk][0], k8_dma,
                                            8 * blk * row_bytes);
                }
            } else if constexpr (!QUANT) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    // (default policy: each 128-byte line of a row comes
                    // from two 64-byte loads.  Over the bf16 policy sweep,
                    // page sets rotated over a 1 GiB pool, streaming them
                    // measured 2.6% slower in geometric mean: 4-9% slower
                    // where a wave reads 2 or more pages of a split, 4-5%
                    // faster below one page)
                    kr[t][c] = buf_ld16<0>(r, k_lane + 64 * c, 16 * t * row_bytes);
            } else {
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2)
                    // (default policy, as for bf16 above: a row's two
                    // 64-byte halves come from two loads; streamed, 6.5%
                    // slower in geometric mean over the int8 and fp8
                    // policy sweeps)
                    kr8[t][c2] = buf_ld16<0>(r, k_lane + 64 * c2, 16 * t * row_bytes);
            }
        }
        if constexpr (QUANT && !KSTAGE) load_k_scales(page, valid_rows);
    };
    // V in two halves (tokens 0..31, 32..63): P.V consumes the first half's
    // registers first, so the next page's first half can be requested early.
    auto load_v_half = [&](int64_t page, int valid_rows, int half) {
        const auto r = rsrc(p.v_pages, page, (int64_t)P * row_stride, (int64_t)kvh * D, ES,
                            valid_rows * row_bytes);
#pragma unroll
        for (int i = 8 * half; i < 8 * half + 8; ++i) {
            if constexpr (!QUANT)
                vr16[i] = buf_ld16<KV_POLICY>(r, v_lane, 4 * i * row_bytes);
            else
                vr8[i] = buf_ld8<KV_POLICY>(r, v_lane, 4 * i * row_bytes);
        }
    };
    // value scales of a page, requested a whole page ahead (with the next
    // page's K) into vsc_next; vsc_tok takes them at the end of an iteration
    auto load_v_scales = [&](int64_t page, int valid_rows) {
        const auto rs = rsrc(p.v_scales, page, (int64_t)P * p.hkv, kvh, 4, valid_rows * p.hkv * 4);
        vsc_next = buf_ldf(rs, s_lane64, 0);
    };

    // Partial-state writes: write-through stores in the fused mode (read back
    // by another workgroup in this launch), plain stores otherwise.
    auto put = [&](float *ptr, float v) {
        if constexpr (FUSED) st_sys(ptr, v);
        else *ptr = v;
    };
    // Wave state of a finished split: the int8 value bias removed, l summed
    // over the 16 lanes of a row, acc over the 4 token phases.
    auto reduce_state = [&]() {
        if constexpr (I8) {
            // remove the 1152 bias carried by every f16 value code
#pragma unroll
            for (int h = 0; h < 4; ++h)
#pragma unroll
                for (int d = 0; d < 8; ++d) acc[h][d] = __builtin_fmaf(-kI8Bias, psum[h], acc[h][d]);
        }
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            lpart[h] = row_sum16(lpart[h]);
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                float x = acc[h][d];
                x = add_xor32(add_xor16(x));
                acc[h][d] = x;
            }
        }
    };
    auto reset_state = [&]() {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            m[h] = kNegInf;
            lpart[h] = 0.f;
            psum[h] = 0.f;
#pragma unroll
            for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;
        }
    };
    // Head-grouped: the reduced state of this wave's kv head as split jw's
    // partial state.
    // Head-grouped: the empty state (no tokens) as split jw's partial state.
    auto store_empty = [&](int jw) {
        const int64_t idx0 = ((int64_t)b * p.hq + kvh * kGroup) * S + jw;
        const int off = (vr * S * D + 8 * vc) * 4;   // bytes from this wave's first row
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (FUSED) {
            const auto r = __builtin_amdgcn_make_buffer_rsrc(p.part_acc + idx0 * D, (short)0,
                                                             (3 * S + 1) * D * 4, kBufferWord3);
            buf_st16<kSysCoherent>(z, r, off);
            buf_st16<kSysCoherent>(z, r, off + 16);
        } else {
            char *base = reinterpret_cast<char *>(p.part_acc + idx0 * D) + off;
            *reinterpret_cast<uint4 *>(base) = z;
            *reinterpret_cast<uint4 *>(base + 16) = z;
        }
        if (lane < 4) {
            put(p.part_max + idx0 + (int64_t)lane * S, kNegInf);
            put(p.part_sum + idx0 + (int64_t)lane * S, 0.f);
        }
    };

    // Matrix-core P.V: this wave's split jw is complete; write its
    // partial state from the matrix-core layout (lane (j, g) holds head g at
    // dims 16T + j) and start the next split.  A bf16 split before its
    // walk's last goes to the LDS stash instead, in the [head][dim] layout
    // the stash write-out reads.
    auto finish_split_mx = [&](int jw, bool to_stash) {
        if constexpr (I8) {
            // remove the 1152 bias of the value codes
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int h = 0; h < 4; ++h) oacc[t][h] = __builtin_fmaf(-kI8Bias, pacc[h], oacc[t][h]);
        }
        // the sums over the tokens (int8: lane l holds token l's; bf16: lane
        // (n, g) tokens 16t + n, every row of 16 lanes the same)
        float lsum[4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            float x = row_sum16(lpart[h]);
            if constexpr (I8) x = add_xor32(add_xor16(x));
            lsum[h] = x;
        }
        const int64_t idx0 = ((int64_t)b * p.hq + kvh * kGroup) * S + jw;
        const int jl = lane & 15;
        const int off = (g * S * D + jl) * 4;   // bytes: head g's row, dim jl
        float o[8];
#pragma unroll
        for (int t = 0; t < 8; ++t)
            o[t] = pick4(oacc[t][0], oacc[t][1], oacc[t][2], oacc[t][3], g);
        if (to_stash) {
            float *st = stash + (wave * (walk - 1) + nstash) * kStashFloats;
#pragma unroll
            for (int t = 0; t < 8; ++t) st[g * D + 16 * t + jl] = o[t];
            if (lane == 0) {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    st[4 * D + h] = m[h];
                    st[4 * D + 4 + h] = lsum[h];
                }
            }
            ++nstash;
        } else if constexpr (FUSED) {
            const auto r = __builtin_amdgcn_make_buffer_rsrc(p.part_acc + idx0 * D, (short)0,
                                                             (3 * S + 1) * D * 4, kBufferWord3);
#pragma unroll
            for (int t = 0; t < 8; ++t) buf_st4<kSysCoherent>(__float_as_uint(o[t]), r, off + 64 * t);
        } else {
            float *base = reinterpret_cast<float *>(reinterpret_cast<char *>(p.part_acc + idx0 * D) + off);
#pragma unroll
            for (int t = 0; t < 8; ++t) base[16 * t] = o[t];
        }
        if (!to_stash && lane == 0) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                put(p.part_max + idx0 + (int64_t)h * S, m[h] == kNegInf ? kNegInf : m[h] * kLn2);
                put(p.part_sum + idx0 + (int64_t)h * S, lsum[h]);
            }
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) oacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        pacc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            m[h] = kNegInf;
            lpart[h] = 0.f;
        }
    };

    // Software pipeline over this wave's pages: the next page's K loads are
    // issued as soon as QK^T has consumed the K registers, each half of its V
    // loads as soon as P.V has consumed that half of the V registers, so
    // loads stay in flight while the current page is computed.
    constexpr int PSTEP = HG ? 1 : NW;              // page stride of one wave
    int pg = HG ? pg0 : pg0 + wave;
    // Rows of logical page i that are loaded: a page id outside the pool is
    // loaded with a zero range (reads 0, touches no memory) instead of
    // faulting, so a bad page table gives wrong numbers, never a fault; a
    // page at or past the split's end loads nothing.
    auto page_rows = [&](int i, int64_t &page) {
        page = 0;
        if (i >= pg1) return 0;
        const int32_t id = pt_row[i];
        const bool ok = (uint32_t)id < (uint32_t)p.num_pages;
        page = ok ? id : 0;
        return ok ? min(P, L - i * P) : 0;
    };
    if (pg < pg1) {
        int64_t page;
        const int rows = page_rows(pg, page);
        SPA_TL(kTlFirstPageId);
        load_k(page, rows);
        if constexpr (QUANT && KSTAGE) load_k_scales(page, rows);
        load_v_half(page, rows, 0);
        load_v_half(page, rows, 1);
        if constexpr (QUANT) {
            load_v_scales(page, rows);
            vsc_tok = vsc_next * (I8 ? 1.f : kF8ValueScale);
        }
    }
    // The matrix-core P.V loop keeps its loads in flight across iterations;
    // the first page's loads complete before it starts, so the compiler's
    // wait insertion, which merges the state on entry with the loop's own,
    // does not make every iteration wait for them.
    if constexpr (MXPV) __builtin_amdgcn_s_waitcnt(kWaitVm0);
    SPA_TL_VAL(kTlWhat, (uint64_t)b | ((uint64_t)kvh << 16) | ((uint64_t)j << 32));
    SPA_TL_VAL(kTlPages, pg1 - pg0);
    [[maybe_unused]] const int pg_first = pg;
    for (; pg < pg1; pg += PSTEP) {
        int64_t page_next;
        const int valid_next = page_rows(pg + PSTEP, page_next);
        const int valid = min(P, L - pg * P);       // tokens of this page that count

        if constexpr (MXPV) {
            // ---- this page's K rows are in the tile: the loads issued after
            // their direct-to-LDS loads are the two V halves (16 instructions).
            // (The builtin, unlike an asm wait, is seen by the compiler's own
            // wait insertion, which then knows the older loads are done.)
            __builtin_amdgcn_s_waitcnt(kWaitVm16);
            __builtin_amdgcn_sched_barrier(0);
            load_v_scales(page_next, valid_next);
            __builtin_amdgcn_sched_barrier(0);
            // ---- S = Q K^T: lane (n, g) gets s[head h][token 16t + n] in sacc[t][h]
            uint8_t(*kt)[KROWB] = ktile[wave];
            f32x4_t sacc[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                sacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint2 h = *reinterpret_cast<const uint2 *>(
                        &kt[16 * t + n][(((4 * (c >> 1) + g) ^ (n & 7)) << 4) + 8 * (c & 1)]);
                    sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        qa16[c], i8x8_to_f16(h), sacc[t], 0, 0, 0);
                }
            }
            // From here on lane (n, g) takes token 16g + n, its own lane
            // index: the scores of tile g (every row group holds all 4 heads
            // of every tile), and the key and value scales it loaded itself.
            // Tokens past the context get -inf (the minimum with -inf).
            float sc[4];
            {
                const float lim = lane < valid ? kPosInf : kNegInf;
                const float kts = ksc_tok;
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float x = pick4(sacc[0][h], sacc[1][h], sacc[2][h], sacc[3][h], g);
                    sc[h] = fminf(x * (qscale[h] * kts), lim);
                }
            }
            if (pg == pg_first) SPA_TL(kTlFirstScores);
            __builtin_amdgcn_sched_barrier(0);
            load_k_scales(page_next, valid_next);   // after the scores' last read
            // the next page's K rows go into the tile once this page's
            // operand reads have returned
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            load_k(page_next, valid_next, 0, 4);
            __builtin_amdgcn_sched_barrier(0);

            // ---- online softmax (base 2); maxima over the wave's 64 tokens
            float alpha[4], pr[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float mx = wave_max(sc[h]);
                const float mnew = mx > m[h] ? mx : m[h];   // (no NaN-quieting as with fmaxf)
                alpha[h] = exp2_fast(m[h] - mnew);
                m[h] = mnew;
                pr[h] = exp2_fast(sc[h] - mnew);
                lpart[h] = __builtin_fmaf(lpart[h], alpha[h], pr[h]);
            }
            {   // P' = p * value scale, f16 (11 significant bits), row = token
                const float vs = vsc_tok;
                *reinterpret_cast<uint2 *>(&ptile[wave][lane][0]) =
                    make_uint2(pack_f16x2(pr[0] * vs, pr[1] * vs), pack_f16x2(pr[2] * vs, pr[3] * vs));
            }
            if (alpha[0] != 1.f || alpha[1] != 1.f || alpha[2] != 1.f || alpha[3] != 1.f) {
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int h = 0; h < 4; ++h) oacc[t][h] *= alpha[h];
#pragma unroll
                for (int h = 0; h < 4; ++h) pacc[h] *= alpha[h];
            }
            __asm__ volatile("" ::: "memory");

            // ---- O += P' V on the matrix cores, one half page (32 tokens,
            // one k-step) at a time.  Contraction order: lane group G holds
            // tokens 32 hf + 8G .. +7, element e = token 32 hf + 8G + e, in
            // both operands.  A (P'): lane 16G + i gets head i & 3 through
            // two 4-token transposed reads (lane 16G + q addresses token row
            // 32 hf + 8G + 4r + q/4).  B (V): lane 16G + j gets dim 16T + j
            // through one 8-token transposed byte read (lane 16G + q addresses
            // token row 8G + q/2, bytes 16T + 8 (q & 1) ..).
            const int q16 = lane & 15;
            const int vt_rd = (wave * (P / 2) + 8 * g + (q16 >> 1)) * VROWB + 8 * (q16 & 1);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                // this half's value codes into the tile (lane (r, c): token
                // 4i + r, dims 8c .. 8c + 7)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<uint2 *>(&vtile[wave][4 * i + vr][8 * vc]) = vr8[8 * hf + i];
                __asm__ volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                const uint16_t *prow = &ptile[wave][32 * hf + 8 * g + (q16 >> 2)][0];
                const f16x8_t pa = join_f16x8(lds_tr16_b64(prow), lds_tr16_b64(prow + 16));
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    // one flat offset from the tile's base: the compiler then
                    // still knows which LDS object each read touches, and does
                    // not hold it back for the key rows' direct-to-LDS loads
                    const uint2 w = lds_tr8_b64(&vtile[0][0][0] + vt_rd + 16 * t);
                    oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        pa, i8x8_to_f16_biased(w),
                        oacc[t], 0, 0, 0);
                }
                const f16x8_t ones = {1, 1, 1, 1, 1, 1, 1, 1};
                pacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, ones, pacc, 0, 0, 0);
                __asm__ volatile("" ::: "memory");
            }
            vsc_tok = vsc_next;
            if (pg + 1 == split_end) {
                finish_split_mx(jcur, false);
                ++jcur;
                split_end = min(split_end + pps, pages);
            }
            // the next page's values, both halves, once this page's P.V has
            // issued (issued between the two halves' matrix-core steps, the
            // ragged int8 batch's producer measured 0.8% slower)
            __asm__ volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            load_v_half(page_next, valid_next, 0);
            load_v_half(page_next, valid_next, 1);
            continue;
        }


        // ---- S = Q K^T: lane (n, g) gets s[head h][token 16t + n] in sacc[t][h]
        f32x4_t sacc[4];
        if constexpr (KSTAGE) {
            // K rows into the wave's LDS tile; the registers then take the
            // next page's K at once
            uint8_t(*kt)[KROWB] = ktile[wave];
            if constexpr (!QUANT) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    *reinterpret_cast<uint4 *>(&kt[4 * i + vr][16 * vc]) = kr[i >> 2][i & 3];
            } else {
                // this page's rows were written by the loads issued after the
                // previous page's scores; the loads issued after them are the
                // two V halves (16 instructions), so vmcnt <= 16 means the K
                // rows are in the tile
                __asm__ volatile("s_waitcnt vmcnt(16)" ::: "memory");
            }
            __asm__ volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!QUANT) load_k(page_next, valid_next, 0, 2);
            if constexpr (QUANT) load_v_scales(page_next, valid_next);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                sacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
                if constexpr (!QUANT) {
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            qa[c],
                            *reinterpret_cast<const bf16x8_t *>(&kt[16 * t + n][64 * c + 16 * g]),
                            sacc[t], 0, 0, 0);
                } else {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint2 h = *reinterpret_cast<const uint2 *>(
                            &kt[16 * t + n][(((4 * (c >> 1) + g) ^ (n & 7)) << 4) + 8 * (c & 1)]);
                        sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            qa16[c], I8 ? i8x8_to_f16(h) : e4m3x8_to_f16(h), sacc[t], 0, 0, 0);
                    }
                }
            }
        } else if constexpr (!QUANT) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                sacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        qa[c], __builtin_bit_cast(bf16x8_t, kr[t][c]), sacc[t], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                sacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint4 w = kr8[t][c >> 1];
                    const uint2 h = (c & 1) ? make_uint2(w.z, w.w) : make_uint2(w.x, w.y);
                    sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        qa16[c], I8 ? i8x8_to_f16(h) : e4m3x8_to_f16(h), sacc[t], 0, 0, 0);
                }
            }
        }
        float s[4][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bool ok = (16 * t + n) < valid;
            const float kt = QUANT ? lane_value(ksc_tok, 16 * t + n) : 1.f;
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                const float f = QUANT ? qscale[h] * kt : p.qk_scale_log2;
                s[t][h] = ok ? sacc[t][h] * f : kNegInf;
            }
        }
        if (pg == pg_first) SPA_TL(kTlFirstScores);
        if constexpr (!KSTAGE) {
            // keep the prefetch after the last read of the K registers it reuses
            __builtin_amdgcn_sched_barrier(0);
            load_k(page_next, valid_next);
            if constexpr (QUANT) load_v_scales(page_next, valid_next);
            __builtin_amdgcn_sched_barrier(0);
        } else if constexpr (QUANT) {
            // the scores have read this page's key scales
            __builtin_amdgcn_sched_barrier(0);
            load_k_scales(page_next, valid_next);
            __builtin_amdgcn_sched_barrier(0);
        }

        if constexpr (KDMA) {
            // the next page's K rows go into the tile once this page's
            // operand reads have returned
            __builtin_amdgcn_sched_barrier(0);
            __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            load_k(page_next, valid_next, 0, 4);
            __builtin_amdgcn_sched_barrier(0);
        } else if constexpr (KSTAGE) {
            // the next page's K rows 32..63 (rows 0..31 went out with the tile
            // write): spread over the page, the requests measured 1% faster
            __builtin_amdgcn_sched_barrier(0);
            load_k(page_next, valid_next, 2, 4);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- online softmax (base 2)
        float alpha[4], pv[4][4];
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            float mx = fmaxf(fmaxf(s[0][h], s[1][h]), fmaxf(s[2][h], s[3][h]));
            mx = row_max16(mx);
            const float mnew = fmaxf(m[h], mx);
            alpha[h] = exp2_fast(m[h] - mnew);
            m[h] = mnew;
            float rs = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                pv[t][h] = exp2_fast(s[t][h] - mnew);
                rs += pv[t][h];
            }
            lpart[h] = __builtin_fmaf(lpart[h], alpha[h], rs);
        }

        if constexpr (BFPV) {
            // ---- this page's probabilities into the P tile, token-major,
            // hi and lo terms; lane (n, g) writes token 16g + n (every row of
            // 16 lanes holds all 64 tokens)
            {
                float a[4];
#pragma unroll
                for (int h = 0; h < 4; ++h) a[h] = pick4(pv[0][h], pv[1][h], pv[2][h], pv[3][h], g);
                const uint2 hi = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
                *reinterpret_cast<uint2 *>(&ptile[wave][lane][0]) = hi;
                *reinterpret_cast<uint2 *>(&ptile_lo[wave][lane][0]) =
                    make_uint2(bf16x2_residual(a[0], a[1], hi.x), bf16x2_residual(a[2], a[3], hi.y));
            }
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int h = 0; h < 4; ++h) oacc[t][h] *= alpha[h];
            // ---- O += P V on the matrix cores, 32 tokens per step.  A = P:
            // lane (i, G) takes head i % 4 at tokens 8G .. 8G + 7 (two
            // transposed reads of 4 token rows); B = V: lane (j, G) takes dim
            // 16T + j at tokens 8G .. 8G + 7.  The low terms go first.
            const int tr_row = 8 * g + (n >> 2), tr_col = 4 * (n & 3);
            auto pv_step = [&](int kb, const uint16_t *vbase, int vrow0) {
                // vbase: a token-major tile of rows of VROWB16 bytes whose row
                // vrow0 holds token 32 kb
                constexpr int RE = VROWB16 / 2;   // elements per row
                const uint16_t *prh = &ptile[wave][32 * kb + 8 * g + (n >> 2)][0];
                const uint16_t *prl = &ptile_lo[wave][32 * kb + 8 * g + (n >> 2)][0];
                const bf16x8_t pah = join_bf16x8(lds_tr16_b64(prh), lds_tr16_b64(prh + 16));
                const bf16x8_t pal = join_bf16x8(lds_tr16_b64(prl), lds_tr16_b64(prl + 16));
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const uint16_t *vr0 = vbase + (vrow0 + tr_row) * RE + 16 * t + tr_col;
                    const bf16x8_t vb = join_bf16x8(lds_tr16_b64(vr0), lds_tr16_b64(vr0 + 4 * RE));
                    oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pal, vb, oacc[t], 0, 0, 0);
                    oacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pah, vb, oacc[t], 0, 0, 0);
                }
            };
            if constexpr (HG) {
                // ---- this page's values into the key tile, whose rows QK^T
                // has read (a wave's LDS operations complete in order),
                // token-major like the keys; the registers then take the next
                // page's values
                static_assert(KROWB == VROWB16, "values staged in the key tile's rows");
                uint8_t(*kt)[KROWB] = ktile[wave];
                __asm__ volatile("" ::: "memory");
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    *reinterpret_cast<uint4 *>(&kt[4 * i + vr][16 * vc]) = vr16[i];
                __asm__ volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                load_v_half(page_next, valid_next, 0);
                load_v_half(page_next, valid_next, 1);
                __builtin_amdgcn_sched_barrier(0);
                const uint16_t *vbase = reinterpret_cast<const uint16_t *>(&kt[0][0]);
                pv_step(0, vbase, 0);
                pv_step(1, vbase, 32);
                // the next page's keys overwrite the tile only after these reads
                __asm__ volatile("" ::: "memory");
                if (pg + 1 == split_end) {
                    finish_split_mx(jcur, pg + 1 < pg1);
                    ++jcur;
                    split_end = min(split_end + pps, pages);
                }
            } else {
                // ---- page split: each half page of values into the wave's
                // half-page tile in turn, its registers then taking the next
                // page's half
                uint8_t(*vt)[VROWB16] = vtile16[wave];
                const uint16_t *vbase = reinterpret_cast<const uint16_t *>(&vt[0][0]);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    __asm__ volatile("" ::: "memory");
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        *reinterpret_cast<uint4 *>(&vt[4 * i + vr][16 * vc]) = vr16[8 * kb + i];
                    __asm__ volatile("" ::: "memory");
                    __builtin_amdgcn_sched_barrier(0);
                    load_v_half(page_next, valid_next, kb);
                    __builtin_amdgcn_sched_barrier(0);
                    pv_step(kb, vbase, 0);
                    // the second half overwrites the tile only after these reads
                    __asm__ volatile("" ::: "memory");
                }
            }
            continue;
        }

        // ---- vector-ALU P.V (1-byte codes: e4m3 head grouped, both codes
        // page split).  Probabilities: pair (token 32q + n, token 32q + 16 +
        // n), stored by row 0 of the wave as pbuf[pair u][phase r][h] with
        // u = 4q + n/4, r = n % 4, in f16 with the value scale folded in.
        {   // every row g holds the same values, so all lanes may store
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                uint4 w;
                float a0 = pv[2 * qq][0], a1 = pv[2 * qq][1], a2 = pv[2 * qq][2], a3 = pv[2 * qq][3];
                float b0 = pv[2 * qq + 1][0], b1 = pv[2 * qq + 1][1], b2 = pv[2 * qq + 1][2],
                      b3 = pv[2 * qq + 1][3];
                const float va = lane_value(vsc_tok, 32 * qq + n);
                const float vb = lane_value(vsc_tok, 32 * qq + 16 + n);
                a0 *= va; a1 *= va; a2 *= va; a3 *= va;
                b0 *= vb; b1 *= vb; b2 *= vb; b3 *= vb;
                // f16 keeps 11 significant bits
                w.x = pack_f16x2(a0, b0);
                w.y = pack_f16x2(a1, b1);
                w.z = pack_f16x2(a2, b2);
                w.w = pack_f16x2(a3, b3);
                *reinterpret_cast<uint4 *>(&pbuf[wave][4 * qq + (n >> 2)][n & 3][0]) = w;
            }
        }
        // LDS ops of one wave complete in order; this only stops the compiler
        // from moving the reads above the writes.
        __asm__ volatile("" ::: "memory");

        // ---- P.V.  Pair u: tokens 4*ia + r and 4*ia + r + 16, ia = u < 4 ? u : u + 4.
#pragma unroll
        for (int h = 0; h < 4; ++h) {
#pragma unroll
            for (int d = 0; d < 8; ++d) acc[h][d] *= alpha[h];
            if constexpr (I8) psum[h] *= alpha[h];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            if (u == 4) {   // tokens 0..31 done: request the next page's first half
                __builtin_amdgcn_sched_barrier(0);
                load_v_half(page_next, valid_next, 0);
                __builtin_amdgcn_sched_barrier(0);
            }
            const uint4 pk = *reinterpret_cast<const uint4 *>(&pbuf[wave][u][vr][0]);
            const int ia = u < 4 ? u : u + 4;       // token 4*ia + r
            const int ib = ia + 4;                  // token 4*ia + r + 16
            const uint32_t ph[4] = {pk.x, pk.y, pk.z, pk.w};
            {
                // codes are finite (rows past the context read as 0) and
                // masked tokens have probability 0, so no masking is needed;
                // for int8, psum tracks sum(p') for the 1152 bias.
                uint32_t vp[8];
                if constexpr (I8) {
#pragma unroll
                    for (int h = 0; h < 4; ++h) psum[h] = dot2_f16(ph[h], kF16One2, psum[h]);
                    vp[0] = i8_pair_f16<0>(vr8[ib].x, vr8[ia].x);
                    vp[1] = i8_pair_f16<1>(vr8[ib].x, vr8[ia].x);
                    vp[2] = i8_pair_f16<2>(vr8[ib].x, vr8[ia].x);
                    vp[3] = i8_pair_f16<3>(vr8[ib].x, vr8[ia].x);
                    vp[4] = i8_pair_f16<0>(vr8[ib].y, vr8[ia].y);
                    vp[5] = i8_pair_f16<1>(vr8[ib].y, vr8[ia].y);
                    vp[6] = i8_pair_f16<2>(vr8[ib].y, vr8[ia].y);
                    vp[7] = i8_pair_f16<3>(vr8[ib].y, vr8[ia].y);
                } else {
                    e4m3_pairs_f16<0>(vr8[ib].x, vr8[ia].x, vp[0], vp[1]);
                    e4m3_pairs_f16<2>(vr8[ib].x, vr8[ia].x, vp[2], vp[3]);
                    e4m3_pairs_f16<0>(vr8[ib].y, vr8[ia].y, vp[4], vp[5]);
                    e4m3_pairs_f16<2>(vr8[ib].y, vr8[ia].y, vp[6], vp[7]);
                }
#pragma unroll
                for (int d = 0; d < 8; ++d)
#pragma unroll
                    for (int h = 0; h < 4; ++h) acc[h][d] = dot2_f16(ph[h], vp[d], acc[h][d]);
            }
        }
        __asm__ volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
        load_v_half(page_next, valid_next, 1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (QUANT) vsc_tok = vsc_next * (I8 ? 1.f : kF8ValueScale);
        if constexpr (HG) {
            if (pg + 1 == split_end) {
                // split jcur complete: write its state (a split before the
                // walk's last goes to the LDS stash, written out after the
                // loop), start the next one
                reduce_state();
                if (pg + 1 < pg1) {
                    float *st = stash + (wave * (walk - 1) + nstash) * kStashFloats;
                    float v8[8];
#pragma unroll
                    for (int d = 0; d < 8; ++d)
                        v8[d] = vr == 0 ? acc[0][d] : vr == 1 ? acc[1][d] : vr == 2 ? acc[2][d] : acc[3][d];
                    *reinterpret_cast<float4 *>(st + vr * D + 8 * vc) =
                        make_float4(v8[0], v8[1], v8[2], v8[3]);
                    *reinterpret_cast<float4 *>(st + vr * D + 8 * vc + 4) =
                        make_float4(v8[4], v8[5], v8[6], v8[7]);
                    if (lane == 0) {
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            st[4 * D + h] = m[h];
                            st[4 * D + 4 + h] = lpart[h];
                        }
                    }
                    ++nstash;
                } else {
                    const int jw = jcur;
                    // One wave = one kv head: write its split state straight from
                    // registers.  After the butterfly every lane holds the reduced sums
                    // for its 8 dims, so lane group r publishes head r: two 16-byte
                    // stores per lane cover the wave's 4 heads x 128 dims.
                    const int64_t idx0 = ((int64_t)b * p.hq + kvh * kGroup) * S + jw;
                    float v8[8];
#pragma unroll
                    for (int d = 0; d < 8; ++d)
                        v8[d] = vr == 0 ? acc[0][d] : vr == 1 ? acc[1][d] : vr == 2 ? acc[2][d] : acc[3][d];
                    const uint4 lo = make_uint4(__float_as_uint(v8[0]), __float_as_uint(v8[1]),
                                                __float_as_uint(v8[2]), __float_as_uint(v8[3]));
                    const uint4 hi = make_uint4(__float_as_uint(v8[4]), __float_as_uint(v8[5]),
                                                __float_as_uint(v8[6]), __float_as_uint(v8[7]));
                    const int off = (vr * S * D + 8 * vc) * 4;   // bytes from this wave's first row
                    if constexpr (FUSED) {
                        const auto r = __builtin_amdgcn_make_buffer_rsrc(p.part_acc + idx0 * D, (short)0,
                                                                         (3 * S + 1) * D * 4, kBufferWord3);
                        buf_st16<kSysCoherent>(lo, r, off);
                        buf_st16<kSysCoherent>(hi, r, off + 16);
                    } else {
                        char *base = reinterpret_cast<char *>(p.part_acc + idx0 * D) + off;
                        *reinterpret_cast<uint4 *>(base) = lo;
                        *reinterpret_cast<uint4 *>(base + 16) = hi;
                    }
                    if (lane == 0) {
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            put(p.part_max + idx0 + (int64_t)h * S, m[h] == kNegInf ? kNegInf : m[h] * kLn2);
                            put(p.part_sum + idx0 + (int64_t)h * S, lpart[h]);
                        }
                    }
                }
                reset_state();
                ++jcur;
                split_end = min(split_end + pps, pages);
            }
        }
    }
    SPA_TL(kTlPagesDone);
    if constexpr (HG) {
        // splits of this workgroup with no pages (past the context): empty
        // states (the others were written at their last page)
        for (int jw = jcur; jw < j + walk; ++jw) store_empty(jw);
        // the stashed splits j .. j + nstash - 1
        for (int k = 0; k < nstash; ++k) {
            const float *st = stash + (wave * (walk - 1) + k) * kStashFloats;
            const int64_t idx0 = ((int64_t)b * p.hq + kvh * kGroup) * S + j + k;
            const int off = (vr * S * D + 8 * vc) * 4;   // bytes from this wave's first row
            const uint4 lo = *reinterpret_cast<const uint4 *>(st + vr * D + 8 * vc);
            const uint4 hi = *reinterpret_cast<const uint4 *>(st + vr * D + 8 * vc + 4);
            if constexpr (FUSED) {
                const auto r = __builtin_amdgcn_make_buffer_rsrc(p.part_acc + idx0 * D, (short)0,
                                                                 (3 * S + 1) * D * 4, kBufferWord3);
                buf_st16<kSysCoherent>(lo, r, off);
                buf_st16<kSysCoherent>(hi, r, off + 16);
            } else {
                char *base = reinterpret_cast<char *>(p.part_acc + idx0 * D) + off;
                *reinterpret_cast<uint4 *>(base) = lo;
                *reinterpret_cast<uint4 *>(base + 16) = hi;
            }
            if (lane < 4) {
                const float mk = st[4 * D + lane];
                put(p.part_max + idx0 + (int64_t)lane * S, mk == kNegInf ? kNegInf : mk * kLn2);
                put(p.part_sum + idx0 + (int64_t)lane * S, st[4 * D + 4 + lane]);
            }
        }
    } else {
        if constexpr (BFPV) {
            // matrix-core layout: lane (j, g) holds head g at dims 16T + j;
            // the softmax sums are per lane over tokens 16t + n, the same in
            // every row of 16 lanes
#pragma unroll
            for (int h = 0; h < 4; ++h) lpart[h] = row_sum16(lpart[h]);
            const int jl = lane & 15;
#pragma unroll
            for (int t = 0; t < 8; ++t)
                sm_acc[wave][g][16 * t + jl] = pick4(oacc[t][0], oacc[t][1], oacc[t][2], oacc[t][3], g);
        } else {
            reduce_state();
            if (lane < 16) {
#pragma unroll
                for (int h = 0; h < 4; ++h)
#pragma unroll
                    for (int d = 0; d < 8; ++d) sm_acc[wave][h][8 * vc + d] = acc[h][d];
            }
        }
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                sm_m[wave][h] = m[h];
                sm_l[wave][h] = lpart[h];
            }
        }
        __syncthreads();

        // merge the NW waves (wave order) and write this split's partial state
        const int64_t head0 = (int64_t)b * p.hq + kvh * kGroup;
        for (int e = threadIdx.x; e < kGroup * D; e += NW * 64) {
            const int h = e / D, d = e - h * D;
            float M = kNegInf;
#pragma unroll
            for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][h]);
            float l = 0.f, o = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float mw = sm_m[w][h];
                if (mw == kNegInf) continue;
                const float wt = exp2_fast(mw - M);
                l = __builtin_fmaf(wt, sm_l[w][h], l);
                o = __builtin_fmaf(wt, sm_acc[w][h][d], o);
            }
            const int64_t idx = (head0 + h) * S + j;
            put(p.part_acc + idx * D + d, o);
            if (d == 0) {
                put(p.part_max + idx, M == kNegInf ? kNegInf : M * kLn2);
                put(p.part_sum + idx, l);
            }
        }
    }

    SPA_TL(kTlStatesIssued);
    if constexpr (FUSED) {
        // Last-split-done: the partial state above went to memory with
        // write-through stores; once every wave's stores have completed, one
        // thread counts this split in with a memory-side atomic.  The split
        // that arrives last (count S-1) reads all S partial states from memory,
        // merges them in split order and resets the counter for the next call.
        // Ordering (the AMDGPU memory model's system-scope release/acquire
        // sequences for gfx94x/gfx950, with the cache maintenance they carry
        // made unnecessary): a store with sc0 sc1 writes through to memory and
        // leaves no dirty L2 line, so the release's L2 writeback has nothing
        // to do; vmcnt counts a store as done only once memory has acknowledged
        // it, so after s_waitcnt vmcnt(0) in every wave and the barrier, all
        // of the workgroup's state is in memory before the atomic is issued,
        // and no XCD can see the count without the state.  The merger's loads
        // bypass the caches (sc0 sc1) and are issued after the atomic has
        // returned, so the acquire's cache invalidation has nothing stale to
        // drop.
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        SPA_TL(kTlStatesInMemory);
        if (threadIdx.x == 0) {
            const int old = __hip_atomic_fetch_add(p.counters + grp, 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_SYSTEM);
            // (a group's splits arrive as S / walk workgroups)
            sm_last = (old == S / walk - 1);
        }
        __syncthreads();
        SPA_TL(kTlArrived);
        if (sm_last) {
            // all query heads of this workgroup's kv heads: HEADS rows of
            // D outputs, VEC consecutive outputs per thread
            constexpr int HEADS = (HG ? NW : 1) * kGroup;
            constexpr int VEC = HEADS * D / (NW * 64);
            static_assert(VEC * NW * 64 == HEADS * D, "merge tiling");
            const int64_t mhead0 = (int64_t)b * p.hq + kvblock * kv_per_grp * kGroup;
            const int rows_bytes = HEADS * S * 4;
            const auto racc = __builtin_amdgcn_make_buffer_rsrc(p.part_acc + mhead0 * S * D, (short)0,
                                                                rows_bytes * D, kBufferWord3);
            const auto rmax = __builtin_amdgcn_make_buffer_rsrc(p.part_max + mhead0 * S, (short)0,
                                                                rows_bytes, kBufferWord3);
            const auto rsum = __builtin_amdgcn_make_buffer_rsrc(p.part_sum + mhead0 * S, (short)0,
                                                                rows_bytes, kBufferWord3);
            const int e0 = threadIdx.x * VEC;
            const int hl = e0 / D, d0 = e0 - hl * D;
            merge_vec_sys<VEC>(racc, rmax, rsum, S, D, hl, d0, p.out + (mhead0 + hl) * D + d0,
                               p.lse != nullptr ? p.lse + (mhead0 + hl) : nullptr,
                               p.lse != nullptr && d0 == 0);
            if (threadIdx.x == 0)
                __hip_atomic_store(p.counters + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            SPA_TL(kTlMergeDone);
        }
    }
    SPA_TL(kTlEnd);
}

// Separate merge: one workgroup per (b, h) row.
__global__ __launch_bounds__(128) void split_merge_kernel(const float *__restrict__ acc,
                                                          const float *__restrict__ mx,
                                                          const float *__restrict__ sum,
                                                          int splits, int head_dim,
                                                          uint16_t *__restrict__ out,
                                                          float *__restrict__ lse) {
    const int64_t row = blockIdx.x;
    for (int d = threadIdx.x; d < head_dim; d += blockDim.x)
        merge_element<kMergeChunkSeparate>(acc, mx, sum, splits, head_dim, row, d, out, lse);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t *__restrict__ ptr, size_t words) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride)
        ptr[i] = 0u;
}

template <int KV, int NW, bool HG>
hipError_t launch_nw(const DecodeParams &p_in, bool fused, hipStream_t stream) {
    DecodeParams p = p_in;
    p.split_walk = HG ? split_walk_for(p, KV == kKvInt8, NW) : 1;
    // e4m3 codes walk at most 2 splits: the stash of 2 keeps 3 workgroups
    // per CU (batch 32 / 8K producer 94.8 -> 92.4 us; a ragged batch, which
    // does not walk, 1% slower for the length check)
    if (KV == kKvFp8 && p.split_walk > 2) p.split_walk = 2;
    if (p.split_walk > 1) {
        // the stash must fit beside the kernel's static LDS
        auto lds_of = [](const void *f) {
            hipFuncAttributes a{};
            return hipFuncGetAttributes(&a, f) == hipSuccess ? a.sharedSizeBytes : (size_t)65536;
        };
        static const size_t static_lds_sep =
            lds_of(reinterpret_cast<const void *>(&decode_kernel<KV, NW, false, HG>));
        static const size_t static_lds_fused =
            lds_of(reinterpret_cast<const void *>(&decode_kernel<KV, NW, true, HG>));
        const size_t static_lds = fused ? static_lds_fused : static_lds_sep;
        const size_t max_lds = max_lds_per_block();
        while (p.split_walk > 1 &&
               static_lds + (size_t)NW * (p.split_walk - 1) * kStashFloats * sizeof(float) > max_lds)
            p.split_walk /= 2;
    }
    const int kv_per_grp = HG ? NW : 1;
    const int64_t per_split = (int64_t)p.batch * (p.hkv / kv_per_grp) * p.splits;
    p.walk_checked = walk_checked_for(per_split, p.split_walk);
    // checked walks: a workgroup per split, the kernel deciding (those past
    // the walked grid then exit at once)
    const unsigned grid = (unsigned)(p.walk_checked ? per_split : per_split / p.split_walk);
    // LDS stash for the states of all but the last split of a walk
    const size_t stash_bytes = (size_t)NW * (p.split_walk - 1) * kStashFloats * sizeof(float);
    if (fused)
        hipLaunchKernelGGL((decode_kernel<KV, NW, true, HG>), dim3(grid), dim3(NW * 64),
                           (unsigned)stash_bytes, stream, p, p.page_table, p.seq_lens);
    else
        hipLaunchKernelGGL((decode_kernel<KV, NW, false, HG>), dim3(grid), dim3(NW * 64),
                           (unsigned)stash_bytes, stream, p, p.page_table, p.seq_lens);
    return hipGetLastError();
}

}  // namespace

// A device attribute of the current device (cached per device), or
// fallback if it cannot be read.
template <hipDeviceAttribute_t ATTR>
int device_attr(int fallback) {
    static int cached[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return fallback;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, ATTR, dev) != hipSuccess || n <= 0) n = fallback;
        cached[dev] = n;
    }
    return cached[dev];
}
int cu_count() { return device_attr<hipDeviceAttributeMultiprocessorCount>(256); }
size_t max_lds_per_block() {
    return (size_t)device_attr<hipDeviceAttributeMaxSharedMemoryPerBlock>(65536);
}

// Splits one bf16 head-grouped workgroup walks when the batch's requests
// have about the same number of pages (the kernel checks that), from a
// sweep over batch 8-32 x context 1K-8K x 4/8/16 splits: fewer, longer page
// streams read faster.  Walks first cut the grid to one round of resident
// workgroups (4 per CU); splits of at least 4 pages then walk on down to one
// workgroup per CU (batch 32 / 8K / 16 splits: 187 us with one split per
// workgroup, 168 us walking 8); shorter splits stop at one round, their
// boundaries costing more than the longer streams save.  1-byte codes walk
// one split (int8) or at most 2 (e4m3, see launch_nw): their waves move
// half the bytes per page and lose with fewer of them (fp8 walking 4: a
// ragged batch 21% slower, its stash costing occupancy; equal lengths at
// most 4% faster).
constexpr int kMaxSplitWalk = 8;
constexpr int kLongSplitPages = 4;
// A walked grid of at least kWalkRounds rounds of kWalkRoundWgsPerCu
// workgroups per CU walks whatever the lengths (the dispatcher evens out
// ragged workgroups over the rounds: batch 512, lengths U[1, 1K], 8 splits,
// walking 8 262 us, one split per workgroup 311 us); a smaller one walks
// only a balanced batch.
constexpr int kWalkRounds = 2;
constexpr int kWalkRoundWgsPerCu = 4;
int walk_checked_for(int64_t split_wgs, int walk) {
    return walk > 1 && split_wgs / walk < (int64_t)kWalkRounds * kWalkRoundWgsPerCu * cu_count();
}
int split_walk_for(const DecodeParams &p, bool quant, int nw) {
    if (quant) return 1;
    const int64_t wgs = (int64_t)p.batch * (p.hkv / nw) * p.splits;
    const int64_t split_pages = (p.pt_stride + p.splits - 1) / p.splits;   // bound from the table
    const int64_t cus = cu_count();
    int w = 1;
    auto can_double = [&] { return 2 * w <= kMaxSplitWalk && p.splits % (2 * w) == 0; };
    while (can_double() && wgs / w > 4 * cus) w *= 2;
    while (can_double() && split_pages >= kLongSplitPages && wgs / (2 * w) >= cus) w *= 2;
    return w;
}


// Producer shapes.  Head-grouped: a block of kv heads per workgroup, one
// wave each, each wave walking all pages of its split (long per-wave
// streams, row-aligned reads; the block's waves read adjacent pieces of the
// same token rows).  bf16: 2 kv heads (4 measured 1% slower per call at
// batch 32 / 8K).  1-byte codes: 4 kv heads when the kv heads divide into
// blocks of 4, else 2 (4 against 2, alternating runs: ragged int8 batch
// producer 53.4-53.8 -> 51.4-51.7 us, fp8 batch 32 / 8K 97.8-98.0 -> 96.6
// us).  Page-split: one kv head per workgroup, 4 waves sharing its pages
// (4x the waves, for grids too small to fill the GPU otherwise).
constexpr int kNwHeadGrouped = 2;        // also the kv-head multiple head grouping needs
constexpr int kNwHeadGroupedCodes = 4;
constexpr int kNwPageSplit = 4;
// Producer choice, from a sweep over batch 1-32 x context 1K-8K x 4/8/16
// splits (32 query / 8 kv heads) for each KV type, equal lengths and ragged
// batches.  1-byte codes: head grouped from 1024 (request, kv head, split)
// triples, page split below (the page-split producer's keys in 64-byte
// pieces read faster with the default cache policy, which moved the
// threshold back up from 512).  bf16: head grouped from 1024 triples, from
// 256 when splits hold at most 8 pages and from 128 when they hold at most
// 2 (the pages per split bounded by the page table's width); page split
// for small grids of long splits, where its four waves per split shorten
// the longest request's chain (ragged batch of 8 requests up to 8K, 8
// splits: 30.4 against 34.8 us).  Over the sweep the default is within 5%
// of the best choice in 68 of 72 equal-length shapes and 10 of 12 ragged
// ones (with 512 triples as the only bound: 67 and 9).
constexpr int64_t kHeadGroupedMinWaves = 1024;
constexpr int64_t kHeadGroupedMinWavesMid = 256;     // splits of <= 8 pages
constexpr int64_t kHeadGroupedMinWavesShort = 128;   // splits of <= 2 pages
constexpr int64_t kHeadGroupedMinWavesQuant = 1024;

template <int KV>
hipError_t launch_kv(const DecodeParams &p, DecodeMode mode, bool fused, hipStream_t stream) {
    if (mode == DecodeMode::kHeadGrouped) {
        if constexpr (KV != 0)
            if (p.hkv % kNwHeadGroupedCodes == 0)
                return launch_nw<KV, kNwHeadGroupedCodes, true>(p, fused, stream);
        return launch_nw<KV, kNwHeadGrouped, true>(p, fused, stream);
    }
    return launch_nw<KV, kNwPageSplit, false>(p, fused, stream);
}

namespace {
hipError_t launch_producer(const DecodeParams &p, int kv_type, DecodeMode mode, bool fused,
                           hipStream_t stream) {
    if (kv_type == kKvInt8) return launch_kv<1>(p, mode, fused, stream);
    if (kv_type == kKvFp8) return launch_kv<2>(p, mode, fused, stream);
    return launch_kv<0>(p, mode, fused, stream);
}
}  // namespace

hipError_t launch_decode_producer(const DecodeParams &p, int kv_type, DecodeMode mode,
                                  hipStream_t stream) {
    return launch_producer(p, kv_type, mode, /*fused=*/false, stream);
}

hipError_t launch_decode(const DecodeParams &p, int kv_type, DecodeMode mode, bool fused,
                         hipStream_t stream) {
    const hipError_t err = launch_producer(p, kv_type, mode, fused, stream);
    if (err != hipSuccess || fused) return err;
    return launch_split_merge(p.part_acc, p.part_max, p.part_sum, p.batch * p.hq, kHeadDim,
                              p.splits, p.out, p.lse, stream);
}

DecodeMode default_mode(int batch, int hkv, int splits, int kv_type, int64_t pt_stride) {
    if (hkv % kNwHeadGrouped != 0) return DecodeMode::kPageSplit;
    const int64_t waves = (int64_t)batch * hkv * splits;
    if (kv_type != kKvBf16)
        return waves >= kHeadGroupedMinWavesQuant ? DecodeMode::kHeadGrouped : DecodeMode::kPageSplit;
    const int64_t split_pages = (pt_stride + splits - 1) / splits;
    const bool hg = waves >= kHeadGroupedMinWaves ||
                    (waves >= kHeadGroupedMinWavesMid && split_pages <= 8) ||
                    (waves >= kHeadGroupedMinWavesShort && split_pages <= 2);
    return hg ? DecodeMode::kHeadGrouped : DecodeMode::kPageSplit;
}

bool mode_supported(DecodeMode mode, int hkv) {
    return mode == DecodeMode::kPageSplit || hkv % kNwHeadGrouped == 0;
}

hipError_t launch_split_merge(const float *acc, const float *mx, const float *sum,
                              int32_t rows, int32_t head_dim, int32_t splits, uint16_t *out,
                              float *lse, hipStream_t stream) {
    hipLaunchKernelGGL(split_merge_kernel, dim3(rows), dim3(128), 0, stream, acc, mx, sum,
                       splits, head_dim, out, lse);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *ptr, size_t words, hipStream_t stream) {
    size_t blocks = (words + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t *>(ptr), words);
    return hipGetLastError();
}

}  // namespace spa

#ifdef SPA_TIMELINE
#include "spa.h"
#include "spa_timeline.h"
static_assert(SPA_TIMELINE_SLOTS == spa::kTimelineSlots && SPA_TIMELINE_WAVES == spa::kTimelineWaves,
              "timeline shape");
extern "C" int spa_timeline_clear(void) {
    void *ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(spa::timeline_buf));
    if (e == hipSuccess) e = hipMemset(ptr, 0, sizeof(spa::timeline_buf));
    if (e == hipSuccess) e = hipDeviceSynchronize();
    return e == hipSuccess ? SPA_OK : SPA_ERR_HIP;
}
extern "C" int spa_timeline_read(uint64_t *dst, size_t bytes) {
    if (dst == nullptr || bytes > sizeof(spa::timeline_buf)) return SPA_ERR_INVALID_ARGUMENT;
    const hipError_t e = hipMemcpyFromSymbol(dst, HIP_SYMBOL(spa::timeline_buf), bytes, 0,
                                             hipMemcpyDeviceToHost);
    return e == hipSuccess ? SPA_OK : SPA_ERR_HIP;
}
#endif
