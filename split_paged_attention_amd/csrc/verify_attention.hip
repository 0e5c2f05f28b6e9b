// Multi-token query decode (target verify / draft extend) over the paged KV
// cache, split-K like the one-token decode.
//
// Request b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (n_b of
// them); the last n_b of its L_b cached tokens are those queries' own, so
// query token i sees tokens 0 .. L_b - n_b + i (sglang's fused metadata
// update prepares cu_seqlens_q for exactly these steps: module docstring and
// the cumsum branch's Q modes).
//
// A workgroup is one (request, block of NW = 2 or 4 kv heads, split, chunk
// of up to 4 RB query tokens); wave w is kv head NW*block + w and walks the
// split's pages.  Per page:
//   * QK^T on the matrix cores in RB blocks of 16 MFMA rows, each 4 heads x
//     4 query tokens (row 4i + h of block r: token 4r + i, head h), all
//     blocks sharing every K operand, so the chunk's query tokens read K and
//     V once; lane group g then holds the scores of query tokens 4r + g and
//     keeps their online-softmax states, each with its own causal limit as a
//     mask;
//   * P.V on the matrix cores too: the page's V goes from registers
//     (loaded a page ahead) into a per-wave LDS tile, token-major (1-byte
//     codes converted to exact f16 on the way), the probabilities into a
//     token-major per-wave LDS tile, and the transposed LDS read
//     (ds_read_b64_tr_b16) turns both into MFMA operands: O[16 rows][128
//     dims] += P[16 rows][32 tokens] x V[32 tokens][128 dims], 16 MFMAs per
//     page and row block, the V operands shared by the blocks, with the
//     output rows in the same lanes as the softmax state.
// A request with more query tokens than one workgroup takes is cut into
// chunks of 4 RB tokens (a grid dimension); each chunk reads the request's
// K and V again.  The partial states go to the workspace and the ordinary
// split merge combines them, one (query row, head) at a time.
#include "internal.h"
#include "kernel_common.h"

namespace spa {
namespace {

// kv heads per workgroup, one per wave: 4 when the kv heads divide into
// fours, else 2 (4 against 2 at batch 32 / 8K, graph replay p50: bf16 4
// tokens 207.0 -> 203.2 us, fp8 4 tokens 124.8 -> 122.2, bf16 6 tokens
// 226.7 -> 219.2; the workgroup's waves read adjacent pieces of the same
// token rows)
constexpr int kVerifyWaves = 2;        // also the kv-head multiple the kernel needs
constexpr int kVerifyWavesWide = 4;
// One stashed split state of a wave: 32 accumulators per lane (64 lanes) and
// row block, then the maxima and sums of the RB blocks' 16 rows.
template <int RB>
constexpr int verify_stash_floats() { return RB * (32 * 64 + 32); }

// KV: 0 = bf16 pages, 1 = int8 codes, 2 = e4m3 codes (with fp32 scales).
// RB: row blocks of 4 query tokens x 4 heads; a workgroup takes 4 RB tokens.
// Two blocks hold twice the accumulators, so they run one wave per SIMD.
// NW: kv heads per workgroup.
template <int KV, int RB, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RB == 1 ? 2 : 1)))
void verify_kernel(DecodeParams p, const int32_t *__restrict__ page_table,
                   const int32_t *__restrict__ seq_lens, const int32_t *__restrict__ cu_q) {
    constexpr int D = kHeadDim, P = kPageSize;
    constexpr int QT = 4 * RB;                   // query tokens per workgroup
    constexpr int PW = 16 * RB;                  // P tile width: the blocks' MFMA rows
    constexpr int STASH = verify_stash_floats<RB>();
    constexpr bool QUANT = KV != 0;
    constexpr bool I8 = KV == 1;
    // K/V cache policy: values stream past the caches (non-temporal loads,
    // as in the one-token decode; bf16 at batch 32 / 8K, 4 query tokens
    // 200.2 -> 173.3 us per call, 6 tokens 215.4 -> 196.6 us with keys
    // and values streamed).  Keys, whose rows go out in 64-byte pieces,
    // keep the default policy except for bf16 with one row block (1-byte
    // codes, values streamed, keys default: fp8 4 tokens 118.9 -> 110.1 us,
    // ragged int8 82.2 -> 81.6 us, keys streamed too: 117.6 and 88.0 us;
    // bf16 keys default: 4 tokens 174.2 -> 183.5 us, 6 tokens 197.2 ->
    // 194.4 us).
    constexpr int K_POLICY = (QUANT || RB == 2) ? 0 : kStreaming;
    constexpr int V_POLICY = kStreaming;
    constexpr int ES = QUANT ? 1 : 2;            // bytes per element
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // QK layout: lane (n, g) = KV token n of a 16-token block, query token
    // 4 rb + g of row block rb; the P.V output has the same rows in the same
    // lanes, with dims 16 blk + n.  V registers: lane (g, n) holds token
    // 4i + g, dims 8n .. 8n+7.
    const int n = lane & 15, g = lane >> 4;

    // blockIdx -> (query-token chunk, group = b * blocks + kv block, split j).
    // The chunk is the slowest dimension; within a chunk the workgroups are
    // placed on the 8 XCDs as in the one-token decode: for 1-byte codes and a
    // batch that is a multiple of 8, all kv blocks and splits of a request
    // share an XCD; otherwise the S splits of a group do when the group count
    // allows.  Both placements need a chunk size that is a multiple of 8, so
    // the XCD of a block id is that of its offset in the chunk.
    const int S = p.splits;
    // Lane i holds request i's length (the walk choice and, for batches of
    // up to 64, the request ranking below read it).
    const int Li = lane < p.batch ? seq_lens[lane] : INT32_MIN;
    // bf16 and e4m3: a workgroup may walk `walk` consecutive splits (S a
    // multiple of it) with one page pipeline, as the one-token decode does: the states
    // of all but the last wait in dynamic LDS until the workgroup ends, each
    // split's arithmetic unchanged.  As there, a walked grid of about one
    // round walks only a batch whose requests have about the same number of
    // pages (walk_checked): the grid then has a workgroup per split and
    // chunk, and when the batch walks, those past the walked part of each
    // chunk exit at once.
    int walk = 1;
    if constexpr (!I8) {
        if (p.split_walk > 1 &&
            (!p.walk_checked || pages_balanced(seq_lens, p.batch, Li, p.pt_stride * P, P, lane)))
            walk = p.split_walk;
    }
    const int SG = S / walk;
    const int grp_per_b = p.hkv / NW;
    const int ngroups = p.batch * grp_per_b;
    const int per_chunk = ngroups * (p.walk_checked ? S : SG);   // launched per chunk
    const int chunk = blockIdx.x / per_chunk;
    int grp, j;
    {
        const int bid = blockIdx.x - chunk * per_chunk;
        if (bid >= ngroups * SG) return;
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
    // Requests are taken longest first, as in the one-token decode: rank r
    // is the r-th longest request (ties by index), so that the long
    // requests' workgroups are dispatched first and the serpentine deal
    // above gives each XCD about the same number of pages.  Batches of more
    // than 64 requests keep their natural order.
    // (Lane i also loads request i's query-row bounds, so the ranking adds
    // no load to the chain, and equal lengths skip it: ragged
    // int8 batch, 4 query tokens 81.1 -> 75.9 us per call; batch 32 / 8K
    // unchanged.)
    const int r = grp / grp_per_b;
    const int kvh = (grp - r * grp_per_b) * NW + wave;
    int b = r, L, q0, q1;
    if (p.batch > 1 && p.batch <= 64) {
        const bool in = lane < p.batch;
        const int Qa = in ? cu_q[lane] : 0, Qb = in ? cu_q[lane + 1] : 0;
        const int L0 = __builtin_amdgcn_readfirstlane(Li);
        if (__ballot(in && Li != L0) != 0) {
            int rank = 0;
            for (int k = 0; k < p.batch; ++k) {
                const int Lk = __builtin_amdgcn_readlane(Li, k);
                rank += (Lk > Li) || (Lk == Li && k < lane);
            }
            const unsigned long long hit = __ballot(in && rank == r);
            b = __builtin_amdgcn_readfirstlane(__ffsll((long long)hit) - 1);
        }
        L = __builtin_amdgcn_readlane(Li, b);
        q0 = __builtin_amdgcn_readlane(Qa, b);
        q1 = __builtin_amdgcn_readlane(Qb, b);
    } else {
        L = seq_lens[b];
        q0 = cu_q[b];
        q1 = cu_q[b + 1];
    }

    // This request's query rows; rows outside [0, total_q) are never touched.
    int nq = (int)max((int64_t)q1 - q0, (int64_t)0);
    if (q0 < 0 || q1 > p.total_q) nq = 0;
    const int c0 = chunk * QT;                  // this chunk's first query token
    const int nqc = min(min(nq, p.max_q_len) - c0, QT);   // its query tokens (none if <= 0)

    L = (int)min((int64_t)max(L, 0), p.pt_stride * P);
    const int pages = (L + P - 1) / P;
    const int pps = (pages + S - 1) / S;
    const int pg0 = min(j * pps, pages);
    const int pg1 = min(j * pps + walk * pps, pages);   // end of this workgroup's pages
    int jcur = j;                                        // split being accumulated
    int split_end = min(pg0 + pps, pages);               // its end page

    // One (query row, this wave's kv head) state of split jw: acc values of
    // head h at dims 16 blk + n from av(h, blk), m and l from lane n == 0.
    auto put_state = [&](int row, int jw, auto av, const float (&mh)[4], const float (&lh)[4]) {
        const int64_t row0 = ((int64_t)row * p.hq + kvh * kGroup) * S + jw;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const int64_t idx = row0 + (int64_t)h * S;
            float *dst = p.part_acc + idx * D + n;
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) dst[16 * blk] = av(h, blk);
            if (n == 0) {
                p.part_max[idx] = mh[h] == kNegInf ? kNegInf : mh[h] * kLn2;
                p.part_sum[idx] = lh[h];
            }
        }
    };
    const float kEmptyM[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
    const float kEmptyL[4] = {0.f, 0.f, 0.f, 0.f};
    auto zero_acc = [](int, int) { return 0.f; };
    // Rows past the declared maximum max_q_len (a request with more query
    // tokens in the device data) get the empty state, so the merge gives
    // them out = 0 and lse = -inf instead of reading stale workspace.
    if (chunk == p.q_chunks - 1) {
        for (int i = p.max_q_len + g; i < nq; i += 4)
            for (int jw = j; jw < j + walk; ++jw) put_state(q0 + i, jw, zero_acc, kEmptyM, kEmptyL);
    }
    if (nqc <= 0) return;   // the whole workgroup

    extern __shared__ __attribute__((aligned(16))) float vstash[];
    int nstash = 0;
    const int row_stride = p.hkv * D;
    // query token 4 rb + g of this chunk sees tokens < vis[rb]
    int vis[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) vis[rb] = L - nq + c0 + 4 * rb + g + 1;

    // A operand of block rb: row n is head n & 3 of query token 4 rb + n / 4
    // (rows of tokens past the chunk's last repeat it and are never stored).
    // Same contraction order as the one-token decode.
    bf16x8_t qa[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
        const int tq = min(4 * rb + (n >> 2), nqc - 1);
        const uint16_t *qp = reinterpret_cast<const uint16_t *>(p.q) +
                             ((int64_t)(q0 + c0 + tq) * p.hq + kvh * kGroup + (n & 3)) * D;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int d0 = QUANT ? 64 * (c >> 1) + 16 * g + 8 * (c & 1) : 32 * c + 8 * g;
            qa[rb][c] = *reinterpret_cast<const bf16x8_t *>(qp + d0);
        }
    }
    // 1-byte codes: the query goes to f16, each row scaled by a power of two
    // putting its largest |q| in [2^14, 2^15) (exact); score row 4g + h of
    // block rb is unscaled with the factor of lane 4g + h.
    f16x8_t qa16[RB][4];
    float qscale[RB][4];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int h = 0; h < 4; ++h) qscale[rb][h] = p.qk_scale_log2;
    if constexpr (QUANT) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
            float amax = 0.f;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf((float)qa[rb][c][e]));
            amax = max_xor32(max_xor16(amax));   // lane n: row n, all 128 dims
            const int sh = amax > 0.f ? 15 - __builtin_amdgcn_frexp_expf(amax) : 0;
            const float up = __builtin_ldexpf(1.f, sh);
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int e = 0; e < 8; ++e) qa16[rb][c][e] = (_Float16)((float)qa[rb][c][e] * up);
#pragma unroll
            for (int h = 0; h < 4; ++h)
                qscale[rb][h] = p.qk_scale_log2 * __builtin_ldexpf(1.f, -__shfl(sh, 4 * g + h));
        }
    }

    // softmax state of row (query token 4 rb + g, head h); acc[rb][blk] =
    // output row (4 rb + g, h), dim 16 blk + n (the MFMA output layout)
    float m[RB][4], lpart[RB][4];
    f32x4_t acc[RB][8];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            m[rb][h] = kNegInf;
            lpart[rb][h] = 0.f;
        }
#pragma unroll
        for (int blk = 0; blk < 8; ++blk) acc[rb][blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // Per-wave LDS tiles, 16-bit elements, token-major: half a page of V
    // (32 tokens x 128 dims, bf16 or the f16 values of the codes; the two
    // halves take turns) and P[64 tokens][16 RB rows].
    // V rows are padded by 16 elements (32 bytes): the 4 rows a transposed
    // read touches per 16 lanes then sit 8 banks apart instead of on the same
    // banks (bank-conflict cycles per call at batch 32 / 8K / 4 tokens: 16.5M
    // unpadded, 3.9M padded; the call time did not change).
    constexpr int VROW = D + 16;
    __shared__ __attribute__((aligned(16))) uint16_t vbuf[NW][P / 2][VROW];
    __shared__ __attribute__((aligned(16))) uint16_t pbuf[NW][P][PW];
    // bf16: the probabilities' low terms (p = hi + lo to 16 significant
    // bits; both terms' products with bf16 values are exact in fp32, so P.V
    // carries p to 2^-17 instead of the 2^-9 of one bf16 term, which can
    // cost 0.007 on an output of a few tokens)
    __shared__ __attribute__((aligned(16))) uint16_t pbuf_lo[QUANT ? 1 : NW][QUANT ? 1 : P][PW];
    uint16_t(*vt)[VROW] = vbuf[wave];
    uint16_t(*pt16)[PW] = pbuf[wave];
    uint16_t(*ptl16)[PW] = pbuf_lo[QUANT ? 0 : wave];
    // Transposed-read addressing: lane 16G + 4e + qd supplies row 8G + e
    // (+ 4 for the second read), columns 4qd .. 4qd+3; lane 16G + i then
    // receives column i of rows 8G .. 8G+3 (8G+4 .. 8G+7): the MFMA operand
    // lane (i, k-chunk G).
    const int tr_row = 8 * g + ((lane & 15) >> 2), tr_col = 4 * (lane & 3);

    const int32_t *pt_row = page_table + (int64_t)b * p.pt_stride;
    const int row_bytes = row_stride * ES;
    const int k_lane = (n * row_stride + (QUANT ? 16 : 8) * g) * ES;
    const int v_lane = (g * row_stride + 8 * n) * ES;   // token 4i + g, dims 8n ..
    const int s_lane64 = lane * p.hkv * 4;
    uint4 kr[4][4];
    uint4 vr16[16];
    uint4 kr8[4][2];
    uint2 vr8[16];
    float ksc_tok = 0.f, vsc_tok = 0.f;
    auto rsrc = [&](const void *base, int64_t page, int64_t elem_per_page, int64_t elem_off,
                    int esize, int nbytes) {
        const char *ptr = static_cast<const char *>(base) + (page * elem_per_page + elem_off) * esize;
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(ptr), (short)0, nbytes,
                                                 kBufferWord3);
    };
    auto load_k = [&](int64_t page, int valid_rows) {
        const auto r = rsrc(p.k_pages, page, (int64_t)P * row_stride, (int64_t)kvh * D, ES,
                            valid_rows * row_bytes);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            if constexpr (!QUANT) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    kr[t][c] = buf_ld16<K_POLICY>(r, k_lane + 64 * c, 16 * t * row_bytes);
            } else {
#pragma unroll
                for (int c2 = 0; c2 < 2; ++c2)
                    kr8[t][c2] = buf_ld16<K_POLICY>(r, k_lane + 64 * c2, 16 * t * row_bytes);
            }
        }
        if constexpr (QUANT) {
            const auto rs = rsrc(p.k_scales, page, (int64_t)P * p.hkv, kvh, 4,
                                 valid_rows * p.hkv * 4);
            ksc_tok = buf_ldf(rs, s_lane64, 0);
        }
    };
    auto load_v = [&](int64_t page, int valid_rows, int half) {
        const auto r = rsrc(p.v_pages, page, (int64_t)P * row_stride, (int64_t)kvh * D, ES,
                            valid_rows * row_bytes);
#pragma unroll
        for (int i = 8 * half; i < 8 * half + 8; ++i) {
            if constexpr (!QUANT)
                vr16[i] = buf_ld16<V_POLICY>(r, v_lane, 4 * i * row_bytes);
            else
                vr8[i] = buf_ld8<V_POLICY>(r, v_lane, 4 * i * row_bytes);
        }
        if (QUANT && half == 0) {
            const auto rs = rsrc(p.v_scales, page, (int64_t)P * p.hkv, kvh, 4,
                                 valid_rows * p.hkv * 4);
            vsc_tok = buf_ldf(rs, s_lane64, 0) * (I8 ? 1.f : kF8ValueScale);
        }
    };
    // Loaded rows of logical page i (zero range past the split or for a page
    // id outside the pool: reads 0, touches no memory).
    auto page_rows = [&](int i, int64_t &page) {
        page = 0;
        if (i >= pg1) return 0;
        const int32_t id = pt_row[i];
        const bool ok = (uint32_t)id < (uint32_t)p.num_pages;
        page = ok ? id : 0;
        return ok ? min(P, L - i * P) : 0;
    };

    // V rows 32 half .. 32 half + 31 of the page into the half-page tile
    auto put_v_half = [&](int half) {
#pragma unroll
        for (int i = 8 * half; i < 8 * half + 8; ++i) {
            uint4 w;
            if constexpr (!QUANT) {
                w = vr16[i];
            } else if constexpr (I8) {
                w = __builtin_bit_cast(uint4, i8x8_to_f16(vr8[i]));
            } else {
                const uint2 c = vr8[i];
                w = make_uint4(
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                                                     c.x, 1.f / kF8ValueScale, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                                                     c.x, 1.f / kF8ValueScale, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                                                     c.y, 1.f / kF8ValueScale, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(
                                                     c.y, 1.f / kF8ValueScale, true)));
            }
            *reinterpret_cast<uint4 *>(&vt[4 * (i - 8 * half) + g][8 * n]) = w;
        }
    };

    int pg = pg0;
    if (pg < pg1) {
        int64_t page;
        const int rows = page_rows(pg, page);
        load_k(page, rows);
        load_v(page, rows, 0);
        load_v(page, rows, 1);
    }
    for (; pg < pg1; ++pg) {
        int64_t page_next;
        const int valid_next = page_rows(pg + 1, page_next);
        const int valid = min(P, L - pg * P);

        // ---- the first half of this page's V into the LDS tile (token 4i + g,
        // dims 8n ..); its registers then take the next page's first half
        put_v_half(0);
        const float vsc_cur = vsc_tok;
        __builtin_amdgcn_sched_barrier(0);
        load_v(page_next, valid_next, 0);
        __builtin_amdgcn_sched_barrier(0);

        // ---- S = Q K^T: lane (n, g) gets s[query token 4 rb + g, head h]
        // [KV token 16t + n] in sacc[rb][t][h]; each K operand feeds every block
        f32x4_t sacc[RB][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) sacc[rb][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if constexpr (!QUANT) {
                    const bf16x8_t kb = __builtin_bit_cast(bf16x8_t, kr[t][c]);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        sacc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[rb][c], kb,
                                                                              sacc[rb][t], 0, 0, 0);
                } else {
                    const uint4 w = kr8[t][c >> 1];
                    const uint2 h = (c & 1) ? make_uint2(w.z, w.w) : make_uint2(w.x, w.y);
                    const f16x8_t kb = I8 ? i8x8_to_f16(h) : e4m3x8_to_f16(h);
#pragma unroll
                    for (int rb = 0; rb < RB; ++rb)
                        sacc[rb][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa16[rb][c], kb,
                                                                             sacc[rb][t], 0, 0, 0);
                }
            }
        }
        float s[RB][4][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int tok = 16 * t + n;
            const float kt = QUANT ? lane_value(ksc_tok, tok) : 1.f;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const bool ok = tok < valid && pg * P + tok < vis[rb];
#pragma unroll
                for (int h = 0; h < 4; ++h)
                    s[rb][t][h] = ok ? sacc[rb][t][h] * (qscale[rb][h] * kt) : kNegInf;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        load_k(page_next, valid_next);
        __builtin_amdgcn_sched_barrier(0);

        // ---- online softmax (base 2) per (query token, head); a row that
        // has seen no token yet keeps m = -inf and weights 0
        float alpha[RB][4], pv[RB][4][4];
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                float mx = fmaxf(fmaxf(s[rb][0][h], s[rb][1][h]), fmaxf(s[rb][2][h], s[rb][3][h]));
                mx = row_max16(mx);
                const float mnew = fmaxf(m[rb][h], mx);
                const float mref = mnew == kNegInf ? 0.f : mnew;
                alpha[rb][h] = exp2_fast(m[rb][h] - mref);
                m[rb][h] = mnew;
                float rs = 0.f;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    pv[rb][t][h] = exp2_fast(s[rb][t][h] - mref);
                    rs += pv[rb][t][h];
                }
                lpart[rb][h] = __builtin_fmaf(lpart[rb][h], alpha[rb][h], rs);
            }
        }
        // probabilities of row (4 rb + g, h) for tokens 16t + n into the P
        // tile, column 16 rb + 4 g + h (1-byte codes: value scale folded in, f16)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float vs = QUANT ? lane_value(vsc_cur, 16 * t + n) : 1.f;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                const float *a = pv[rb][t];
                uint2 w;
                if constexpr (QUANT) {
                    w = make_uint2(pack_f16x2(a[0] * vs, a[1] * vs), pack_f16x2(a[2] * vs, a[3] * vs));
                } else {
                    w = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
                    *reinterpret_cast<uint2 *>(&ptl16[16 * t + n][16 * rb + 4 * g]) =
                        make_uint2(bf16x2_residual(a[0], a[1], w.x), bf16x2_residual(a[2], a[3], w.y));
                }
                *reinterpret_cast<uint2 *>(&pt16[16 * t + n][16 * rb + 4 * g]) = w;
            }
        }
        // LDS ops of one wave complete in order; this only keeps the compiler
        // from moving the reads above the writes.
        __asm__ volatile("" ::: "memory");

        // ---- O += P V on the matrix cores, 32 tokens per step
#pragma unroll
        for (int rb = 0; rb < RB; ++rb)
#pragma unroll
            for (int h = 0; h < 4; ++h)
#pragma unroll
                for (int blk = 0; blk < 8; ++blk) acc[rb][blk][h] *= alpha[rb][h];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb == 1) {
                // the first half's reads are issued (LDS ops of a wave run in
                // order): the second half takes the tile, and its registers
                // the next page's second half
                __asm__ volatile("" ::: "memory");
                put_v_half(1);
                __asm__ volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                load_v(page_next, valid_next, 1);
                __builtin_amdgcn_sched_barrier(0);
            }
            const int r0 = 32 * kb + tr_row;
            // (a_lo / a_hi: tokens r0.. and r0 + 4..; al_*: the low terms)
            uint64_t a_lo[RB], a_hi[RB], al_lo[RB], al_hi[RB];
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
                a_lo[rb] = lds_tr16_b64(&pt16[r0][16 * rb + tr_col]);
                a_hi[rb] = lds_tr16_b64(&pt16[r0 + 4][16 * rb + tr_col]);
                if constexpr (!QUANT) {
                    al_lo[rb] = lds_tr16_b64(&ptl16[r0][16 * rb + tr_col]);
                    al_hi[rb] = lds_tr16_b64(&ptl16[r0 + 4][16 * rb + tr_col]);
                }
            }
#pragma unroll
            for (int blk = 0; blk < 8; ++blk) {
                const uint64_t b_lo = lds_tr16_b64(&vt[tr_row][16 * blk + tr_col]);
                const uint64_t b_hi = lds_tr16_b64(&vt[tr_row + 4][16 * blk + tr_col]);
#pragma unroll
                for (int rb = 0; rb < RB; ++rb) {
                    if constexpr (!QUANT) {
                        const bf16x8_t vb = join_bf16x8(b_lo, b_hi);
                        acc[rb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            join_bf16x8(al_lo[rb], al_hi[rb]), vb, acc[rb][blk], 0, 0, 0);
                        acc[rb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            join_bf16x8(a_lo[rb], a_hi[rb]), vb, acc[rb][blk], 0, 0, 0);
                    } else
                        acc[rb][blk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                            join_f16x8(a_lo[rb], a_hi[rb]), join_f16x8(b_lo, b_hi), acc[rb][blk],
                            0, 0, 0);
                }
            }
        }
        // the next page's V overwrites the tile only after these reads
        __asm__ volatile("" ::: "memory");
        if (!I8 && pg + 1 == split_end && pg + 1 < pg1) {
            // split jcur complete and not this workgroup's last: its state
            // into the LDS stash, then start the next one
            float *st = vstash + (wave * (walk - 1) + nstash) * STASH;
#pragma unroll
            for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
                for (int h = 0; h < 4; ++h) {
                    const float l = row_sum16(lpart[rb][h]);
#pragma unroll
                    for (int blk = 0; blk < 8; ++blk)
                        st[((rb * 8 + blk) * 4 + h) * 64 + lane] = acc[rb][blk][h];
                    if (n == 0) {
                        st[RB * 32 * 64 + 16 * rb + 4 * g + h] = m[rb][h];
                        st[RB * 32 * 64 + 16 * RB + 16 * rb + 4 * g + h] = l;
                    }
                    m[rb][h] = kNegInf;
                    lpart[rb][h] = 0.f;
                }
#pragma unroll
                for (int blk = 0; blk < 8; ++blk) acc[rb][blk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            }
            ++nstash;
            ++jcur;
            split_end = min(split_end + pps, pages);
        }
    }
    // ---- partial states of this chunk's query tokens: l over the 16 lanes
    // of a group; then the walk's splits past the context (empty) and the
    // stashed splits j .. j + nstash - 1
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int h = 0; h < 4; ++h) lpart[rb][h] = row_sum16(lpart[rb][h]);
        const int tq = 4 * rb + g;
        if (tq >= nqc) continue;
        const int row = q0 + c0 + tq;
        put_state(row, jcur, [&](int h, int blk) { return acc[rb][blk][h]; }, m[rb], lpart[rb]);
        for (int jw = jcur + 1; jw < j + walk; ++jw) put_state(row, jw, zero_acc, kEmptyM, kEmptyL);
        for (int k = 0; k < nstash; ++k) {
            const float *st = vstash + (wave * (walk - 1) + k) * STASH;
            float mk[4], lk[4];
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                mk[h] = st[RB * 32 * 64 + 16 * rb + 4 * g + h];
                lk[h] = st[RB * 32 * 64 + 16 * RB + 16 * rb + 4 * g + h];
            }
            put_state(row, j + k,
                      [&](int h, int blk) { return st[((rb * 8 + blk) * 4 + h) * 64 + lane]; }, mk,
                      lk);
        }
    }
}

template <int KV, int RB, int NW>
hipError_t launch_verify_kv(const DecodeParams &p_in, hipStream_t stream) {
    constexpr int STASH = verify_stash_floats<RB>();
    DecodeParams p = p_in;
    p.split_walk = split_walk_for(p, KV == kKvInt8, NW);
    // e4m3 codes walk at most 2 splits, whose stash keeps 2 workgroups per
    // CU (batch 32 / 8K, 4 tokens: 110.5 -> 108.4 us per call; int8 codes,
    // walking too, cost the ragged batch 2%)
    if (KV == kKvFp8 && p.split_walk > 2) p.split_walk = 2;
    if (p.split_walk > 1) {
        // the stash must fit beside the kernel's static LDS
        static const size_t static_lds = [] {
            hipFuncAttributes a{};
            return hipFuncGetAttributes(&a, reinterpret_cast<const void *>(&verify_kernel<KV, RB, NW>)) ==
                           hipSuccess
                       ? a.sharedSizeBytes
                       : (size_t)65536;
        }();
        const size_t max_lds = max_lds_per_block();
        while (p.split_walk > 1 &&
               static_lds + (size_t)NW * (p.split_walk - 1) * STASH * sizeof(float) > max_lds)
            p.split_walk /= 2;
    }
    const int64_t per_split = (int64_t)p.batch * (p.hkv / NW) * p.splits;
    p.walk_checked = walk_checked_for(per_split * p.q_chunks, p.split_walk);
    // checked walks: a workgroup per split and chunk, the kernel deciding
    // (those past the walked grid then exit at once)
    const unsigned grid = (unsigned)((p.walk_checked ? per_split : per_split / p.split_walk) *
                                     p.q_chunks);
    const size_t stash_bytes = (size_t)NW * (p.split_walk - 1) * STASH * sizeof(float);
    hipLaunchKernelGGL((verify_kernel<KV, RB, NW>), dim3(grid), dim3(NW * 64),
                       (unsigned)stash_bytes, stream, p, p.page_table, p.seq_lens, p.cu_seqlens_q);
    return hipGetLastError();
}

template <int RB, int NW>
hipError_t launch_verify_nw(const DecodeParams &p, int kv_type, hipStream_t stream) {
    if (kv_type == kKvInt8) return launch_verify_kv<1, RB, NW>(p, stream);
    if (kv_type == kKvFp8) return launch_verify_kv<2, RB, NW>(p, stream);
    return launch_verify_kv<0, RB, NW>(p, stream);
}

template <int RB>
hipError_t launch_verify_rb(const DecodeParams &p, int kv_type, hipStream_t stream) {
    if (p.hkv % kVerifyWavesWide == 0) return launch_verify_nw<RB, kVerifyWavesWide>(p, kv_type, stream);
    return launch_verify_nw<RB, kVerifyWaves>(p, kv_type, stream);
}

}  // namespace

// Query tokens one workgroup takes: 4 (one row block) up to max_q_len 4,
// else 8 (two blocks sharing the K and V operands); more tokens per request
// are cut into chunks of that size.
int verify_tokens_per_workgroup(int max_q_len) { return max_q_len <= 4 ? 4 : 8; }

hipError_t launch_verify(const DecodeParams &p_in, int kv_type, int max_q_len,
                         hipStream_t stream) {
    DecodeParams p = p_in;
    const int qt = verify_tokens_per_workgroup(max_q_len);
    p.max_q_len = max_q_len;
    p.q_chunks = (max_q_len + qt - 1) / qt;
    const hipError_t err = qt == 4 ? launch_verify_rb<1>(p, kv_type, stream)
                                   : launch_verify_rb<2>(p, kv_type, stream);
    if (err != hipSuccess) return err;
    return launch_split_merge(p.part_acc, p.part_max, p.part_sum, p.total_q * p.hq, kHeadDim,
                              p.splits, p.out, p.lse, stream);
}

bool verify_supported(int hkv) { return hkv % kVerifyWaves == 0; }

}  // namespace spa
