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
//   * P.V on the vector ALUs with v_dot2_f32_bf16: lane (r, c) owns dims
//     8c..8c+7 of tokens 4i + r (so one V load instruction reads 4 whole
//     256-byte rows), pairs tokens t and t + 16 in one dot2, and gets the
//     packed bf16 probabilities of its tokens from a 512-byte per-wave LDS
//     buffer.  P.V with K = tokens would need V transposed for the MFMA B
//     operand; the VALU form reads V in its stored order instead.
// The path is HBM-bound (about 4 flop per KV byte for bf16), so the design
// goal is bytes in flight and a single pass over K and V.
#include "internal.h"

namespace spa {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// DPP lane permutations inside a 16-lane row.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
// Butterfly over the 16 lanes of a row: xor 1, xor 2, half-row mirror, row mirror.
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<0xB1>(x));
    x = fmaxf(x, dpp<0x4E>(x));
    x = fmaxf(x, dpp<0x141>(x));
    x = fmaxf(x, dpp<0x140>(x));
    return x;
}
__device__ __forceinline__ float row_sum16(float x) {
    x = x + dpp<0xB1>(x);
    x = x + dpp<0x4E>(x);
    x = x + dpp<0x141>(x);
    x = x + dpp<0x140>(x);
    return x;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t v;
    v[0] = (__bf16)lo;   // round to nearest even
    v[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
}
// bf16 bit pattern of (float)(signed byte k of w); exact for |x| <= 127.
__device__ __forceinline__ uint32_t i8_bf16_hi(uint32_t w, int k) {
    float f = (float)(int32_t)__builtin_amdgcn_sbfe(w, 8 * k, 8);
    return __float_as_uint(f);
}
// Two bf16 (upper halves of two fp32 bit patterns) -> one packed dword.
__device__ __forceinline__ uint32_t pack_hi16(uint32_t lo_f, uint32_t hi_f) {
    return __builtin_amdgcn_perm(hi_f, lo_f, 0x07060302u);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    f16x2_t v;
    v[0] = (_Float16)lo;   // round to nearest even
    v[1] = (_Float16)hi;
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float dot2_f16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, a), __builtin_bit_cast(f16x2_t, b),
                                  c, false);
}
// int8 value codes -> exact f16, biased: byte k of wa (token a) and of wb
// (token b) become the f16 pair (1152 + a_k, 1152 + b_k).  With its sign bit
// flipped a code is x + 128 in [1, 255]; placed as the low mantissa byte under
// the f16 exponent of 1024 it reads 1024 + x + 128.
constexpr float kI8Bias = 1152.f;
constexpr uint32_t kF16One2 = 0x3C003C00u;   // f16 pair (1, 1)
template <int K>
__device__ __forceinline__ uint32_t i8_pair_f16(uint32_t wb, uint32_t wa) {
    constexpr uint32_t sel = (uint32_t)K | (0x0Cu << 8) | ((uint32_t)(4 + K) << 16) | (0x0Cu << 24);
    return __builtin_amdgcn_perm(wb, wa, sel) ^ 0x64806480u;
}

// ---------------------------------------------------------------------------
// The log-sum-exp merge of one output element.  Shared, unchanged, by the
// fused tail and by the separate merge kernel, so both give the same bits.
// SYS_LOADS: read through to memory (system scope, no cached copy), used by
// the fused tail, which reads state other workgroups published in this launch.
template <bool SYS_LOADS>
__device__ __forceinline__ float ld(const float *p) {
    if constexpr (SYS_LOADS)
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    else
        return *p;
}
// Store that is written through to memory (system scope): visible to every
// XCD once the issuing wave's store counter drains, with no L2 writeback.
__device__ __forceinline__ void st_sys(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

template <bool SYS_LOADS>
__device__ __forceinline__ void merge_element(const float *__restrict__ acc,
                                              const float *__restrict__ mx,
                                              const float *__restrict__ sum, int splits,
                                              int head_dim, int64_t row, int d,
                                              uint16_t *__restrict__ out,
                                              float *__restrict__ lse) {
    const float *mrow = mx + row * splits;
    const float *lrow = sum + row * splits;
    const float *arow = acc + row * splits * (int64_t)head_dim + d;
    // Splits are visited in order j = 0..splits-1; loads are issued CH at a
    // time (clamped indices, masked values) so their latencies overlap.
    constexpr int CH = 8;
    float M = kNegInf;
    for (int j0 = 0; j0 < splits; j0 += CH) {
        float mv[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) mv[u] = ld<SYS_LOADS>(mrow + min(j0 + u, splits - 1));
#pragma unroll
        for (int u = 0; u < CH; ++u) M = fmaxf(M, mv[u]);
    }
    float l = 0.f, o = 0.f;
    for (int j0 = 0; j0 < splits; j0 += CH) {
        float mv[CH], lv[CH], av[CH];
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            const int j = min(j0 + u, splits - 1);
            mv[u] = ld<SYS_LOADS>(mrow + j);
            lv[u] = ld<SYS_LOADS>(lrow + j);
            av[u] = ld<SYS_LOADS>(arow + (int64_t)j * head_dim);
        }
#pragma unroll
        for (int u = 0; u < CH; ++u) {
            if (j0 + u >= splits || mv[u] == kNegInf) continue;   // past the end / empty split
            const float w = exp2_fast((mv[u] - M) * kLog2e);
            l = __builtin_fmaf(w, lv[u], l);
            o = __builtin_fmaf(w, av[u], o);
        }
    }
    const float res = l > 0.f ? o / l : 0.f;
    out[row * head_dim + d] = to_bf16_bits(res);
    if (lse != nullptr && d == 0)
        lse[row] = l > 0.f ? M + __builtin_amdgcn_logf(l) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------------------
// Producer (+ fused merge).
template <int KV_INT8, int NW, bool FUSED>
__global__ __launch_bounds__(NW * 64) void decode_kernel(DecodeParams p) {
    constexpr int D = kHeadDim, P = kPageSize;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;     // QK layout: token n of a 16-block, k-chunk g
    const int vr = lane >> 4, vc = lane & 15;   // PV layout: token phase r, dims 8c..8c+7

    // blockIdx -> (group = b * Hkv + kvh, split j).  The S split workgroups of a
    // group get ids congruent mod 8 so they land on one XCD (dispatch is round
    // robin over the 8 XCDs) and share its L2 for the merge.
    const int S = p.splits;
    const int ngroups = p.batch * p.hkv;
    int grp, j;
    {
        const int bid = blockIdx.x;
        if ((ngroups & 7) == 0) {
            const int xcd = bid & 7, slot = bid >> 3;
            grp = (slot / S) * 8 + xcd;
            j = slot % S;
        } else {
            grp = bid / S;
            j = bid % S;
        }
    }
    const int b = grp / p.hkv, kvh = grp - b * p.hkv;
    const int L = p.seq_lens[b];
    const int pages = (L + P - 1) / P;
    const int pps = (pages + S - 1) / S;
    const int pg0 = min(j * pps, pages);
    const int pg1 = min(pg0 + pps, pages);
    const int row_stride = p.hkv * D;           // elements between consecutive token rows

    // A operand: row i of the MFMA is query head (kvh*4 + (i & 3)); k-chunk g of
    // MFMA c covers dims 32c + 8g .. +8.
    bf16x8_t qa[4];
    {
        const uint16_t *qp = reinterpret_cast<const uint16_t *>(p.q) +
                             ((int64_t)b * p.hq + kvh * kGroup + (n & 3)) * D + 8 * g;
#pragma unroll
        for (int c = 0; c < 4; ++c) qa[c] = *reinterpret_cast<const bf16x8_t *>(qp + 32 * c);
    }

    float m[4], lpart[4], acc[4][8], psum[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        m[h] = kNegInf;
        lpart[h] = 0.f;
        psum[h] = 0.f;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;
    }

    __shared__ uint32_t pbuf[NW][8][4][4];          // [wave][pair u][phase r][head]
    __shared__ float sm_m[NW][4], sm_l[NW][4];
    __shared__ float sm_acc[NW][4][D];
    __shared__ int sm_last;

    const int32_t *pt_row = p.page_table + (int64_t)b * p.pt_stride;

    for (int pg = pg0 + wave; pg < pg1; pg += NW) {
        const int64_t page = pt_row[pg];
        const int64_t page_elem = page * (int64_t)(P * row_stride) + (int64_t)kvh * D;
        const int tok0 = pg * P;
        const int valid = min(P, L - tok0);         // tokens of this page that count

        // ---- loads: K in MFMA B layout, V in PV layout
        bf16x8_t kb[4][4];
        uint32_t vw[16][4];      // bf16 V words (bf16 pages)
        uint2 vraw[16];          // int8 V codes (int8 pages)
        float ksc[4], vsc[4];
        if constexpr (KV_INT8 == 0) {
            const uint16_t *kp = reinterpret_cast<const uint16_t *>(p.k_pages) + page_elem;
            const uint16_t *vp = reinterpret_cast<const uint16_t *>(p.v_pages) + page_elem;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    kb[t][c] = *reinterpret_cast<const bf16x8_t *>(
                        kp + (16 * t + n) * row_stride + 32 * c + 8 * g);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint4 w = *reinterpret_cast<const uint4 *>(
                    vp + (4 * i + vr) * row_stride + 8 * vc);
                vw[i][0] = w.x; vw[i][1] = w.y; vw[i][2] = w.z; vw[i][3] = w.w;
            }
        } else {
            const int8_t *kp = reinterpret_cast<const int8_t *>(p.k_pages) + page_elem;
            const int8_t *vp = reinterpret_cast<const int8_t *>(p.v_pages) + page_elem;
            uint2 kraw[4][4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    kraw[t][c] = *reinterpret_cast<const uint2 *>(
                        kp + (16 * t + n) * row_stride + 32 * c + 8 * g);
#pragma unroll
            for (int i = 0; i < 16; ++i)
                vraw[i] = *reinterpret_cast<const uint2 *>(vp + (4 * i + vr) * row_stride + 8 * vc);
            const int64_t srow = page * (int64_t)(P * p.hkv) + kvh;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                ksc[t] = p.k_scales[srow + (int64_t)(16 * t + n) * p.hkv];
                vsc[t] = p.v_scales[srow + (int64_t)(16 * t + n) * p.hkv];
            }
            // int8 -> bf16 (exact)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    uint32_t wds[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t src = e < 2 ? kraw[t][c].x : kraw[t][c].y;
                        const int k0 = (e & 1) * 2;
                        wds[e] = pack_hi16(i8_bf16_hi(src, k0), i8_bf16_hi(src, k0 + 1));
                    }
                    uint4 u = make_uint4(wds[0], wds[1], wds[2], wds[3]);
                    kb[t][c] = __builtin_bit_cast(bf16x8_t, u);
                }
        }

        // ---- S = Q K^T: lane (n, g) gets s[head h][token 16t + n] in sacc[t][h]
        f32x4_t sacc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            sacc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                sacc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[c], kb[t][c], sacc[t], 0, 0, 0);
        }
        float s[4][4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float f = KV_INT8 ? p.qk_scale_log2 * ksc[t] : p.qk_scale_log2;
            const bool ok = (16 * t + n) < valid;
#pragma unroll
            for (int h = 0; h < 4; ++h) s[t][h] = ok ? sacc[t][h] * f : kNegInf;
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

        // ---- probabilities for P.V: pair (token 32q + n, token 32q + 16 + n),
        // packed bf16; stored by row 0 of the wave as pbuf[pair u][phase r][h]
        // with u = 4q + n/4, r = n % 4.
        if (g == 0) {
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) {
                uint4 w;
                float a0 = pv[2 * qq][0], a1 = pv[2 * qq][1], a2 = pv[2 * qq][2], a3 = pv[2 * qq][3];
                float b0 = pv[2 * qq + 1][0], b1 = pv[2 * qq + 1][1], b2 = pv[2 * qq + 1][2],
                      b3 = pv[2 * qq + 1][3];
                if constexpr (KV_INT8 != 0) {
                    a0 *= vsc[2 * qq]; a1 *= vsc[2 * qq]; a2 *= vsc[2 * qq]; a3 *= vsc[2 * qq];
                    b0 *= vsc[2 * qq + 1]; b1 *= vsc[2 * qq + 1]; b2 *= vsc[2 * qq + 1];
                    b3 *= vsc[2 * qq + 1];
                }
                if constexpr (KV_INT8 != 0) {
                    // value scale folded in; f16 keeps 11 significant bits
                    w.x = pack_f16x2(a0, b0);
                    w.y = pack_f16x2(a1, b1);
                    w.z = pack_f16x2(a2, b2);
                    w.w = pack_f16x2(a3, b3);
                } else {
                    w.x = pack_bf16x2(a0, b0);
                    w.y = pack_bf16x2(a1, b1);
                    w.z = pack_bf16x2(a2, b2);
                    w.w = pack_bf16x2(a3, b3);
                }
                *reinterpret_cast<uint4 *>(&pbuf[wave][4 * qq + (n >> 2)][n & 3][0]) = w;
            }
        }
        // LDS ops of one wave complete in order; this only stops the compiler
        // from moving the reads above the writes.
        __asm__ volatile("" ::: "memory");

        // ---- P.V
#pragma unroll
        for (int h = 0; h < 4; ++h) {
#pragma unroll
            for (int d = 0; d < 8; ++d) acc[h][d] *= alpha[h];
            if constexpr (KV_INT8 != 0) psum[h] *= alpha[h];
        }
        if constexpr (KV_INT8 == 0) {
            // rows past the context may hold anything (even NaN): zero them,
            // their probabilities are already 0
            if (valid < P) {
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (4 * i + vr >= valid) {
                        vw[i][0] = 0u; vw[i][1] = 0u; vw[i][2] = 0u; vw[i][3] = 0u;
                    }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint4 pk = *reinterpret_cast<const uint4 *>(&pbuf[wave][u][vr][0]);
                const int ia = u < 4 ? u : u + 4;       // token 4*ia + r
                const int ib = ia + 4;                  // token 4*ia + r + 16
                const uint32_t ph[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t lo = __builtin_amdgcn_perm(vw[ib][e], vw[ia][e], 0x05040100u);
                    const uint32_t hi = __builtin_amdgcn_perm(vw[ib][e], vw[ia][e], 0x07060302u);
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        acc[h][2 * e] = dot2(ph[h], lo, acc[h][2 * e]);
                        acc[h][2 * e + 1] = dot2(ph[h], hi, acc[h][2 * e + 1]);
                    }
                }
            }
        } else {
            // int8 codes are finite and masked tokens have probability 0, so
            // no masking is needed; psum tracks sum(p') for the 1152 bias.
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const uint4 pk = *reinterpret_cast<const uint4 *>(&pbuf[wave][u][vr][0]);
                const int ia = u < 4 ? u : u + 4;
                const int ib = ia + 4;
                const uint32_t ph[4] = {pk.x, pk.y, pk.z, pk.w};
#pragma unroll
                for (int h = 0; h < 4; ++h) psum[h] = dot2_f16(ph[h], kF16One2, psum[h]);
                uint32_t vp[8];
                vp[0] = i8_pair_f16<0>(vraw[ib].x, vraw[ia].x);
                vp[1] = i8_pair_f16<1>(vraw[ib].x, vraw[ia].x);
                vp[2] = i8_pair_f16<2>(vraw[ib].x, vraw[ia].x);
                vp[3] = i8_pair_f16<3>(vraw[ib].x, vraw[ia].x);
                vp[4] = i8_pair_f16<0>(vraw[ib].y, vraw[ia].y);
                vp[5] = i8_pair_f16<1>(vraw[ib].y, vraw[ia].y);
                vp[6] = i8_pair_f16<2>(vraw[ib].y, vraw[ia].y);
                vp[7] = i8_pair_f16<3>(vraw[ib].y, vraw[ia].y);
#pragma unroll
                for (int d = 0; d < 8; ++d)
#pragma unroll
                    for (int h = 0; h < 4; ++h) acc[h][d] = dot2_f16(ph[h], vp[d], acc[h][d]);
            }
        }
        __asm__ volatile("" ::: "memory");
    }
    if constexpr (KV_INT8 != 0) {
        // remove the 1152 bias carried by every f16 value code
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int d = 0; d < 8; ++d) acc[h][d] = __builtin_fmaf(-kI8Bias, psum[h], acc[h][d]);
    }

    // ---- wave epilogue: l over the 16 lanes of a row; acc over the 4 token phases
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        lpart[h] = row_sum16(lpart[h]);
#pragma unroll
        for (int d = 0; d < 8; ++d) {
            float x = acc[h][d];
            x += __shfl_xor(x, 16);
            x += __shfl_xor(x, 32);
            acc[h][d] = x;
        }
    }
    if (lane == 0) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            sm_m[wave][h] = m[h];
            sm_l[wave][h] = lpart[h];
        }
    }
    if (lane < 16) {
#pragma unroll
        for (int h = 0; h < 4; ++h)
#pragma unroll
            for (int d = 0; d < 8; ++d) sm_acc[wave][h][8 * vc + d] = acc[h][d];
    }
    __syncthreads();

    // ---- merge the NW waves (wave order) and write this split's partial state
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
        const float mnat = M == kNegInf ? kNegInf : M * kLn2;
        if constexpr (FUSED) {
            st_sys(p.part_acc + idx * D + d, o);
            if (d == 0) {
                st_sys(p.part_max + idx, mnat);
                st_sys(p.part_sum + idx, l);
            }
        } else {
            p.part_acc[idx * D + d] = o;
            if (d == 0) {
                p.part_max[idx] = mnat;
                p.part_sum[idx] = l;
            }
        }
    }

    if constexpr (FUSED) {
        // Last-split-done: the partial state above went to memory with
        // write-through stores; once every wave's stores have completed, one
        // thread counts this split in with a memory-side atomic.  The split
        // that arrives last (count S-1) reads all S partial states from memory,
        // merges them in split order and resets the counter for the next call.
        __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) {
            const int old = __hip_atomic_fetch_add(p.counters + grp, 1, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_SYSTEM);
            sm_last = (old == S - 1);
        }
        __syncthreads();
        if (sm_last) {
            for (int e = threadIdx.x; e < kGroup * D; e += NW * 64) {
                const int h = e / D, d = e - h * D;
                merge_element<true>(p.part_acc, p.part_max, p.part_sum, S, D, head0 + h, d,
                                    p.out, p.lse);
            }
            if (threadIdx.x == 0)
                __hip_atomic_store(p.counters + grp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
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
        merge_element<false>(acc, mx, sum, splits, head_dim, row, d, out, lse);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t *__restrict__ ptr, size_t words) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < words; i += stride)
        ptr[i] = 0u;
}

template <int KV, int NW>
hipError_t launch_nw(const DecodeParams &p, bool fused, hipStream_t stream) {
    const unsigned grid = (unsigned)(p.batch * p.hkv * p.splits);
    if (fused)
        hipLaunchKernelGGL((decode_kernel<KV, NW, true>), dim3(grid), dim3(NW * 64), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_kernel<KV, NW, false>), dim3(grid), dim3(NW * 64), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams &p, int kv_int8, bool fused, hipStream_t stream) {
    hipError_t err = kv_int8 ? launch_nw<1, 4>(p, fused, stream) : launch_nw<0, 4>(p, fused, stream);
    if (err != hipSuccess || fused) return err;
    return launch_split_merge(p.part_acc, p.part_max, p.part_sum, p.batch * p.hq, kHeadDim,
                              p.splits, p.out, p.lse, stream);
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
