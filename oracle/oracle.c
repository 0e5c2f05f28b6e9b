/*
 * oracle.c -- plain, slow, fp64 CPU reference for split-K paged-attention
 * decode and its page-table / cu_seqlens metadata build.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file or the library built from it; only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg use it.  It shares no code,
 * header or constant with the HIP kernels.
 *
 * Sources it follows (the pages, not any implementation):
 *  - sglang "trtllm_mha_graph_metadata.py", module docstring and the kernel's
 *    row and cumsum branches: cache_seqlens = seq_lens + seqlen_offset (int32),
 *    cu_seqlens_k[1:] = cumsum(cache_seqlens) (int32), page_table[i, p] =
 *    req_to_token[req_pool_indices[i], p * page_size] // page_size for every
 *    p < max_seq_pages; and its optional outputs (the docstring, the row
 *    branch's sliding-window part, the cumsum branch's q modes, the
 *    swa-out branch and the launcher's num_out_tokens): cu_seqlens_q by
 *    cumsum of qlens or by (i + 1) * q_stride, the sliding-window page table
 *    through full_to_swa with -1 for unmapped slots, and swa_out_cache_loc
 *    translated through full_to_swa and zero padded.
 *  - lmdeploy PR "use PDL for paged attention", Summary/Changes: split-K
 *    paged attention for decode, a producer writing per-split scratch and a
 *    reducer that merges it.  The attention itself is the plain definition
 *    of scaled-dot-product softmax attention of one query token over the
 *    request's cached tokens; split-K is an exact reformulation of it, so
 *    oracle_paged_attention computes the definition directly and the split
 *    functions exist only to pin the split-merge contract.
 *
 * Readings where the pages are silent (all documented with the design):
 *  - KV pool layout [num_pages, P, Hkv, D]; token t of request b is row
 *    (page_table[b, t / P], t % P).
 *  - query head h reads KV head h / (Hq / Hkv).
 *  - s_t = scale * q . k_t with scale the float32 value given, widened.
 *  - int8 KV: k = (double)q8 * (double)sigma per (token, kv head).
 *  - fp8 KV (OCP e4m3, bias 7, no infinities; codes 0x7F / 0xFF are NaN):
 *    k = e4m3(code) * (double)sigma per (token, kv head).
 *  - lse = m + ln(sum_t exp(s_t - m)), natural log, scale applied.
 *  - split j of a request covers logical pages [j*pps, min((j+1)*pps, pages))
 *    with pages = ceil(L/P), pps = ceil(pages/S); an empty split's state is
 *    (m = -inf, l = 0, acc = 0); the merge walks j = 0..S-1 in order.
 *  - L = 0: out = 0, lse = -inf.
 *  - floor division (Python "//") for negative token slots.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_KV_BF16 0
#define ORACLE_KV_INT8 1
#define ORACLE_KV_FP8 2

/* bf16 bit pattern -> double: the bits are the top half of a float32. */
static double bf16_to_double(uint16_t bits) {
    uint32_t u = ((uint32_t)bits) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Value of an OCP e4m3 code: sign bit 7, exponent bits 6..3 with bias 7,
 * mantissa bits 2..0; exponent field 0 is subnormal (2^-6 * m/8); exponent
 * 15 with mantissa 7 is NaN; there are no infinities. */
static double e4m3_to_double(uint8_t code) {
    int sign = code >> 7, e = (code >> 3) & 15, m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double v = e == 0 ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Python-style floor division of a (possibly negative) int by a positive int. */
static int64_t floor_div(int64_t a, int64_t b) {
    int64_t q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) q -= 1;
    return q;
}

/* Metadata build, by definition (sglang docstring / row + cumsum branches). */
int oracle_build_page_table(const int32_t *req_to_token, int64_t req_to_token_stride,
                            const int32_t *req_pool_indices, const int32_t *seq_lens,
                            int32_t bs, int32_t seqlen_offset, int32_t page_size,
                            int32_t max_seq_pages, int32_t *page_table,
                            int64_t page_table_stride, int32_t *cache_seqlens,
                            int32_t *cu_seqlens_k) {
    if (bs == 0) return 0;
    if (page_size <= 0) return 1;
    for (int32_t i = 0; i < bs; ++i) {
        /* int32 wrap-around, as an int32 add would do */
        cache_seqlens[i] = (int32_t)(uint32_t)((uint32_t)seq_lens[i] + (uint32_t)seqlen_offset);
        int64_t row = (int64_t)req_pool_indices[i];
        for (int32_t p = 0; p < max_seq_pages; ++p) {
            int64_t slot = req_to_token[row * req_to_token_stride + (int64_t)p * page_size];
            page_table[(int64_t)i * page_table_stride + p] = (int32_t)floor_div(slot, page_size);
        }
    }
    uint32_t run = 0;
    cu_seqlens_k[0] = 0;
    for (int32_t i = 0; i < bs; ++i) {
        run += (uint32_t)cache_seqlens[i];
        cu_seqlens_k[i + 1] = (int32_t)run;
    }
    return 0;
}

/* The full metadata update, by definition (sglang docstring, kernel row,
 * cumsum and swa-out branches, launcher):
 *   everything oracle_build_page_table computes, plus
 *   cu_seqlens_q[1 + i] = sum_{i' <= i} qlens[i']        (q_mode 1, int32)
 *   cu_seqlens_q[1 + i] = (i + 1) * q_stride             (q_mode 2, int32)
 *   cu_seqlens_q untouched                               (q_mode 0)
 *   swa_page_table[i, p] = -1 if token < 0 or swa[token] < 0,
 *                          else floor(swa[token] / page_size),
 *     token = req_to_token[req_pool_indices[i], p * page_size]  (when swa given)
 *   swa_out_cache_loc[k] = -1 if loc < 0, else swa[loc], loc = out_cache_loc[k],
 *     for k < num_out = min(swa_out_len, n_out_cache_loc); 0 for
 *     num_out <= k < swa_out_len                         (when swa_out given)
 * Like cu_seqlens_k[0], cu_seqlens_q[0] is written as 0 in modes 1 and 2
 * (the source writes [1:] and relies on a preset 0).  bs == 0 writes nothing
 * at all, the zero padding included (the launcher returns first). */
int oracle_build_metadata(const int32_t *req_to_token, int64_t req_to_token_stride,
                          const int32_t *req_pool_indices, const int32_t *seq_lens, int32_t bs,
                          int32_t seqlen_offset, int32_t page_size, int32_t max_seq_pages,
                          int32_t *page_table, int64_t page_table_stride,
                          int32_t *cache_seqlens, int32_t *cu_seqlens_k, int q_mode,
                          const int32_t *qlens, int32_t q_stride, int32_t *cu_seqlens_q,
                          const int64_t *swa, int32_t *swa_page_table,
                          int64_t swa_page_table_stride, const int64_t *out_cache_loc,
                          int64_t n_out_cache_loc, int64_t *swa_out_cache_loc,
                          int64_t swa_out_len) {
    if (bs == 0) return 0;
    int rc = oracle_build_page_table(req_to_token, req_to_token_stride, req_pool_indices,
                                     seq_lens, bs, seqlen_offset, page_size, max_seq_pages,
                                     page_table, page_table_stride, cache_seqlens,
                                     cu_seqlens_k);
    if (rc) return rc;
    if (q_mode == 1 || q_mode == 2) cu_seqlens_q[0] = 0;
    if (q_mode == 1) {
        uint32_t run = 0;
        for (int32_t i = 0; i < bs; ++i) {
            run += (uint32_t)qlens[i];
            cu_seqlens_q[i + 1] = (int32_t)run;
        }
    } else if (q_mode == 2) {
        for (int32_t i = 0; i < bs; ++i)
            cu_seqlens_q[i + 1] = (int32_t)(uint32_t)((uint64_t)(i + 1) * (uint64_t)(uint32_t)q_stride);
    } else if (q_mode != 0) {
        return 1;
    }
    if (swa_page_table) {
        for (int32_t i = 0; i < bs; ++i) {
            int64_t row = (int64_t)req_pool_indices[i];
            for (int32_t p = 0; p < max_seq_pages; ++p) {
                int64_t token = req_to_token[row * req_to_token_stride + (int64_t)p * page_size];
                int64_t v = token < 0 ? -1 : swa[token];
                swa_page_table[(int64_t)i * swa_page_table_stride + p] =
                    (int32_t)(v < 0 ? -1 : floor_div(v, page_size));
            }
        }
    }
    if (swa_out_cache_loc) {
        int64_t num_out = n_out_cache_loc < swa_out_len ? n_out_cache_loc : swa_out_len;
        if (!out_cache_loc) num_out = 0;
        for (int64_t k = 0; k < swa_out_len; ++k) {
            if (k < num_out) {
                int64_t loc = out_cache_loc[k];
                swa_out_cache_loc[k] = loc < 0 ? -1 : swa[loc];
            } else {
                swa_out_cache_loc[k] = 0;
            }
        }
    }
    return 0;
}

typedef struct {
    const uint16_t *q;
    const void *k_pages, *v_pages;
    const float *k_scales, *v_scales;
    int kv_dtype;
    const int32_t *page_table;
    int64_t page_table_stride;
    const int32_t *seq_lens;
    int B, Hq, Hkv, D, P;
    double scale;
    int64_t q_row;   /* query row to use instead of b (multi-token decode), or -1 */
} oracle_args;

/* Dequantised element idx of the int8 / e4m3 K (which = 0) or V pool: the
 * code's value times the scale of its (pool row, kv head).  Kept out of line
 * so that the bf16 element read stays small enough to be inlined. */
static __attribute__((noinline)) double quantized_elem(const oracle_args *a, int which,
                                                      int64_t row, int kvh, int64_t idx) {
    const float *sc = which ? a->v_scales : a->k_scales;
    double sigma = (double)sc[row * a->Hkv + kvh];
    if (a->kv_dtype == ORACLE_KV_FP8) {
        const uint8_t *base = (const uint8_t *)(which ? a->v_pages : a->k_pages);
        return e4m3_to_double(base[idx]) * sigma;
    }
    const int8_t *base = (const int8_t *)(which ? a->v_pages : a->k_pages);
    return (double)base[idx] * sigma;
}

/* Element d of the K (which = 0) or V (which = 1) row of token t, KV head kvh. */
static double kv_elem(const oracle_args *a, int which, int b, int t, int kvh, int d) {
    int64_t page = a->page_table[(int64_t)b * a->page_table_stride + t / a->P];
    int64_t row = page * a->P + (t % a->P);
    int64_t idx = (row * a->Hkv + kvh) * a->D + d;
    if (a->kv_dtype == ORACLE_KV_BF16) {
        const uint16_t *base = (const uint16_t *)(which ? a->v_pages : a->k_pages);
        return bf16_to_double(base[idx]);
    }
    return quantized_elem(a, which, row, kvh, idx);
}

/* s_t = scale * q[b,h,:] . k_t */
static double score(const oracle_args *a, int b, int h, int t) {
    int kvh = h / (a->Hq / a->Hkv);
    double acc = 0.0;
    int64_t row = a->q_row >= 0 ? a->q_row : b;
    for (int d = 0; d < a->D; ++d)
        acc += bf16_to_double(a->q[(row * a->Hq + h) * a->D + d]) *
               kv_elem(a, 0, b, t, kvh, d);
    return a->scale * acc;
}

/* Softmax attention over tokens [t0, t1) of request b, head h:
 * m = max s, l = sum exp(s - m), acc = sum exp(s - m) v  (unnormalised). */
static void attend_range(const oracle_args *a, int b, int h, int t0, int t1,
                         double *m_out, double *l_out, double *acc) {
    int kvh = h / (a->Hq / a->Hkv);
    for (int d = 0; d < a->D; ++d) acc[d] = 0.0;
    if (t1 <= t0) {
        *m_out = -INFINITY;
        *l_out = 0.0;
        return;
    }
    double *s = (double *)malloc(sizeof(double) * (size_t)(t1 - t0));
    double m = -INFINITY;
    for (int t = t0; t < t1; ++t) {
        s[t - t0] = score(a, b, h, t);
        if (s[t - t0] > m) m = s[t - t0];
    }
    double l = 0.0;
    for (int t = t0; t < t1; ++t) {
        double p = exp(s[t - t0] - m);
        l += p;
        for (int d = 0; d < a->D; ++d) acc[d] += p * kv_elem(a, 1, b, t, kvh, d);
    }
    free(s);
    *m_out = m;
    *l_out = l;
}

static void set_args(oracle_args *a, const uint16_t *q, const void *k_pages, const void *v_pages,
                     const float *k_scales, const float *v_scales, int kv_dtype,
                     const int32_t *page_table, int64_t page_table_stride,
                     const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int P,
                     float scale) {
    a->q = q;
    a->k_pages = k_pages;
    a->v_pages = v_pages;
    a->k_scales = k_scales;
    a->v_scales = v_scales;
    a->kv_dtype = kv_dtype;
    a->page_table = page_table;
    a->page_table_stride = page_table_stride;
    a->seq_lens = seq_lens;
    a->B = B;
    a->Hq = Hq;
    a->Hkv = Hkv;
    a->D = D;
    a->P = P;
    a->scale = (double)scale;
    a->q_row = -1;
}

static int check_shape(int B, int Hq, int Hkv, int D, int P) {
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || P <= 0) return 1;
    if (Hq % Hkv != 0) return 1;
    return 0;
}

/* Plain definition: out[b,h,:] = sum_t softmax(s)_t v_t, lse = m + ln l. */
int oracle_paged_attention(const uint16_t *q, const void *k_pages, const void *v_pages,
                           const float *k_scales, const float *v_scales, int kv_dtype,
                           const int32_t *page_table, int64_t page_table_stride,
                           const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int P,
                           float scale, double *out, double *lse) {
    if (check_shape(B, Hq, Hkv, D, P)) return 1;
    oracle_args a;
    set_args(&a, q, k_pages, v_pages, k_scales, v_scales, kv_dtype, page_table,
             page_table_stride, seq_lens, B, Hq, Hkv, D, P, scale);
    long n = (long)B * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (long bh = 0; bh < n; ++bh) {
        int b = (int)(bh / Hq), h = (int)(bh % Hq);
        double m, l;
        double *o = out + bh * D;
        attend_range(&a, b, h, 0, seq_lens[b], &m, &l, o);
        if (l > 0.0) {
            for (int d = 0; d < D; ++d) o[d] /= l;
            lse[bh] = m + log(l);
        } else {
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            lse[bh] = -INFINITY;
        }
    }
    return 0;
}

/* Multi-token query decode (target verify / draft extend), by definition.
 * Request b owns query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (n_b of
 * them) and L_b = seq_lens[b] cached tokens, the last n_b of which are the
 * query tokens' own: query token i (row cu_seqlens_q[b] + i) attends the
 * tokens 0 .. L_b - n_b + i (causal within the draft).  For each row r and
 * head h: out[r,h,:] = sum_t softmax(s)_t v_t over those tokens, lse = m +
 * ln l; out = 0 and lse = -inf where a row sees no token.  q, out: [total_q,
 * Hq, D]; lse [total_q, Hq]. */
int oracle_paged_verify_attention(const uint16_t *q, const void *k_pages, const void *v_pages,
                                  const float *k_scales, const float *v_scales, int kv_dtype,
                                  const int32_t *page_table, int64_t page_table_stride,
                                  const int32_t *seq_lens, const int32_t *cu_seqlens_q, int B,
                                  int total_q, int Hq, int Hkv, int D, int P, float scale,
                                  double *out, double *lse) {
    if (check_shape(B, Hq, Hkv, D, P) || total_q < 0) return 1;
    for (int b = 0; b < B; ++b)
        if (cu_seqlens_q[b + 1] < cu_seqlens_q[b] || cu_seqlens_q[b] < 0 ||
            cu_seqlens_q[b + 1] > total_q)
            return 1;
    long n = (long)total_q * Hq;
#pragma omp parallel for schedule(dynamic, 1)
    for (long rh = 0; rh < n; ++rh) {
        int row = (int)(rh / Hq), h = (int)(rh % Hq);
        double *o = out + rh * D;
        int b = -1;
        for (int bb = 0; bb < B; ++bb)
            if (row >= cu_seqlens_q[bb] && row < cu_seqlens_q[bb + 1]) b = bb;
        int visible = 0;
        if (b >= 0) {
            int nq = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
            int i = row - cu_seqlens_q[b];
            visible = seq_lens[b] - nq + i + 1;
            if (visible < 0) visible = 0;
            if (visible > seq_lens[b]) visible = seq_lens[b];
        }
        oracle_args a;
        set_args(&a, q, k_pages, v_pages, k_scales, v_scales, kv_dtype, page_table,
                 page_table_stride, seq_lens, B, Hq, Hkv, D, P, scale);
        a.q_row = row;
        double m = -INFINITY, l = 0.0;
        if (b >= 0) attend_range(&a, b, h, 0, visible, &m, &l, o);
        if (l > 0.0) {
            for (int d = 0; d < D; ++d) o[d] /= l;
            lse[rh] = m + log(l);
        } else {
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            lse[rh] = -INFINITY;
        }
    }
    return 0;
}

/* Per-split partial state (split rule in the header comment).
 * acc [B, Hq, S, D], m and l [B, Hq, S]; m in natural-log units of s. */
int oracle_split_partials(const uint16_t *q, const void *k_pages, const void *v_pages,
                          const float *k_scales, const float *v_scales, int kv_dtype,
                          const int32_t *page_table, int64_t page_table_stride,
                          const int32_t *seq_lens, int B, int Hq, int Hkv, int D, int P,
                          float scale, int S, double *acc, double *m, double *l) {
    if (check_shape(B, Hq, Hkv, D, P) || S <= 0) return 1;
    oracle_args a;
    set_args(&a, q, k_pages, v_pages, k_scales, v_scales, kv_dtype, page_table,
             page_table_stride, seq_lens, B, Hq, Hkv, D, P, scale);
    long n = (long)B * Hq * S;
#pragma omp parallel for schedule(dynamic, 1)
    for (long idx = 0; idx < n; ++idx) {
        int j = (int)(idx % S);
        long bh = idx / S;
        int b = (int)(bh / Hq), h = (int)(bh % Hq);
        int L = seq_lens[b];
        int pages = (L + P - 1) / P;
        int pps = (pages + S - 1) / S;
        int p0 = j * pps, p1 = (j + 1) * pps;
        if (p1 > pages) p1 = pages;
        int t0 = p0 * P, t1 = p1 * P;
        if (t1 > L) t1 = L;
        if (t0 > t1) t0 = t1;
        attend_range(&a, b, h, t0, t1, &m[idx], &l[idx], acc + idx * D);
    }
    return 0;
}

/* Log-sum-exp merge of S partial states, j = 0..S-1 in order:
 * M = max m_j; w_j = exp(m_j - M) (0 for an empty split);
 * out = sum w_j acc_j / sum w_j l_j; lse = M + ln(sum w_j l_j). */
int oracle_split_merge(const double *acc, const double *m, const double *l, int B, int Hq,
                       int D, int S, double *out, double *lse) {
    if (B < 0 || Hq <= 0 || D <= 0 || S <= 0) return 1;
    long n = (long)B * Hq;
    for (long bh = 0; bh < n; ++bh) {
        const double *mj = m + bh * S, *lj = l + bh * S;
        double M = -INFINITY;
        for (int j = 0; j < S; ++j)
            if (mj[j] > M) M = mj[j];
        double *o = out + bh * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        double lsum = 0.0;
        for (int j = 0; j < S; ++j) {
            if (mj[j] == -INFINITY) continue;
            double w = exp(mj[j] - M);
            lsum += w * lj[j];
            const double *aj = acc + (bh * S + j) * D;
            for (int d = 0; d < D; ++d) o[d] += w * aj[d];
        }
        if (lsum > 0.0) {
            for (int d = 0; d < D; ++d) o[d] /= lsum;
            lse[bh] = M + log(lsum);
        } else {
            for (int d = 0; d < D; ++d) o[d] = 0.0;
            lse[bh] = -INFINITY;
        }
    }
    return 0;
}

int oracle_abi_version(void) { return 1; }
