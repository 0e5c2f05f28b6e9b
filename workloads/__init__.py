"""Seeded synthetic inputs for split-K paged-attention decode.

This module is the only code shared by the HIP path's tests/bench and the CPU
oracle.  It draws data and lays it out; it holds none of the decode method's
arithmetic (no dot products, no softmax, no page-table division).

What it builds, following the workloads the source pages measure (lmdeploy PR
"use PDL for paged attention", Performance table: batch 1/8/32, context 1K/8K)
and the metadata layout of sglang's fused CUDA-graph metadata kernel (kernel
argument list: req_to_token [pool, stride] int32, req_pool_indices [bs],
seq_lens [bs]):

* a pool of ``num_pages`` physical KV pages, layout [num_pages, P, Hkv, D]
  (a flat token slot s is row (s // P, s % P) of that pool); EVERY page is
  filled with N(0,1) data, used or not, so a read of a wrong page changes the
  result;
* request b's logical page p lives at physical page perm[offset_b + p], where
  perm is a seeded permutation of the pool and offset_b the running page count
  (so pages of different requests interleave at random);
* req_to_token rows: row req_pool_indices[b] holds slot perm[offset_b + t//P]*P
  + t%P for t < ceil(L_b/P)*P and random valid slots after that; rows used by
  no request hold random valid slots;
* bf16 values are N(0,1) float32 rounded to bf16 (round half to even) and
  stored as raw uint16 bit patterns;
* int8 values: per (page, row, kv_head) a float32 N(0,1) vector over D is
  quantised symmetrically, sigma = amax/127 (float32),
  q8 = clamp(rint(x/sigma), -127, 127) with rint rounding half to even.
* fp8 values (OCP e4m3, "e4m3fn": bias 7, no infinities, 448 the largest
  finite value): per (page, row, kv_head) sigma = amax/448 (float32) and
  each x/sigma (float32) is rounded to the nearest e4m3 value, ties to the
  even code, stored as uint8 codes (never a NaN code).

Determinism: large arrays are split into fixed chunks along their first axis
and chunk i draws from PCG64(SeedSequence(seed, spawn_key=(tag, i))); the
result does not depend on how many threads fill the chunks.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# Shapes fixed by the measured workloads (32 query heads over 8 KV heads,
# head_dim 128, 64-token pages) and by the metadata kernel's req_to_token map.
NUM_Q_HEADS = 32
NUM_KV_HEADS = 8
HEAD_DIM = 128
PAGE_SIZE = 64
REQ_POOL_ROWS = 64
REQ_TO_TOKEN_STRIDE = 8192
MAX_SEQ_PAGES = 128
SCALE = np.float32(1.0 / np.sqrt(np.float64(HEAD_DIM)))

_TAG_Q, _TAG_K, _TAG_V, _TAG_PERM, _TAG_LEN, _TAG_RPI, _TAG_FILL, _TAG_QROWS, _TAG_ROT = range(1, 10)
_CHUNK_ELEMS = 1 << 22


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen(seed: int, tag: int, idx: int = 0) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tag, idx))))


def _chunked(shape, seed: int, tag: int, fill_chunk) -> None:
    """Split axis 0 of ``shape`` into chunks and call fill_chunk(i, lo, hi, rng)."""
    n0 = shape[0]
    inner = int(np.prod(shape[1:])) if len(shape) > 1 else 1
    rows = max(1, _CHUNK_ELEMS // max(1, inner))
    spans = [(i, lo, min(n0, lo + rows)) for i, lo in enumerate(range(0, n0, rows))]
    if len(spans) <= 1:
        for i, lo, hi in spans:
            fill_chunk(i, lo, hi, _gen(seed, tag, i))
        return
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda s: fill_chunk(s[0], s[1], s[2], _gen(seed, tag, s[0])), spans))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round half to even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(shape, seed: int, tag: int) -> np.ndarray:
    out = np.empty(shape, dtype=np.uint16)

    def fill(i, lo, hi, rng):
        x = rng.standard_normal((hi - lo,) + tuple(shape[1:]), dtype=np.float32)
        out[lo:hi] = f32_to_bf16_bits(x)

    _chunked(shape, seed, tag, fill)
    return out


def normal_int8(shape, seed: int, tag: int):
    """Symmetric int8 quantisation of N(0,1) vectors over the last axis.

    Returns (q8 int8 [..., D], sigma float32 [...])."""
    q8 = np.empty(shape, dtype=np.int8)
    sig = np.empty(shape[:-1], dtype=np.float32)

    def fill(i, lo, hi, rng):
        x = rng.standard_normal((hi - lo,) + tuple(shape[1:]), dtype=np.float32)
        amax = np.max(np.abs(x), axis=-1)
        s = (amax / np.float32(127.0)).astype(np.float32)
        s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
        q = np.rint(x / s[..., None])
        q8[lo:hi] = np.clip(q, -127, 127).astype(np.int8)
        sig[lo:hi] = s

    _chunked(shape, seed, tag, fill)
    return q8, sig


def _e4m3_magnitudes() -> np.ndarray:
    """Values of the non-negative finite e4m3 codes 0..126, increasing."""
    c = np.arange(127)
    e, m = c >> 3, (c & 7).astype(np.float64)
    return np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))


def encode_e4m3(y: np.ndarray) -> np.ndarray:
    """Round float values to e4m3 codes: nearest, ties to the even code,
    magnitudes above 448 saturated to 448."""
    tab = _e4m3_magnitudes()
    a = np.minimum(np.abs(y.astype(np.float64)), tab[-1])
    hi = np.clip(np.searchsorted(tab, a, side="left"), 0, 126)
    lo = np.maximum(hi - 1, 0)
    dlo, dhi = a - tab[lo], tab[hi] - a
    code = np.where((dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0)), hi, lo)
    return (code | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def normal_fp8(shape, seed: int, tag: int):
    """e4m3 quantisation of N(0,1) vectors over the last axis, scaled so the
    largest magnitude becomes 448.  Returns (codes uint8 [..., D], sigma
    float32 [...])."""
    codes = np.empty(shape, dtype=np.uint8)
    sig = np.empty(shape[:-1], dtype=np.float32)

    def fill(i, lo, hi, rng):
        x = rng.standard_normal((hi - lo,) + tuple(shape[1:]), dtype=np.float32)
        amax = np.max(np.abs(x), axis=-1)
        s = (amax / np.float32(448.0)).astype(np.float32)
        s = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
        codes[lo:hi] = encode_e4m3((x / s[..., None]).astype(np.float32))
        sig[lo:hi] = s

    _chunked(shape, seed, tag, fill)
    return codes, sig


@dataclass
class DecodeCase:
    """One seeded decode batch: query, paged KV pool and the req_to_token map."""
    name: str
    seed: int
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    num_splits: int
    kv_dtype: str                       # "bf16", "int8" or "fp8"
    scale: np.float32
    q: np.ndarray                       # uint16 bf16 bits [B, Hq, D]
    k_pages: np.ndarray                 # uint16, int8 or uint8 (e4m3) [num_pages, P, Hkv, D]
    v_pages: np.ndarray
    k_scales: Optional[np.ndarray]      # float32 [num_pages, P, Hkv] (int8 / fp8 only)
    v_scales: Optional[np.ndarray]
    seq_lens: np.ndarray                # int32 [B]
    req_to_token: np.ndarray            # int32 [rows, stride]
    req_pool_indices: np.ndarray        # int32 [B]
    page_list: np.ndarray               # int32 [B, max_seq_pages]; -1 past the request's pages
    max_seq_pages: int
    seqlen_offset: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def dense_kv(self, b: int):
        """Logical K/V rows of request b in token order, from the generator's
        own placement (page_list), not from req_to_token or a page table.

        Returns (k [L, Hkv, D], v [L, Hkv, D], k_scales [L, Hkv] | None,
        v_scales [L, Hkv] | None) in the stored dtypes."""
        L = int(self.seq_lens[b])
        P = self.page_size
        npg = -(-L // P)
        pages = self.page_list[b, :npg]
        k = self.k_pages[pages].reshape(npg * P, self.num_kv_heads, self.head_dim)[:L]
        v = self.v_pages[pages].reshape(npg * P, self.num_kv_heads, self.head_dim)[:L]
        if self.k_scales is None:
            return k, v, None, None
        ks = self.k_scales[pages].reshape(npg * P, self.num_kv_heads)[:L]
        vs = self.v_scales[pages].reshape(npg * P, self.num_kv_heads)[:L]
        return k, v, ks, vs

    def kv_bytes_per_token(self) -> int:
        per = self.num_kv_heads * self.head_dim * (2 if self.kv_dtype == "bf16" else 1)
        if self.kv_dtype != "bf16":
            per += self.num_kv_heads * 4
        return 2 * per


def make_case(*, seed: int, seq_lens, num_pages: int, num_splits: int,
              kv_dtype: str = "bf16", num_q_heads: int = NUM_Q_HEADS,
              num_kv_heads: int = NUM_KV_HEADS, head_dim: int = HEAD_DIM,
              page_size: int = PAGE_SIZE, req_pool_rows: int = REQ_POOL_ROWS,
              req_to_token_stride: int = REQ_TO_TOKEN_STRIDE,
              max_seq_pages: int = MAX_SEQ_PAGES, scale=None, name: str = "custom",
              q_override: Optional[np.ndarray] = None) -> DecodeCase:
    """Build a seeded case.  ``seq_lens`` is a sequence of ints (one per request)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int32).reshape(-1)
    B = int(seq_lens.shape[0])
    P = page_size
    if kv_dtype not in ("bf16", "int8", "fp8"):
        raise ValueError(kv_dtype)
    if B > req_pool_rows:
        raise ValueError("batch larger than the req_to_token pool")
    pages_needed = [-(-int(L) // P) for L in seq_lens]
    if sum(pages_needed) > num_pages:
        raise ValueError(f"pool of {num_pages} pages cannot hold {sum(pages_needed)}")
    if max(pages_needed, default=0) > max_seq_pages:
        raise ValueError("a request needs more pages than max_seq_pages")
    if (max_seq_pages - 1) * P >= req_to_token_stride:
        raise ValueError("req_to_token_stride too small for max_seq_pages")

    perm = _gen(seed, _TAG_PERM).permutation(num_pages).astype(np.int32)
    if q_override is not None:
        q = np.ascontiguousarray(q_override, dtype=np.uint16)
    else:
        q = normal_bf16((B, num_q_heads, head_dim), seed, _TAG_Q)
    shape = (num_pages, P, num_kv_heads, head_dim)
    if kv_dtype == "bf16":
        k_pages = normal_bf16(shape, seed, _TAG_K)
        v_pages = normal_bf16(shape, seed, _TAG_V)
        k_scales = v_scales = None
    elif kv_dtype == "int8":
        k_pages, k_scales = normal_int8(shape, seed, _TAG_K)
        v_pages, v_scales = normal_int8(shape, seed, _TAG_V)
    else:
        k_pages, k_scales = normal_fp8(shape, seed, _TAG_K)
        v_pages, v_scales = normal_fp8(shape, seed, _TAG_V)

    rpi = _gen(seed, _TAG_RPI).choice(req_pool_rows, size=B, replace=False).astype(np.int32)
    fill_rng = _gen(seed, _TAG_FILL)
    r2t = fill_rng.integers(0, num_pages * P, size=(req_pool_rows, req_to_token_stride),
                            dtype=np.int64).astype(np.int32)
    page_list = np.full((B, max_seq_pages), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = pages_needed[b]
        pg = perm[off:off + n]
        off += n
        page_list[b, :n] = pg
        if n:
            slots = (pg.astype(np.int64)[:, None] * P + np.arange(P, dtype=np.int64)[None, :])
            r2t[rpi[b], :n * P] = slots.reshape(-1).astype(np.int32)
    if scale is None:
        scale = np.float32(1.0 / np.sqrt(np.float64(head_dim)))
    return DecodeCase(
        name=name, seed=seed, batch=B, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, page_size=P, num_pages=num_pages, num_splits=num_splits,
        kv_dtype=kv_dtype, scale=np.float32(scale), q=q, k_pages=k_pages, v_pages=v_pages,
        k_scales=k_scales, v_scales=v_scales, seq_lens=seq_lens, req_to_token=r2t,
        req_pool_indices=rpi, page_list=page_list, max_seq_pages=max_seq_pages)


# The five measured workloads: lmdeploy's H200 table (batch 1/ctx 1K,
# batch 1/ctx 8K, batch 8/ctx 1K, batch 32/ctx 8K) plus a ragged int8 batch;
# then the headline shape with e4m3 KV.
CONFIGS = {
    1: dict(name="b1_ctx1k_s4_bf16", lens=("const", 1, 1024), num_pages=256,
            num_splits=4, kv_dtype="bf16"),
    2: dict(name="b1_ctx8k_s16_bf16", lens=("const", 1, 8192), num_pages=1024,
            num_splits=16, kv_dtype="bf16"),
    3: dict(name="b8_ctx1k_s4_bf16", lens=("const", 8, 1024), num_pages=1024,
            num_splits=4, kv_dtype="bf16"),
    4: dict(name="b32_ctx8k_s16_bf16", lens=("const", 32, 8192), num_pages=4096,
            num_splits=16, kv_dtype="bf16"),
    5: dict(name="b32_ragged8k_s16_int8", lens=("uniform", 32, 1, 8192), num_pages=4096,
            num_splits=16, kv_dtype="int8"),
    6: dict(name="b32_ctx8k_s16_fp8", lens=("const", 32, 8192), num_pages=4096,
            num_splits=16, kv_dtype="fp8"),
}


def config_seq_lens(config_id: int) -> np.ndarray:
    spec = CONFIGS[config_id]["lens"]
    if spec[0] == "const":
        return np.full(spec[1], spec[2], dtype=np.int32)
    _, B, lo, hi = spec
    return _gen(config_id, _TAG_LEN).integers(lo, hi + 1, size=B).astype(np.int32)


def make_config(config_id: int) -> DecodeCase:
    spec = CONFIGS[config_id]
    case = make_case(seed=config_id, seq_lens=config_seq_lens(config_id),
                     num_pages=spec["num_pages"], num_splits=spec["num_splits"],
                     kv_dtype=spec["kv_dtype"], name=spec["name"])
    return case


def verify_queries(case: DecodeCase, q_lens, seed: Optional[int] = None):
    """Query rows for multi-token decode (target verify / draft extend) over
    a case's KV cache: request b gets q_lens[b] rows, laid out back to back.
    Returns (q_rows uint16 bf16 bits [total_q, Hq, D], cu_seqlens_q int32
    [B + 1]).  The last q_lens[b] cached tokens of request b are the draft
    tokens these rows stand for."""
    q_lens = np.asarray(q_lens, dtype=np.int32).reshape(-1)
    if q_lens.shape[0] != case.batch or np.any(q_lens < 0) or np.any(q_lens > case.seq_lens):
        raise ValueError("need 0 <= q_lens[b] <= seq_lens[b] for every request")
    cu = np.zeros(case.batch + 1, dtype=np.int32)
    cu[1:] = np.cumsum(q_lens)
    total = int(cu[-1])
    q = normal_bf16((max(total, 1), case.num_q_heads, case.head_dim),
                    case.seed if seed is None else seed, _TAG_QROWS)[:total]
    return np.ascontiguousarray(q), cu


def rotation_layout(case: DecodeCase, copies: int):
    """Layout of ``copies`` disjoint copies of the pages a case's requests
    use, for timing loops that must not find the previous call's data in a
    cache: call i reads copy i % copies.

    Copy c holds every used page once (U pages in all), each at a seeded
    random position of its own range [c*U, (c+1)*U); request b of copy c is
    row c*B + b of a req_to_token map over the copies (the request's slots
    first, random valid slots of the copies after).  Every copy holds the
    same data, so every copy gives the same result.

    Returns (src [copies*U] int64: the case page each copied page holds,
    req_to_token [copies*B, stride] int32, req_pool_indices [copies, B]
    int32)."""
    P, B = case.page_size, case.batch
    stride = case.req_to_token.shape[1]
    npg = [-(-int(L) // P) for L in case.seq_lens]
    used = np.concatenate([case.page_list[b, :n] for b, n in enumerate(npg)]).astype(np.int64)
    U = int(used.shape[0])
    src = np.empty(copies * U, dtype=np.int64)
    rng = _gen(case.seed, _TAG_ROT)
    r2t = rng.integers(0, max(1, copies * U) * P, size=(copies * B, stride),
                       dtype=np.int64).astype(np.int32)
    starts = np.concatenate([[0], np.cumsum(npg)]).astype(np.int64)
    for c in range(copies):
        pos = c * U + rng.permutation(U).astype(np.int64)   # copy c's page for used page i
        src[pos] = used
        for b in range(B):
            n = npg[b]
            if n:
                pg = pos[starts[b]:starts[b] + n]
                slots = pg[:, None] * P + np.arange(P, dtype=np.int64)[None, :]
                r2t[c * B + b, :n * P] = slots.reshape(-1).astype(np.int32)
    rpi = np.arange(copies * B, dtype=np.int32).reshape(copies, B)
    return src, r2t, rpi


def algorithmic_bytes(case: DecodeCase) -> int:
    """Bytes the decode call must move: K/V (+ scales) of exactly the L_b
    tokens, q, out (bf16), lse (fp32), the page-table entries in use and
    seq_lens.  Split scratch is method overhead and is not counted."""
    P = case.page_size
    toks = int(np.sum(case.seq_lens.astype(np.int64)))
    pages = int(sum(-(-int(L) // P) for L in case.seq_lens))
    kv = toks * case.kv_bytes_per_token()
    qo = 2 * case.batch * case.num_q_heads * case.head_dim * 2
    lse = case.batch * case.num_q_heads * 4
    return kv + qo + lse + pages * 4 + case.batch * 4


def verify_algorithmic_bytes(case: DecodeCase, q_lens) -> int:
    """Bytes a multi-token decode call must move: K/V (+ scales) of exactly
    the L_b tokens, the query rows, out (bf16) and lse (fp32) rows, the
    page-table entries in use, seq_lens and cu_seqlens_q."""
    q_lens = np.asarray(q_lens, dtype=np.int64)
    P = case.page_size
    toks = int(np.sum(case.seq_lens.astype(np.int64)))
    pages = int(sum(-(-int(L) // P) for L in case.seq_lens))
    rows = int(q_lens.sum())
    kv = toks * case.kv_bytes_per_token()
    qo = 2 * rows * case.num_q_heads * case.head_dim * 2
    lse = rows * case.num_q_heads * 4
    return kv + qo + lse + pages * 4 + case.batch * 4 + (case.batch + 1) * 4
