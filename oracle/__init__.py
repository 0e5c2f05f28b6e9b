"""fp64 CPU oracle for split-K paged-attention decode (ctypes over liboracle.so).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path (the HIP library
and its Python binding) never does, and shares no code with it.

Every function follows a definition stated in oracle.c:
  build_page_table  -- sglang fused metadata kernel docstring (page_table,
                       cache_seqlens, cu_seqlens_k by definition);
  build_metadata    -- the same update with its optional outputs
                       (cu_seqlens_q modes, sliding-window page table and
                       swa_out_cache_loc);
  paged_attention   -- plain softmax attention of one query token over the
                       paged KV cache (lmdeploy's split-K decode computes this
                       exactly, split-K being a reformulation);
  split_partials    -- per-split (max, sum, unnormalised accumulator) state;
  split_merge       -- log-sum-exp merge of that state.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SPA_ORACLE_LIB lets the mutant test point the pins at a deliberately broken
# copy of the oracle; nothing else sets it.
_LIB_PATH = os.environ.get("SPA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_lib = None

KV_BF16 = 0
KV_INT8 = 1
KV_FP8 = 2

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F32 = ctypes.c_float
_INT = ctypes.c_int


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build(verbose=False)
    lib = ctypes.CDLL(_LIB_PATH)
    lib.oracle_build_page_table.argtypes = [_P, _I64, _P, _P, _I32, _I32, _I32, _I32, _P, _I64,
                                            _P, _P]
    lib.oracle_build_page_table.restype = _INT
    lib.oracle_paged_verify_attention.argtypes = [_P, _P, _P, _P, _P, _INT, _P, _I64, _P, _P,
                                                  _INT, _INT, _INT, _INT, _INT, _INT, _F32, _P,
                                                  _P]
    lib.oracle_paged_verify_attention.restype = _INT
    lib.oracle_build_metadata.argtypes = [_P, _I64, _P, _P, _I32, _I32, _I32, _I32, _P, _I64, _P,
                                          _P, _INT, _P, _I32, _P, _P, _P, _I64, _P, _I64, _P,
                                          _I64]
    lib.oracle_build_metadata.restype = _INT
    att = [_P, _P, _P, _P, _P, _INT, _P, _I64, _P, _INT, _INT, _INT, _INT, _INT, _F32]
    lib.oracle_paged_attention.argtypes = att + [_P, _P]
    lib.oracle_paged_attention.restype = _INT
    lib.oracle_split_partials.argtypes = att + [_INT, _P, _P, _P]
    lib.oracle_split_partials.restype = _INT
    lib.oracle_split_merge.argtypes = [_P, _P, _P, _INT, _INT, _INT, _INT, _P, _P]
    lib.oracle_split_merge.restype = _INT
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def build_page_table(req_to_token, req_pool_indices, seq_lens, page_size, max_seq_pages,
                     seqlen_offset=0, page_table=None):
    """Returns (page_table [bs, stride] int32, cache_seqlens [bs], cu_seqlens_k [bs+1]).

    If ``page_table`` is given it is updated in place (columns >= max_seq_pages
    are left as they are) and its row stride is used."""
    lib = _load()
    r2t = _c(req_to_token, np.int32)
    rpi = _c(req_pool_indices, np.int32)
    sl = _c(seq_lens, np.int32)
    bs = int(rpi.shape[0])
    if page_table is None:
        page_table = np.full((bs, max(1, max_seq_pages)), -0x5A5A5A5A, dtype=np.int32)
    assert page_table.dtype == np.int32 and page_table.flags.c_contiguous
    # poisoned so that an unwritten output entry shows up
    cache = np.full(bs, -0x5A5A5A5A, dtype=np.int32)
    cu = np.full(bs + 1, -0x5A5A5A5A, dtype=np.int32)
    rc = lib.oracle_build_page_table(_ptr(r2t), r2t.shape[1], _ptr(rpi), _ptr(sl), bs,
                                     int(seqlen_offset), int(page_size), int(max_seq_pages),
                                     _ptr(page_table), page_table.shape[1], _ptr(cache), _ptr(cu))
    if rc != 0:
        raise ValueError("oracle_build_page_table: invalid arguments")
    return page_table, cache, cu


def build_metadata(req_to_token, req_pool_indices, seq_lens, page_size, max_seq_pages, *,
                   seqlen_offset=0, page_table=None, q_mode=0, qlens=None, q_stride=0,
                   cu_seqlens_q=None, swa_mapping=None, swa_page_table=None,
                   out_cache_loc=None, swa_out_cache_loc=None):
    """The full metadata update.  Outputs given as arrays are updated in place
    (their unwritten entries keep their values); returns a dict of outputs.
    page_table defaults to a poisoned [bs, max_seq_pages]; swa_page_table=True
    asks for one too (None = no sliding-window table, as in the source)."""
    lib = _load()
    r2t = _c(req_to_token, np.int32)
    rpi = _c(req_pool_indices, np.int32)
    sl = _c(seq_lens, np.int32)
    bs = int(rpi.shape[0])
    poison = -0x5A5A5A5A
    if page_table is None:
        page_table = np.full((bs, max(1, max_seq_pages)), poison, dtype=np.int32)
    cache = np.full(bs, poison, dtype=np.int32)
    cu = np.full(bs + 1, poison, dtype=np.int32)
    if cu_seqlens_q is None:
        cu_seqlens_q = np.full(bs + 1, poison, dtype=np.int32)
    ql = _c(qlens, np.int32) if qlens is not None else None
    swa = _c(swa_mapping, np.int64) if swa_mapping is not None else None
    if isinstance(swa_page_table, bool):
        swa_page_table = (np.full((bs, max(1, max_seq_pages)), poison, dtype=np.int32)
                          if swa_page_table else None)
    ocl = _c(out_cache_loc, np.int64) if out_cache_loc is not None else None
    for a in (page_table, cu_seqlens_q, swa_page_table, swa_out_cache_loc):
        assert a is None or a.flags.c_contiguous
    rc = lib.oracle_build_metadata(
        _ptr(r2t), r2t.shape[1], _ptr(rpi), _ptr(sl), bs, int(seqlen_offset), int(page_size),
        int(max_seq_pages), _ptr(page_table), page_table.shape[1], _ptr(cache), _ptr(cu),
        int(q_mode), _ptr(ql), int(q_stride), _ptr(cu_seqlens_q), _ptr(swa),
        _ptr(swa_page_table), 0 if swa_page_table is None else swa_page_table.shape[1],
        _ptr(ocl), 0 if ocl is None else ocl.shape[0], _ptr(swa_out_cache_loc),
        0 if swa_out_cache_loc is None else swa_out_cache_loc.shape[0])
    if rc != 0:
        raise ValueError("oracle_build_metadata: invalid arguments")
    return dict(page_table=page_table, cache_seqlens=cache, cu_seqlens_k=cu,
                cu_seqlens_q=cu_seqlens_q, swa_page_table=swa_page_table,
                swa_out_cache_loc=swa_out_cache_loc)


def _att_args(q, k_pages, v_pages, k_scales, v_scales, kv_dtype, page_table, seq_lens,
              num_kv_heads, page_size, scale):
    q = _c(q, np.uint16)
    B, Hq, D = q.shape
    if kv_dtype in ("bf16", KV_BF16):
        kd = KV_BF16
        k = _c(k_pages, np.uint16)
        v = _c(v_pages, np.uint16)
        ks = vs = None
    elif kv_dtype in ("int8", KV_INT8):
        kd = KV_INT8
        k = _c(k_pages, np.int8)
        v = _c(v_pages, np.int8)
        ks = _c(k_scales, np.float32)
        vs = _c(v_scales, np.float32)
    elif kv_dtype in ("fp8", KV_FP8):
        kd = KV_FP8
        k = _c(k_pages, np.uint8)
        v = _c(v_pages, np.uint8)
        ks = _c(k_scales, np.float32)
        vs = _c(v_scales, np.float32)
    else:
        raise ValueError(f"unknown kv_dtype {kv_dtype!r}")
    pt = _c(page_table, np.int32)
    sl = _c(seq_lens, np.int32)
    keep = (q, k, v, ks, vs, pt, sl)
    args = [_ptr(q), _ptr(k), _ptr(v), _ptr(ks), _ptr(vs), kd, _ptr(pt), pt.shape[1], _ptr(sl),
            B, Hq, int(num_kv_heads), D, int(page_size), float(np.float32(scale))]
    return keep, args, (B, Hq, D)


def paged_attention(q, k_pages, v_pages, page_table, seq_lens, *, num_kv_heads, page_size,
                    scale, kv_dtype="bf16", k_scales=None, v_scales=None):
    """fp64 out [B, Hq, D] and lse [B, Hq] by the plain definition."""
    lib = _load()
    keep, args, (B, Hq, D) = _att_args(q, k_pages, v_pages, k_scales, v_scales, kv_dtype,
                                       page_table, seq_lens, num_kv_heads, page_size, scale)
    out = np.full((B, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((B, Hq), np.nan, dtype=np.float64)
    rc = lib.oracle_paged_attention(*args, _ptr(out), _ptr(lse))
    del keep
    if rc != 0:
        raise ValueError("oracle_paged_attention: invalid arguments")
    return out, lse


def split_partials(q, k_pages, v_pages, page_table, seq_lens, *, num_kv_heads, page_size,
                   scale, num_splits, kv_dtype="bf16", k_scales=None, v_scales=None):
    """fp64 per-split state: acc [B, Hq, S, D], m [B, Hq, S], l [B, Hq, S]."""
    lib = _load()
    keep, args, (B, Hq, D) = _att_args(q, k_pages, v_pages, k_scales, v_scales, kv_dtype,
                                       page_table, seq_lens, num_kv_heads, page_size, scale)
    S = int(num_splits)
    acc = np.full((B, Hq, S, D), np.nan, dtype=np.float64)
    m = np.full((B, Hq, S), np.nan, dtype=np.float64)
    l = np.full((B, Hq, S), np.nan, dtype=np.float64)
    rc = lib.oracle_split_partials(*args, S, _ptr(acc), _ptr(m), _ptr(l))
    del keep
    if rc != 0:
        raise ValueError("oracle_split_partials: invalid arguments")
    return acc, m, l


def split_merge(acc, m, l):
    """Log-sum-exp merge; inputs acc [B, Hq, S, D], m/l [B, Hq, S] (any float dtype)."""
    lib = _load()
    acc = _c(acc, np.float64)
    m = _c(m, np.float64)
    l = _c(l, np.float64)
    B, Hq, S, D = acc.shape
    out = np.full((B, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((B, Hq), np.nan, dtype=np.float64)
    rc = lib.oracle_split_merge(_ptr(acc), _ptr(m), _ptr(l), B, Hq, D, S, _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_split_merge: invalid arguments")
    return out, lse


def verify_attention(q, k_pages, v_pages, page_table, seq_lens, cu_seqlens_q, *,
                     num_kv_heads, page_size, scale, kv_dtype="bf16", k_scales=None,
                     v_scales=None):
    """Multi-token query decode: q [total_q, Hq, D] bf16 bits, request b's
    query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1, query token i of b sees
    tokens 0 .. seq_lens[b] - n_b + i.  Returns (out [total_q, Hq, D] f64,
    lse [total_q, Hq] f64)."""
    lib = _load()
    keep, args, (total_q, Hq, D) = _att_args(q, k_pages, v_pages, k_scales, v_scales, kv_dtype,
                                             page_table, seq_lens, num_kv_heads, page_size,
                                             scale)
    cu = _c(cu_seqlens_q, np.int32)
    B = int(cu.shape[0]) - 1
    out = np.full((total_q, Hq, D), np.nan)
    lse = np.full((total_q, Hq), np.nan)
    # args: q k v ks vs kd pt pts sl B Hq Hkv D P scale -> insert cu, B, total_q
    a = args[:9] + [_ptr(cu), B, total_q] + args[10:] + [_ptr(out), _ptr(lse)]
    if lib.oracle_paged_verify_attention(*a) != 0:
        raise ValueError("oracle_paged_verify_attention: invalid arguments")
    del keep
    return out, lse


def case_attention(case, page_table=None):
    """Oracle attention for a workloads.DecodeCase.  Uses the case's own page
    placement unless a page table is given."""
    pt = case.page_list if page_table is None else page_table
    return paged_attention(case.q, case.k_pages, case.v_pages, pt, case.seq_lens,
                           num_kv_heads=case.num_kv_heads, page_size=case.page_size,
                           scale=case.scale, kv_dtype=case.kv_dtype,
                           k_scales=case.k_scales, v_scales=case.v_scales)


def case_page_table(case, max_seq_pages=None, seqlen_offset=None):
    msp = case.max_seq_pages if max_seq_pages is None else max_seq_pages
    off = case.seqlen_offset if seqlen_offset is None else seqlen_offset
    return build_page_table(case.req_to_token, case.req_pool_indices, case.seq_lens,
                            case.page_size, msp, seqlen_offset=off)
