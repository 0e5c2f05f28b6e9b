"""split_paged_attention_amd -- split-K paged-attention decode for MI355X.

Thin ctypes binding over libspa.so (declared in include/spa.h).  This module
only marshals arguments: it checks tensor dtypes/devices, allocates outputs
with PyTorch when the caller does not pass them, and hands raw device
pointers and the current HIP stream to the library.  Every step of the
computation runs in the library's HIP kernels.  If libspa.so is missing the
import succeeds but every call raises: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "SpaError", "lib", "status_string", "build_page_table", "decode_workspace_bytes",
    "workspace_reset", "new_workspace", "paged_decode_attention", "split_merge",
    "paged_decode_attention_noalloc",
    "SPA_OK", "SPA_ERR_INVALID_ARGUMENT", "SPA_ERR_UNSUPPORTED",
    "SPA_ERR_WORKSPACE_TOO_SMALL", "SPA_ERR_HIP", "SPA_KV_BF16", "SPA_KV_INT8", "SPA_KV_FP8",
    "SPA_DECODE_SEPARATE_MERGE", "SPA_DECODE_FUSED_MERGE", "SPA_DECODE_HEAD_GROUPED",
    "SPA_DECODE_PAGE_SPLIT",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspa.so")

SPA_OK = 0
SPA_ERR_INVALID_ARGUMENT = 1
SPA_ERR_UNSUPPORTED = 2
SPA_ERR_WORKSPACE_TOO_SMALL = 3
SPA_ERR_HIP = 4
SPA_KV_BF16 = 0
SPA_KV_INT8 = 1
SPA_KV_FP8 = 2
SPA_DECODE_SEPARATE_MERGE = 0x1
SPA_DECODE_FUSED_MERGE = 0x2
SPA_DECODE_HEAD_GROUPED = 0x4
SPA_DECODE_PAGE_SPLIT = 0x8

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U32 = ctypes.c_uint32
_SZ = ctypes.c_size_t
_F32 = ctypes.c_float
_ST = ctypes.c_int

_lib = None


class SpaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = status_string(status) if _lib is not None else str(status)
        extra = ""
        if status == SPA_ERR_HIP and _lib is not None:
            extra = f" (hipError_t {_lib.spa_last_hip_error()})"
        super().__init__(f"{where}: {name}{extra}")


def lib():
    """The loaded libspa.so (ctypes.CDLL); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                           "(python split_paged_attention_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    L.spa_status_string.argtypes = [_ST]
    L.spa_status_string.restype = ctypes.c_char_p
    L.spa_last_hip_error.argtypes = []
    L.spa_last_hip_error.restype = ctypes.c_int
    L.spa_abi_version.argtypes = []
    L.spa_abi_version.restype = ctypes.c_int
    L.spa_build_page_table.argtypes = [_P, _I64, _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _I64,
                                       _P, _P, _P]
    L.spa_build_page_table.restype = _ST
    L.spa_build_metadata.argtypes = [_P, _I64, _I32, _P, _P, _I32, _I32, _I32, _I32, _P, _I64,
                                     _P, _P, _I32, _P, _I32, _P, _P, _I64, _P, _I64, _P, _I64,
                                     _P, _I64, _P]
    L.spa_build_metadata.restype = _ST
    L.spa_decode_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32]
    L.spa_decode_workspace_bytes.restype = _SZ
    L.spa_workspace_reset.argtypes = [_P, _SZ, _P]
    L.spa_workspace_reset.restype = _ST
    L.spa_paged_decode_attention.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _P, _I32, _I32, _I32,
                                             _I32, _I32, _I32, _I32, _F32, _ST, _U32, _P, _SZ,
                                             _P, _P, _P]
    L.spa_paged_decode_attention.restype = _ST
    L.spa_paged_decode_attention_noalloc.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _P, _I32,
                                                     _I32, _I32, _I32, _I32, _I32, _I32, _F32,
                                                     _ST, _U32, _P, _P, _P]
    L.spa_paged_decode_attention_noalloc.restype = _ST
    L.spa_decode_default_flags.argtypes = [_I32, _I32, _I32, _ST, _I64]
    L.spa_decode_default_flags.restype = _U32
    L.spa_paged_decode_partials.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _P, _I32, _I32, _I32,
                                            _I32, _I32, _I32, _I32, _F32, _ST, _U32, _P, _P, _P,
                                            _P]
    L.spa_paged_decode_partials.restype = _ST
    L.spa_verify_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32]
    L.spa_verify_workspace_bytes.restype = _SZ
    L.spa_paged_verify_attention.argtypes = [_P, _P, _P, _P, _P, _P, _I64, _P, _P, _I32, _I32,
                                             _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                                             ctypes.c_float, _I32, _P, _SZ, _P, _P, _P]
    L.spa_paged_verify_attention.restype = _ST
    L.spa_split_merge.argtypes = [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P]
    L.spa_split_merge.restype = _ST
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().spa_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != SPA_OK:
        raise SpaError(status, where)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _need(t: torch.Tensor, name: str, dtype, contiguous: bool = True) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------- metadata

def build_page_table(req_to_token: torch.Tensor, req_pool_indices: torch.Tensor,
                     seq_lens: torch.Tensor, page_size: int, max_seq_pages: int, *,
                     seqlen_offset: int = 0, page_table: Optional[torch.Tensor] = None,
                     cache_seqlens: Optional[torch.Tensor] = None,
                     cu_seqlens_k: Optional[torch.Tensor] = None,
                     stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """spa_build_page_table: (page_table [bs, stride], cache_seqlens [bs], cu_seqlens_k [bs+1])."""
    _need(req_to_token, "req_to_token", torch.int32, contiguous=False)
    if req_to_token.dim() != 2 or req_to_token.stride(1) != 1:
        raise ValueError("req_to_token must be 2-D with unit column stride")
    _need(req_pool_indices, "req_pool_indices", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    bs = int(req_pool_indices.shape[0])
    dev = req_to_token.device
    if page_table is None:
        page_table = torch.empty((bs, max(1, max_seq_pages)), dtype=torch.int32, device=dev)
    _need(page_table, "page_table", torch.int32, contiguous=False)
    if page_table.dim() != 2 or page_table.stride(1) != 1:
        raise ValueError("page_table must be 2-D with unit column stride")
    if cache_seqlens is None:
        cache_seqlens = torch.empty((bs,), dtype=torch.int32, device=dev)
    if cu_seqlens_k is None:
        cu_seqlens_k = torch.empty((bs + 1,), dtype=torch.int32, device=dev)
    _need(cache_seqlens, "cache_seqlens", torch.int32)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    st = lib().spa_build_page_table(
        _ptr(req_to_token), req_to_token.stride(0), req_to_token.shape[0],
        _ptr(req_pool_indices), _ptr(seq_lens), bs, int(seqlen_offset), int(page_size),
        int(max_seq_pages), _ptr(page_table), page_table.stride(0), _ptr(cache_seqlens),
        _ptr(cu_seqlens_k), _stream(stream))
    _check(st, "spa_build_page_table")
    return page_table, cache_seqlens, cu_seqlens_k


Q_MODE_NONE, Q_MODE_CUMSUM, Q_MODE_STRIDED = 0, 1, 2


def build_metadata(req_to_token: torch.Tensor, req_pool_indices: torch.Tensor,
                   seq_lens: torch.Tensor, page_size: int, max_seq_pages: int, *,
                   seqlen_offset: int = 0, page_table: Optional[torch.Tensor] = None,
                   cache_seqlens: Optional[torch.Tensor] = None,
                   cu_seqlens_k: Optional[torch.Tensor] = None, q_mode: int = Q_MODE_NONE,
                   qlens: Optional[torch.Tensor] = None, q_stride: int = 0,
                   cu_seqlens_q: Optional[torch.Tensor] = None,
                   full_to_swa: Optional[torch.Tensor] = None,
                   swa_page_table: Optional[torch.Tensor] = None,
                   out_cache_loc: Optional[torch.Tensor] = None,
                   swa_out_cache_loc: Optional[torch.Tensor] = None,
                   stream=None) -> dict:
    """spa_build_metadata.  Outputs not given are allocated (page_table,
    cache_seqlens, cu_seqlens_k always; cu_seqlens_q when q_mode is not NONE);
    swa_page_table and swa_out_cache_loc are produced only when passed in, as
    in the source.  Returns a dict of the output tensors."""
    _need(req_to_token, "req_to_token", torch.int32, contiguous=False)
    if req_to_token.dim() != 2 or req_to_token.stride(1) != 1:
        raise ValueError("req_to_token must be 2-D with unit column stride")
    _need(req_pool_indices, "req_pool_indices", torch.int32)
    _need(seq_lens, "seq_lens", torch.int32)
    bs = int(req_pool_indices.shape[0])
    dev = req_to_token.device

    def table(t, name):
        _need(t, name, torch.int32, contiguous=False)
        if t.dim() != 2 or t.stride(1) != 1:
            raise ValueError(f"{name} must be 2-D with unit column stride")

    if page_table is None:
        page_table = torch.empty((bs, max(1, max_seq_pages)), dtype=torch.int32, device=dev)
    table(page_table, "page_table")
    if cache_seqlens is None:
        cache_seqlens = torch.empty((bs,), dtype=torch.int32, device=dev)
    if cu_seqlens_k is None:
        cu_seqlens_k = torch.empty((bs + 1,), dtype=torch.int32, device=dev)
    _need(cache_seqlens, "cache_seqlens", torch.int32)
    _need(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    if q_mode != Q_MODE_NONE and cu_seqlens_q is None:
        cu_seqlens_q = torch.empty((bs + 1,), dtype=torch.int32, device=dev)
    for t, name, dt in ((qlens, "qlens", torch.int32), (cu_seqlens_q, "cu_seqlens_q", torch.int32),
                        (full_to_swa, "full_to_swa", torch.int64),
                        (out_cache_loc, "out_cache_loc", torch.int64),
                        (swa_out_cache_loc, "swa_out_cache_loc", torch.int64)):
        if t is not None:
            _need(t, name, dt)
    if swa_page_table is not None:
        table(swa_page_table, "swa_page_table")
    st = lib().spa_build_metadata(
        _ptr(req_to_token), req_to_token.stride(0), req_to_token.shape[0],
        _ptr(req_pool_indices), _ptr(seq_lens), bs, int(seqlen_offset), int(page_size),
        int(max_seq_pages), _ptr(page_table), page_table.stride(0), _ptr(cache_seqlens),
        _ptr(cu_seqlens_k), int(q_mode), _ptr(qlens), int(q_stride), _ptr(cu_seqlens_q),
        _ptr(full_to_swa), 0 if full_to_swa is None else full_to_swa.numel(),
        _ptr(swa_page_table),
        0 if swa_page_table is None else swa_page_table.stride(0), _ptr(out_cache_loc),
        0 if out_cache_loc is None else out_cache_loc.numel(), _ptr(swa_out_cache_loc),
        0 if swa_out_cache_loc is None else swa_out_cache_loc.numel(), _stream(stream))
    _check(st, "spa_build_metadata")
    return dict(page_table=page_table, cache_seqlens=cache_seqlens, cu_seqlens_k=cu_seqlens_k,
                cu_seqlens_q=cu_seqlens_q, swa_page_table=swa_page_table,
                swa_out_cache_loc=swa_out_cache_loc)


# ---------------------------------------------------------------- workspace

def decode_workspace_bytes(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           num_splits: int) -> int:
    return int(lib().spa_decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim,
                                                num_splits))


def workspace_reset(workspace: torch.Tensor, stream=None) -> None:
    _need(workspace, "workspace", torch.uint8)
    _check(lib().spa_workspace_reset(_ptr(workspace), workspace.numel(), _stream(stream)),
           "spa_workspace_reset")


def new_workspace(batch: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                  num_splits: int, device="cuda", stream=None) -> torch.Tensor:
    """A zeroed workspace of the size the decode call needs."""
    n = decode_workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, num_splits)
    if n == 0:
        raise ValueError("invalid sizes for a decode workspace")
    ws = torch.empty((n,), dtype=torch.uint8, device=device)
    workspace_reset(ws, stream=stream)
    return ws


# ---------------------------------------------------------------- attention

def _decode_inputs(q, k_pages, v_pages, page_table, seq_lens, kv_dtype, k_scales, v_scales):
    """Checks of the decode inputs; returns (B, Hq, D, num_pages, P, Hkv, kv enum,
    k_scales, v_scales)."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 3:
        raise ValueError("q must be [batch, num_q_heads, head_dim]")
    B, Hq, D = q.shape
    kvd = {"bf16": SPA_KV_BF16, "int8": SPA_KV_INT8, "fp8": SPA_KV_FP8}[kv_dtype]
    kv_t = {SPA_KV_BF16: torch.bfloat16, SPA_KV_INT8: torch.int8, SPA_KV_FP8: torch.uint8}[kvd]
    if kvd == SPA_KV_FP8 and k_pages.dtype == torch.float8_e4m3fn:
        kv_t = torch.float8_e4m3fn
    _need(k_pages, "k_pages", kv_t)
    _need(v_pages, "v_pages", kv_t)
    if k_pages.dim() != 4 or k_pages.shape != v_pages.shape:
        raise ValueError("k_pages/v_pages must be [num_pages, page_size, num_kv_heads, head_dim]")
    num_pages, P, Hkv, Dk = k_pages.shape
    if Dk != D:
        raise ValueError("head_dim of q and the KV pages differ")
    if kvd != SPA_KV_BF16:
        for nm, t in (("k_scales", k_scales), ("v_scales", v_scales)):
            if t is None:
                raise ValueError(f"{nm} is required for {kv_dtype} KV")
            _need(t, nm, torch.float32)
            if tuple(t.shape) != (num_pages, P, Hkv):
                raise ValueError(f"{nm} must be [num_pages, page_size, num_kv_heads]")
    else:
        k_scales = v_scales = None
    _need(page_table, "page_table", torch.int32, contiguous=False)
    if page_table.dim() != 2 or page_table.stride(1) != 1 or page_table.shape[0] != B:
        raise ValueError("page_table must be [batch, stride] with unit column stride")
    _need(seq_lens, "seq_lens", torch.int32)
    if seq_lens.shape != (B,):
        raise ValueError("seq_lens must be [batch]")
    return B, Hq, D, num_pages, P, Hkv, kvd, k_scales, v_scales


_PRODUCER_FLAGS = {None: 0, "head_grouped": SPA_DECODE_HEAD_GROUPED,
                   "page_split": SPA_DECODE_PAGE_SPLIT}


def paged_decode_attention(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                           page_table: torch.Tensor, seq_lens: torch.Tensor, num_splits: int,
                           scale: float, *, kv_dtype: str = "bf16",
                           k_scales: Optional[torch.Tensor] = None,
                           v_scales: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None,
                           separate_merge: bool = False,
                           merge: Optional[str] = None,
                           producer: Optional[str] = None,
                           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """spa_paged_decode_attention.  q [B, Hq, D] bf16; k/v_pages
    [num_pages, P, Hkv, D] bf16, int8, or e4m3 codes (uint8 or
    float8_e4m3fn) for kv_dtype "fp8"; k/v_scales [num_pages, P, Hkv] fp32
    for int8 and fp8; page_table [B, stride] int32; seq_lens [B] int32.
    Returns (out [B, Hq, D] bf16, lse [B, Hq] fp32).

    merge: None (library default), "fused" or "separate" (``separate_merge=True``
    is the same as "separate"); producer: None, "head_grouped" or "page_split"."""
    B, Hq, D, num_pages, P, Hkv, kvd, k_scales, v_scales = _decode_inputs(
        q, k_pages, v_pages, page_table, seq_lens, kv_dtype, k_scales, v_scales)
    if workspace is None:
        workspace = new_workspace(B, Hq, Hkv, D, num_splits, device=q.device, stream=stream)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16)
    _need(lse, "lse", torch.float32)
    if separate_merge:
        if merge not in (None, "separate"):
            raise ValueError("separate_merge=True contradicts merge=" + repr(merge))
        merge = "separate"
    flags = {None: 0, "fused": SPA_DECODE_FUSED_MERGE, "separate": SPA_DECODE_SEPARATE_MERGE}[merge]
    flags |= _PRODUCER_FLAGS[producer]
    st = lib().spa_paged_decode_attention(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scales), _ptr(v_scales), _ptr(page_table),
        page_table.stride(0), _ptr(seq_lens), B, Hq, Hkv, D, P, num_pages, int(num_splits),
        float(scale), kvd, flags, _ptr(workspace), workspace.numel(), _ptr(out), _ptr(lse),
        _stream(stream))
    _check(st, "spa_paged_decode_attention")
    return out, lse


def paged_decode_attention_noalloc(q: torch.Tensor, k_pages: torch.Tensor,
                                   v_pages: torch.Tensor, page_table: torch.Tensor,
                                   seq_lens: torch.Tensor, num_splits: int, scale: float, *,
                                   kv_dtype: str = "bf16", k_scales: Optional[torch.Tensor] = None,
                                   v_scales: Optional[torch.Tensor] = None,
                                   out: Optional[torch.Tensor] = None,
                                   lse: Optional[torch.Tensor] = None,
                                   merge: Optional[str] = None, producer: Optional[str] = None,
                                   stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """spa_paged_decode_attention_noalloc: paged_decode_attention on the
    library's own per-GPU workspace (no workspace argument; the library
    allocates nothing).  Pass ``out`` and ``lse`` to keep the call free of
    allocations on the Python side too."""
    B, Hq, D, num_pages, P, Hkv, kvd, k_scales, v_scales = _decode_inputs(
        q, k_pages, v_pages, page_table, seq_lens, kv_dtype, k_scales, v_scales)
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16)
    _need(lse, "lse", torch.float32)
    flags = {None: 0, "fused": SPA_DECODE_FUSED_MERGE, "separate": SPA_DECODE_SEPARATE_MERGE}[merge]
    flags |= _PRODUCER_FLAGS[producer]
    st = lib().spa_paged_decode_attention_noalloc(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scales), _ptr(v_scales), _ptr(page_table),
        page_table.stride(0), _ptr(seq_lens), B, Hq, Hkv, D, P, num_pages, int(num_splits),
        float(scale), kvd, flags, _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "spa_paged_decode_attention_noalloc")
    return out, lse


def decode_default_flags(batch: int, num_kv_heads: int, num_splits: int, kv_dtype: str,
                         page_table_stride: int) -> int:
    """spa_decode_default_flags: the producer | merge flags of the plan
    paged_decode_attention takes by default (0 for rejected sizes)."""
    kvd = {"bf16": SPA_KV_BF16, "int8": SPA_KV_INT8, "fp8": SPA_KV_FP8}[kv_dtype]
    return int(lib().spa_decode_default_flags(batch, num_kv_heads, num_splits, kvd,
                                              page_table_stride))


def paged_decode_partials(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                          page_table: torch.Tensor, seq_lens: torch.Tensor, num_splits: int,
                          scale: float, *, kv_dtype: str = "bf16",
                          k_scales: Optional[torch.Tensor] = None,
                          v_scales: Optional[torch.Tensor] = None,
                          partial_acc: Optional[torch.Tensor] = None,
                          partial_max: Optional[torch.Tensor] = None,
                          partial_sum: Optional[torch.Tensor] = None,
                          producer: Optional[str] = None,
                          stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """spa_paged_decode_partials: the producer pass alone.  Inputs as in
    paged_decode_attention; returns (partial_acc [B, Hq, S, D], partial_max
    [B, Hq, S], partial_sum [B, Hq, S]), fp32, the layout split_merge reads."""
    B, Hq, D, num_pages, P, Hkv, kvd, k_scales, v_scales = _decode_inputs(
        q, k_pages, v_pages, page_table, seq_lens, kv_dtype, k_scales, v_scales)
    S = int(num_splits)
    if partial_acc is None:
        partial_acc = torch.empty((B, Hq, S, D), dtype=torch.float32, device=q.device)
    if partial_max is None:
        partial_max = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    if partial_sum is None:
        partial_sum = torch.empty((B, Hq, S), dtype=torch.float32, device=q.device)
    _need(partial_acc, "partial_acc", torch.float32)
    _need(partial_max, "partial_max", torch.float32)
    _need(partial_sum, "partial_sum", torch.float32)
    if (tuple(partial_acc.shape) != (B, Hq, S, D) or tuple(partial_max.shape) != (B, Hq, S)
            or tuple(partial_sum.shape) != (B, Hq, S)):
        raise ValueError("partial_acc must be [batch, num_q_heads, num_splits, head_dim] and "
                         "partial_max/partial_sum [batch, num_q_heads, num_splits]")
    st = lib().spa_paged_decode_partials(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scales), _ptr(v_scales), _ptr(page_table),
        page_table.stride(0), _ptr(seq_lens), B, Hq, Hkv, D, P, num_pages, S, float(scale), kvd,
        _PRODUCER_FLAGS[producer], _ptr(partial_acc), _ptr(partial_max), _ptr(partial_sum),
        _stream(stream))
    _check(st, "spa_paged_decode_partials")
    return partial_acc, partial_max, partial_sum


def verify_workspace_bytes(total_q: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           num_splits: int) -> int:
    return int(lib().spa_verify_workspace_bytes(total_q, num_q_heads, num_kv_heads, head_dim,
                                                num_splits))


def paged_verify_attention(q: torch.Tensor, k_pages: torch.Tensor, v_pages: torch.Tensor,
                           page_table: torch.Tensor, seq_lens: torch.Tensor,
                           cu_seqlens_q: torch.Tensor, num_splits: int, scale: float, *,
                           max_q_len: int = 4, kv_dtype: str = "bf16",
                           k_scales: Optional[torch.Tensor] = None,
                           v_scales: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None,
                           out: Optional[torch.Tensor] = None,
                           lse: Optional[torch.Tensor] = None,
                           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """spa_paged_verify_attention (multi-token decode).  q [total_q, Hq, D]
    bf16; cu_seqlens_q [batch + 1] int32 (request b's query rows
    cu[b] .. cu[b+1]-1, at most max_q_len <= 64 of them); the rest as in
    paged_decode_attention.  Returns (out [total_q, Hq, D] bf16,
    lse [total_q, Hq] fp32)."""
    _need(q, "q", torch.bfloat16)
    if q.dim() != 3:
        raise ValueError("q must be [total_q, num_q_heads, head_dim]")
    T, Hq, D = q.shape
    kvd = {"bf16": SPA_KV_BF16, "int8": SPA_KV_INT8, "fp8": SPA_KV_FP8}[kv_dtype]
    kv_t = {SPA_KV_BF16: torch.bfloat16, SPA_KV_INT8: torch.int8, SPA_KV_FP8: torch.uint8}[kvd]
    if kvd == SPA_KV_FP8 and k_pages.dtype == torch.float8_e4m3fn:
        kv_t = torch.float8_e4m3fn
    _need(k_pages, "k_pages", kv_t)
    _need(v_pages, "v_pages", kv_t)
    if k_pages.dim() != 4 or k_pages.shape != v_pages.shape:
        raise ValueError("k_pages/v_pages must be [num_pages, page_size, num_kv_heads, head_dim]")
    num_pages, P, Hkv, Dk = k_pages.shape
    if Dk != D:
        raise ValueError("head_dim of q and the KV pages differ")
    if kvd != SPA_KV_BF16:
        for nm, t in (("k_scales", k_scales), ("v_scales", v_scales)):
            if t is None:
                raise ValueError(f"{nm} is required for {kv_dtype} KV")
            _need(t, nm, torch.float32)
            if tuple(t.shape) != (num_pages, P, Hkv):
                raise ValueError(f"{nm} must be [num_pages, page_size, num_kv_heads]")
    else:
        k_scales = v_scales = None
    _need(seq_lens, "seq_lens", torch.int32)
    B = int(seq_lens.shape[0])
    _need(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    if cu_seqlens_q.shape != (B + 1,):
        raise ValueError("cu_seqlens_q must be [batch + 1]")
    _need(page_table, "page_table", torch.int32, contiguous=False)
    if page_table.dim() != 2 or page_table.stride(1) != 1 or page_table.shape[0] != B:
        raise ValueError("page_table must be [batch, stride] with unit column stride")
    if workspace is None:
        n = verify_workspace_bytes(T, Hq, Hkv, D, num_splits)
        if n == 0:
            raise ValueError("invalid sizes for a multi-token decode workspace")
        workspace = torch.empty((n,), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.bfloat16)
    _need(lse, "lse", torch.float32)
    st = lib().spa_paged_verify_attention(
        _ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(k_scales), _ptr(v_scales), _ptr(page_table),
        page_table.stride(0), _ptr(seq_lens), _ptr(cu_seqlens_q), B, T, int(max_q_len), Hq, Hkv,
        D, P, num_pages, int(num_splits), float(scale), kvd, _ptr(workspace), workspace.numel(),
        _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "spa_paged_verify_attention")
    return out, lse


def split_merge(partial_acc: torch.Tensor, partial_max: torch.Tensor, partial_sum: torch.Tensor,
                *, out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """spa_split_merge: partial_acc [B, Hq, S, D], partial_max/sum [B, Hq, S] fp32."""
    _need(partial_acc, "partial_acc", torch.float32)
    _need(partial_max, "partial_max", torch.float32)
    _need(partial_sum, "partial_sum", torch.float32)
    if partial_acc.dim() != 4:
        raise ValueError("partial_acc must be [batch, num_q_heads, num_splits, head_dim]")
    B, Hq, S, D = partial_acc.shape
    if partial_max.shape != (B, Hq, S) or partial_sum.shape != (B, Hq, S):
        raise ValueError("partial_max/partial_sum must be [batch, num_q_heads, num_splits]")
    if out is None:
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=partial_acc.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=partial_acc.device)
    _need(out, "out", torch.bfloat16)
    _need(lse, "lse", torch.float32)
    st = lib().spa_split_merge(_ptr(partial_acc), _ptr(partial_max), _ptr(partial_sum), B, Hq, D,
                               S, _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "spa_split_merge")
    return out, lse
