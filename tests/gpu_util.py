"""Helpers for the GPU parity tests: move a seeded case to the device, run
the HIP path through the C ABI, and compare with the oracle."""
import functools

import numpy as np
import torch

import split_paged_attention_amd as spa
import workloads as W

# Tolerances stated for this path: bf16 output within 1e-2 max-abs, per-row
# LSE within 1e-3, page-table / cu_seqlens build bit-exact.
OUT_ATOL = 1e-2
LSE_ATOL = 1e-3


@functools.lru_cache(maxsize=None)
def config_case(cfg: int):
    return W.make_config(cfg)


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def bits_host(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return W.bf16_bits_to_f32(bits_host(t)).astype(np.float64)


class DevCase:
    """Device copies of a DecodeCase."""

    def __init__(self, case):
        self.case = case
        self.q = bf16_dev(case.q)
        if case.kv_dtype == "bf16":
            self.k = bf16_dev(case.k_pages)
            self.v = bf16_dev(case.v_pages)
            self.ks = self.vs = None
        else:
            self.k = torch.from_numpy(case.k_pages).cuda()
            self.v = torch.from_numpy(case.v_pages).cuda()
            self.ks = torch.from_numpy(case.k_scales).cuda()
            self.vs = torch.from_numpy(case.v_scales).cuda()
        self.r2t = torch.from_numpy(case.req_to_token).cuda()
        self.rpi = torch.from_numpy(case.req_pool_indices).cuda()
        self.seq_lens = torch.from_numpy(case.seq_lens).cuda()
        self.page_list = torch.from_numpy(case.page_list).cuda()

    def page_table(self, max_seq_pages=None):
        msp = self.case.max_seq_pages if max_seq_pages is None else max_seq_pages
        return spa.build_page_table(self.r2t, self.rpi, self.seq_lens, self.case.page_size, msp,
                                    seqlen_offset=self.case.seqlen_offset)

    def attention(self, page_table=None, num_splits=None, **kw):
        c = self.case
        pt = self.page_list if page_table is None else page_table
        S = c.num_splits if num_splits is None else num_splits
        return spa.paged_decode_attention(self.q, self.k, self.v, pt, self.seq_lens, S,
                                          float(c.scale), kv_dtype=c.kv_dtype,
                                          k_scales=self.ks, v_scales=self.vs, **kw)


def compare_attention(out_dev, lse_dev, o_ref, l_ref, rows=None, label=""):
    """Max-abs errors of the bf16 output and fp32 LSE against fp64 oracle
    values; asserts the stated tolerances.  ``rows`` restricts to a subset
    of batch rows (the oracle values then cover only those rows)."""
    torch.cuda.synchronize()
    o = bf16_to_f64(out_dev)
    l = lse_dev.cpu().numpy().astype(np.float64)
    if rows is not None:
        o, l = o[rows], l[rows]
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(l), fin), f"{label}: LSE finiteness differs"
    assert np.all(l[~fin] == l_ref[~fin]), f"{label}: -inf LSE rows differ"
    err = np.abs(o - o_ref)
    eo = float(np.max(err)) if o.size else 0.0
    el = float(np.max(np.abs(l[fin] - l_ref[fin]))) if fin.any() else 0.0
    # The bound cannot be finer than the bf16 output's own spacing: where one
    # bf16 ulp of the exact value exceeds OUT_ATOL (|o| >= 2), one ulp is allowed.
    tol = np.maximum(OUT_ATOL, bf16_ulp(o_ref))
    worst = float(np.max(err / tol)) if o.size else 0.0
    print(f"[parity] {label}: max|out-oracle|={eo:.3e} (max err/tol {worst:.3f}) "
          f"max|lse-oracle|={el:.3e}", flush=True)
    assert np.all(err <= tol), f"{label}: out error {eo}, err/tol {worst}"
    assert el <= LSE_ATOL, f"{label}: lse error {el}"
    return eo, el


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def counters_view(ws: torch.Tensor, batch, hq, hkv, d, splits) -> torch.Tensor:
    """The arrival-counter region of a decode workspace (layout of the C ABI:
    acc | max | sum | counters, each 256-byte aligned)."""
    def a256(x):
        return (x + 255) & ~255
    rows = batch * hq * splits
    acc = rows * d * 4
    mo = a256(acc)
    so = a256(mo + rows * 4)
    co = a256(so + rows * 4)
    return ws[co:co + batch * hkv * 4].view(torch.int32)
