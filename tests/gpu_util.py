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


def walks_balanced(lens, page_size=64) -> bool:
    """The producers' rule for taking a split walk, as include/spa.h states
    it: the longest request has at most 6/5 of the mean number of pages.
    Tests use it to build batches on either side of the rule."""
    pages = (np.maximum(np.asarray(lens, dtype=np.int64), 0) + page_size - 1) // page_size
    return 5 * int(pages.max()) * len(pages) <= 6 * int(pages.sum())


def balanced_walk_lens(n, seed, hi=4096):
    """n lengths balanced enough for split walks, with the cases a walk must
    get right among them: an empty and a one-token request, exact page
    multiples and splits past the context inside a walk."""
    lens = W._gen(n, seed).integers(hi - 300, hi + 1, size=n)
    lens[:8] = [0, 1, 63, 64, 65, hi, hi - 1, 129]
    assert walks_balanced(lens)
    return lens


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
    tol = out_tolerance(o_ref)
    worst = float(np.max(err / tol)) if o.size else 0.0
    # strict: the error where the stated 1e-2 is reachable at all (|o| < 4)
    small = np.abs(o_ref) < STRICT_BELOW
    es = float(np.max(err[small])) if small.any() else 0.0
    print(f"[parity] {label}: max|out-oracle|={eo:.3e} (|o|<4: {es:.3e}; max err/tol "
          f"{worst:.3f}) max|lse-oracle|={el:.3e}", flush=True)
    assert np.all(err <= tol), f"{label}: out error {eo}, err/tol {worst}"
    assert el <= LSE_ATOL, f"{label}: lse error {el}"
    return eo, el


# Per-element gate on a bf16 output against the exact value o.  Below
# |o| = 4 it is the stated 1e-2: there half a bf16 step is at most 2^-7 =
# 0.0078, so a correctly rounded output can meet it.  From |o| = 4 on half a
# step is 2^-6 = 0.0156 and no bf16 value need lie within 1e-2; there the
# kernel's own bound applies: it forms o' in fp32 and rounds it once, so
# |bf16(o') - o| <= half a bf16 step at |o'| plus |o' - o|, the pre-rounding
# slack s = 1e-3 (fp32 accumulation) + 2^-11 |o| (the probabilities of P.V
# are rounded to f16 for 1-byte KV).
PRE_ROUND_ABS = 1e-3
PRE_ROUND_REL = 2.0 ** -11
STRICT_BELOW = 4.0


def out_tolerance(o_ref):
    ao = np.abs(np.asarray(o_ref, dtype=np.float64))
    s = PRE_ROUND_ABS + PRE_ROUND_REL * ao
    return np.where(ao < STRICT_BELOW, OUT_ATOL,
                    np.maximum(OUT_ATOL, 0.5 * bf16_ulp(ao + s) + s))


def bf16_ulp(x):
    """Spacing of bf16 values at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


# The counter region of a decode / multi-token workspace (C ABI layout: a
# fixed 64 KiB of int32 counters first, then the partial state).
COUNTER_REGION_BYTES = 65536


def counters_view(ws: torch.Tensor) -> torch.Tensor:
    """The whole arrival-counter region of a workspace, as int32."""
    return ws[:COUNTER_REGION_BYTES].view(torch.int32)
