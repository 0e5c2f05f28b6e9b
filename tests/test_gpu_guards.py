"""GPU checks of the decode kernels' guards on device data that breaks the
contract: a page id outside [0, num_pages) is read as a page of zeros
(keys, values and scales), and a length outside [0, page_table_stride *
page_size] is clamped into it.  The oracle sees the same data made valid: a
pool with one extra all-zero page that the bad ids point to, and the
clamped lengths.  The guards never touch memory outside the buffers: page
ids are read only below the (clamped) length's page count, and a bad id's
loads go through a zero-range buffer descriptor."""
import numpy as np
import pytest
import torch

import oracle
import split_paged_attention_amd as spa
import workloads as W
from tests.gpu_util import DevCase, compare_attention

pytestmark = pytest.mark.gpu

PRODUCERS = ["page_split", "head_grouped"]


def guarded_case(kv):
    lens = [700, 64, 1500, 9]
    P = 64
    need = sum(-(-L // P) for L in lens)
    msp = max(-(-L // P) for L in lens)
    return W.make_case(seed=77, seq_lens=lens, num_pages=need + 3, num_splits=4, kv_dtype=kv,
                       num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=P,
                       req_pool_rows=4, req_to_token_stride=msp * P, max_seq_pages=msp,
                       name=f"guards_{kv}")


def with_zero_page(a):
    """The pool with one all-zero page appended (index = old num_pages)."""
    return np.concatenate([a, np.zeros((1,) + a.shape[1:], dtype=a.dtype)], axis=0)


@pytest.mark.parametrize("producer", PRODUCERS)
@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_bad_page_ids_read_as_zero_pages(kv, producer):
    c = guarded_case(kv)
    print(f"[case] bad page ids {kv} {producer}", flush=True)
    npg = c.num_pages
    pt = c.page_list.copy()
    bad = [(0, 2, -3), (2, 5, npg), (2, 10, 2**31 - 1), (3, 0, -(2**31))]
    for b, i, v in bad:
        assert i < -(-int(c.seq_lens[b]) // c.page_size)   # a page the request uses
        pt[b, i] = v
    pt_ref = pt.copy()
    for b, i, v in bad:
        pt_ref[b, i] = npg
    o_ref, l_ref = oracle.paged_attention(
        c.q, with_zero_page(c.k_pages), with_zero_page(c.v_pages), pt_ref, c.seq_lens,
        num_kv_heads=8, page_size=64, scale=c.scale, kv_dtype=kv,
        k_scales=None if kv == "bf16" else with_zero_page(c.k_scales),
        v_scales=None if kv == "bf16" else with_zero_page(c.v_scales))
    d = DevCase(c)
    out, lse = d.attention(page_table=torch.from_numpy(pt).cuda(), producer=producer)
    compare_attention(out, lse, o_ref, l_ref, label=f"bad ids {kv} {producer}")


@pytest.mark.parametrize("producer", PRODUCERS)
@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_lengths_clamped_to_the_page_table(kv, producer):
    c = guarded_case(kv)
    print(f"[case] clamped lengths {kv} {producer}", flush=True)
    width = c.page_list.shape[1] * c.page_size
    sl = c.seq_lens.copy()
    sl[0] = width + 100          # past the row: clamped to the row
    sl[1] = -7                   # negative: clamped to 0 (out = 0, lse = -inf)
    sl_ref = np.clip(sl, 0, width).astype(np.int32)
    # request 0 now reads its whole row: give the row's tail valid pages
    pt = c.page_list.copy()
    n0 = -(-int(c.seq_lens[0]) // c.page_size)
    pt[0, n0:] = np.arange(pt.shape[1] - n0, dtype=np.int32) % c.num_pages
    assert pt[0].min() >= 0
    o_ref, l_ref = oracle.paged_attention(
        c.q, c.k_pages, c.v_pages, pt, sl_ref, num_kv_heads=8, page_size=64,
        scale=c.scale, kv_dtype=kv, k_scales=c.k_scales, v_scales=c.v_scales)
    d = DevCase(c)
    out, lse = spa.paged_decode_attention(d.q, d.k, d.v, torch.from_numpy(pt).cuda(),
                                          torch.from_numpy(sl).cuda(), c.num_splits,
                                          float(c.scale), kv_dtype=kv, k_scales=d.ks,
                                          v_scales=d.vs, producer=producer)
    compare_attention(out, lse, o_ref, l_ref, label=f"clamped lengths {kv} {producer}")
    assert np.isneginf(lse.cpu().numpy()[1]).all()
    assert not torch.any(out[1].float() != 0)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_multi_token_bad_page_ids_read_as_zero_pages(kv):
    """The same guard in the multi-token decode kernel (up to 4 query rows
    per request, causal among them)."""
    c = guarded_case(kv)
    print(f"[case] multi-token bad page ids {kv}", flush=True)
    npg = c.num_pages
    pt = c.page_list.copy()
    bad = [(0, 2, -3), (2, 5, npg), (2, 23, 2**31 - 1), (3, 0, -(2**31))]
    for b, i, v in bad:
        assert i < -(-int(c.seq_lens[b]) // c.page_size)
        pt[b, i] = v
    pt_ref = pt.copy()
    for b, i, v in bad:
        pt_ref[b, i] = npg
    q_rows, cu = W.verify_queries(c, [4, 1, 3, 2])
    o_ref, l_ref = oracle.verify_attention(
        q_rows, with_zero_page(c.k_pages), with_zero_page(c.v_pages), pt_ref, c.seq_lens, cu,
        num_kv_heads=8, page_size=64, scale=c.scale, kv_dtype=kv,
        k_scales=None if kv == "bf16" else with_zero_page(c.k_scales),
        v_scales=None if kv == "bf16" else with_zero_page(c.v_scales))
    d = DevCase(c)
    qd = torch.from_numpy(np.ascontiguousarray(q_rows).view(np.int16)).cuda().view(torch.bfloat16)
    out, lse = spa.paged_verify_attention(qd, d.k, d.v, torch.from_numpy(pt).cuda(), d.seq_lens,
                                          torch.from_numpy(cu).cuda(), c.num_splits,
                                          float(c.scale), max_q_len=4, kv_dtype=kv,
                                          k_scales=d.ks, v_scales=d.vs)
    compare_attention(out, lse, o_ref, l_ref, label=f"multi-token bad ids {kv}")
