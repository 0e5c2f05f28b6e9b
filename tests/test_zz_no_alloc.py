"""GPU test of the no-allocation decode entry point
(spa_paged_decode_attention_noalloc), through the C ABI: two calls in a
row on the library's per-GPU scratch array, the second with a smaller
batch, each equal bit for bit to spa_paged_decode_attention on a fresh
workspace and within tolerance of the oracle."""
import pytest
import torch

import oracle
import split_paged_attention_amd as spa
import workloads as W
from tests.gpu_util import DevCase, compare_attention

pytestmark = pytest.mark.gpu


def case(lens, kv, S, seed):
    P = 64
    need = sum(-(-L // P) for L in lens)
    msp = max(1, max(-(-L // P) for L in lens))
    return W.make_case(seed=seed, seq_lens=lens, num_pages=need + 3, num_splits=S, kv_dtype=kv,
                       num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=P,
                       req_pool_rows=max(4, len(lens)), req_to_token_stride=msp * P,
                       max_seq_pages=msp, name=f"noalloc{lens}_{kv}_S{S}")


def noalloc(d, **kw):
    c = d.case
    return spa.paged_decode_attention_noalloc(d.q, d.k, d.v, d.page_list, d.seq_lens,
                                              c.num_splits, float(c.scale), kv_dtype=c.kv_dtype,
                                              k_scales=d.ks, v_scales=d.vs, **kw)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("plan", [dict(), dict(merge="fused", producer="page_split"),
                                  dict(merge="separate", producer="head_grouped"),
                                  dict(merge="fused", producer="head_grouped")])
def test_noalloc_equals_workspace_call_on_two_calls_in_a_row(kv, plan):
    big = case([3000, 700, 65, 1, 2048, 4000, 9, 130, 64], kv, S=8, seed=61)
    small = case([900, 64, 3], kv, S=4, seed=62)
    for c in (big, small):
        print(f"[case] noalloc {kv} {plan} batch {c.batch}", flush=True)
        d = DevCase(c)
        o_ref, l_ref = d.attention(**plan)
        o, l = noalloc(d, **plan)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
        assert torch.equal(l, l_ref)
        oo, lo = oracle.case_attention(c)
        compare_attention(o, l, oo, lo, label=f"noalloc {kv} {plan} batch {c.batch}")


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    c = case([64] * 2, "bf16", S=4, seed=63)
    d = DevCase(c)
    q = torch.zeros((64, 32, 128), dtype=torch.bfloat16, device="cuda")
    pt = torch.zeros((64, 1), dtype=torch.int32, device="cuda")
    sl = torch.ones((64,), dtype=torch.int32, device="cuda")
    assert spa.decode_workspace_bytes(64, 32, 8, 128, 64) > (32 << 20)
    with pytest.raises(spa.SpaError, match="WORKSPACE_TOO_SMALL"):
        spa.paged_decode_attention_noalloc(q, d.k, d.v, pt, sl, 64, 0.088)
