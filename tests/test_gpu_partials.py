"""GPU parity of the producer pass on its own (spa_paged_decode_partials):
its per-split states against the oracle's split-K reference, and producer +
spa_split_merge against the one-call decode, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import split_paged_attention_amd as spa
import workloads as W
from tests.gpu_util import LSE_ATOL, OUT_ATOL, DevCase, balanced_walk_lens, config_case

pytestmark = pytest.mark.gpu

PRODUCERS = ["page_split", "head_grouped"]


def small_case(lens, kv="bf16", S=4, seed=31):
    P = 64
    need = sum(-(-L // P) for L in lens)
    msp = max(1, max(-(-L // P) for L in lens))
    return W.make_case(seed=seed, seq_lens=lens, num_pages=need + 3, num_splits=S, kv_dtype=kv,
                       num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=P,
                       req_pool_rows=max(4, len(lens)), req_to_token_stride=msp * P,
                       max_seq_pages=msp, name=f"partials{lens}_{kv}_S{S}")


def partials(d, S=None, producer=None):
    c = d.case
    return spa.paged_decode_partials(d.q, d.k, d.v, d.page_list, d.seq_lens,
                                     c.num_splits if S is None else S, float(c.scale),
                                     kv_dtype=c.kv_dtype, k_scales=d.ks, v_scales=d.vs,
                                     producer=producer)


@pytest.mark.parametrize("producer", PRODUCERS)
@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_split_states_match_oracle(kv, producer):
    """Every split's state, compared as the split's own softmax output
    acc_j / l_j (within the output tolerance) and its log-sum-exp
    m_j + ln l_j (within the LSE tolerance); empty splits are exactly
    (-inf, 0, 0).  Lengths cover one token, exact page multiples, a ragged
    tail and splits past the context."""
    S = 5
    c = small_case([1, 64, 65, 700, 2000, 0], kv=kv, S=S)
    print(f"[case] split states {kv} {producer}", flush=True)
    d = DevCase(c)
    acc, m, l = partials(d, producer=producer)
    torch.cuda.synchronize()
    acc, m, l = acc.cpu().numpy(), m.cpu().numpy(), l.cpu().numpy()
    acc_r, m_r, l_r = oracle.split_partials(c.q, c.k_pages, c.v_pages, c.page_list, c.seq_lens,
                                            num_kv_heads=8, page_size=64, scale=c.scale,
                                            num_splits=S, kv_dtype=kv, k_scales=c.k_scales,
                                            v_scales=c.v_scales)
    empty = np.isneginf(m_r)
    assert np.array_equal(np.isneginf(m), empty), "empty splits differ"
    assert np.all(l[empty] == 0) and np.all(acc[empty] == 0)
    full = ~empty
    assert full.sum() > 0 and empty.sum() > 0
    o = acc[full] / l[full][:, None]
    o_r = acc_r[full] / l_r[full][:, None]
    lse = m[full].astype(np.float64) + np.log(l[full].astype(np.float64))
    lse_r = m_r[full] + np.log(l_r[full])
    eo, el = float(np.max(np.abs(o - o_r))), float(np.max(np.abs(lse - lse_r)))
    print(f"[parity] split states {kv} {producer}: max|o_j-oracle|={eo:.3e} "
          f"max|lse_j-oracle|={el:.3e}", flush=True)
    assert eo <= OUT_ATOL and el <= LSE_ATOL
    # the running max is a max of computed scores, not a shifted value
    assert np.max(np.abs(m[full] - m_r[full])) <= LSE_ATOL


@pytest.mark.parametrize("producer", PRODUCERS + [None])
@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_partials_then_merge_equal_one_call(kv, producer):
    c = small_case([3000, 17, 640, 1], kv=kv, S=7)
    print(f"[case] partials + merge vs one call {kv} {producer}", flush=True)
    d = DevCase(c)
    acc, m, l = partials(d, producer=producer)
    o1, l1 = spa.split_merge(acc, m, l)
    o2, l2 = d.attention(producer=producer, merge="separate")
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_partials_split_walk_bit_identical():
    """A bf16 head-grouped grid large enough for walks of several splits per
    workgroup (64 requests balanced enough to walk, 16 splits)."""
    lens = balanced_walk_lens(64, 65)
    c = small_case(lens.tolist(), kv="bf16", S=16, seed=66)
    assert spa.decode_default_flags(64, 8, 16, "bf16", c.max_seq_pages) == (
        spa.SPA_DECODE_HEAD_GROUPED | spa.SPA_DECODE_SEPARATE_MERGE)
    print("[case] partials split walk batch 64 S=16", flush=True)
    d = DevCase(c)
    o1, l1 = spa.split_merge(*partials(d))
    o2, l2 = d.attention()
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("cfg", [4, 5, 6])
def test_headline_partials_then_merge_equal_default_call(cfg):
    """The full batch-32 workloads (8K bf16; ragged int8; 8K fp8), in the launch
    configuration the benchmark times: producer entry point, then the merge
    entry point, against the default one-call decode."""
    c = config_case(cfg)
    print(f"[case] partials + merge at {c.name}", flush=True)
    d = DevCase(c)
    pt, _, _ = d.page_table()
    flags = spa.decode_default_flags(c.batch, c.num_kv_heads, c.num_splits, c.kv_dtype,
                                     pt.shape[1])
    assert flags & spa.SPA_DECODE_SEPARATE_MERGE
    acc, m, l = spa.paged_decode_partials(d.q, d.k, d.v, pt, d.seq_lens, c.num_splits,
                                          float(c.scale), kv_dtype=c.kv_dtype, k_scales=d.ks,
                                          v_scales=d.vs)
    o1, l1 = spa.split_merge(acc, m, l)
    o2, l2 = d.attention(page_table=pt)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_partials_leave_other_buffers_alone():
    """The producer writes exactly its [B, Hq, S, D] / [B, Hq, S] regions:
    guard words around each buffer keep their NaN poison."""
    c = small_case([900, 5], S=3)
    print("[case] partials write bounds", flush=True)
    d = DevCase(c)
    B, Hq, S, D = 2, 32, 3, 128
    pad = 64
    big_acc = torch.full((B * Hq * S * D + 2 * pad,), float("nan"), device="cuda")
    big_m = torch.full((B * Hq * S + 2 * pad,), float("nan"), device="cuda")
    big_l = torch.full((B * Hq * S + 2 * pad,), float("nan"), device="cuda")
    acc = big_acc[pad:pad + B * Hq * S * D].view(B, Hq, S, D)
    m = big_m[pad:pad + B * Hq * S].view(B, Hq, S)
    l = big_l[pad:pad + B * Hq * S].view(B, Hq, S)
    spa.paged_decode_partials(d.q, d.k, d.v, d.page_list, d.seq_lens, S, float(c.scale),
                              partial_acc=acc, partial_max=m, partial_sum=l)
    torch.cuda.synchronize()
    for big, n in ((big_acc, B * Hq * S * D), (big_m, B * Hq * S), (big_l, B * Hq * S)):
        h = big.cpu().numpy()
        assert np.all(np.isnan(h[:pad])) and np.all(np.isnan(h[pad + n:]))
        assert not np.any(np.isnan(h[pad:pad + n]))
