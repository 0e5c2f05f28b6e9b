"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: hand-worked
closed forms (tests/golden), a dense numpy/scipy brute force that never uses
a page table, exact special cases, and invariances the mathematics fixes
(split count, physical page placement, key order, GQA grouping)."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as W
from tests.brute import dense_attention, dense_verify, e4m3_codes_to_f64

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x):
    return W.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def _ev(expr):
    return eval(expr, {"e": math.e, "log": math.log, "__builtins__": {}})


# ---------------------------------------------------------------- metadata

def test_metadata_golden_hand_example():
    g = json.load(open(os.path.join(GOLDEN, "metadata_tiny.json")))
    pt = np.array(g["page_table_preset"], dtype=np.int32)
    pt, cache, cu = oracle.build_page_table(
        np.array(g["req_to_token"], np.int32), np.array(g["req_pool_indices"], np.int32),
        np.array(g["seq_lens"], np.int32), g["page_size"], g["max_seq_pages"],
        seqlen_offset=g["seqlen_offset"], page_table=pt)
    assert pt.tolist() == g["expect_page_table"]
    assert cache.tolist() == g["expect_cache_seqlens"]
    assert cu.tolist() == g["expect_cu_seqlens_k"]


def test_metadata_bs0_is_noop():
    pt, cache, cu = oracle.build_page_table(np.zeros((1, 8), np.int32), np.zeros(0, np.int32),
                                            np.zeros(0, np.int32), 4, 2)
    # the launcher returns before writing anything when bs == 0
    assert pt.shape[0] == 0 and cache.shape == (0,) and cu.tolist() == [-0x5A5A5A5A]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_metadata_inverts_generator_placement(cfg):
    """For page-aligned maps, page_table[i, t // P] * P + t % P must give back
    req_to_token[rpi[i], t] for every t < L_i, and used columns must equal the
    generator's own page placement (which built req_to_token the other way)."""
    c = W.make_config(cfg)
    pt, cache, cu = oracle.case_page_table(c)
    P = c.page_size
    for i in range(c.batch):
        L = int(c.seq_lens[i])
        t = np.arange(L)
        back = pt[i, t // P].astype(np.int64) * P + t % P
        assert np.array_equal(back, c.req_to_token[c.req_pool_indices[i], :L].astype(np.int64))
        npg = -(-L // P)
        assert np.array_equal(pt[i, :npg], c.page_list[i, :npg])
        # columns past the request's own pages come from the filler slots
        assert np.all((pt[i] >= 0) & (pt[i] < c.num_pages))
    assert np.array_equal(cache, c.seq_lens)
    assert cu[0] == 0 and np.array_equal(np.diff(cu), cache)
    assert cu[-1] == int(np.sum(c.seq_lens.astype(np.int64)))


def test_metadata_offset_and_cumsum_wrap_int32():
    r2t = np.arange(16, dtype=np.int32).reshape(2, 8)
    rpi = np.array([1, 0], np.int32)
    sl = np.array([2**31 - 10, 5], np.int32)
    pt, cache, cu = oracle.build_page_table(r2t, rpi, sl, 4, 2, seqlen_offset=3)
    assert cache.tolist() == [2**31 - 7, 8]
    # int32 cumsum wraps like the int32 scan it defines
    assert cu.tolist() == [0, 2**31 - 7, np.int32(np.int64(2**31 - 7 + 8) - 2**32)]
    assert pt.tolist() == [[2, 3], [0, 1]]


def _swa_golden():
    return json.load(open(os.path.join(GOLDEN, "metadata_swa_tiny.json")))


@pytest.mark.parametrize("q_mode", [0, 1, 2])
def test_metadata_full_golden_hand_example(q_mode):
    g = _swa_golden()
    preset_q = np.full(3, 55, np.int32)
    out = oracle.build_metadata(
        np.array(g["req_to_token"], np.int32), np.array(g["req_pool_indices"], np.int32),
        np.array(g["seq_lens"], np.int32), g["page_size"], g["max_seq_pages"],
        seqlen_offset=g["seqlen_offset"], page_table=np.array(g["table_preset"], np.int32),
        q_mode=q_mode, qlens=np.array(g["qlens"], np.int32), q_stride=g["q_stride"],
        cu_seqlens_q=preset_q, swa_mapping=np.array(g["full_to_swa"], np.int64),
        swa_page_table=np.array(g["table_preset"], np.int32),
        out_cache_loc=np.array(g["out_cache_loc"], np.int64),
        swa_out_cache_loc=np.full(g["swa_out_len"], 99, np.int64))
    assert out["page_table"].tolist() == g["expect_page_table"]
    assert out["swa_page_table"].tolist() == g["expect_swa_page_table"]
    assert out["cache_seqlens"].tolist() == g["expect_cache_seqlens"]
    assert out["cu_seqlens_k"].tolist() == g["expect_cu_seqlens_k"]
    assert out["swa_out_cache_loc"].tolist() == g["expect_swa_out_cache_loc"]
    want_q = {0: [55, 55, 55], 1: g["expect_cu_seqlens_q_cumsum"],
              2: g["expect_cu_seqlens_q_strided"]}[q_mode]
    assert out["cu_seqlens_q"].tolist() == want_q


def test_metadata_swa_out_shorter_than_out_cache_loc():
    g = _swa_golden()
    out = oracle.build_metadata(
        np.array(g["req_to_token"], np.int32), np.array(g["req_pool_indices"], np.int32),
        np.array(g["seq_lens"], np.int32), g["page_size"], g["max_seq_pages"],
        swa_mapping=np.array(g["full_to_swa"], np.int64),
        out_cache_loc=np.array(g["out_cache_loc"], np.int64),
        swa_out_cache_loc=np.full(g["short_swa_out_len"], 99, np.int64))
    assert out["swa_out_cache_loc"].tolist() == g["expect_short_swa_out_cache_loc"]
    assert out["swa_page_table"] is None


def test_metadata_swa_out_without_out_cache_loc_is_all_padding():
    """The launcher sets num_out_tokens = 0 when out_cache_loc is absent: the
    whole output is the zero padding and the mapping is never read."""
    r2t = np.arange(16, dtype=np.int32).reshape(2, 8)
    out = oracle.build_metadata(r2t, np.array([0], np.int32), np.array([3], np.int32), 4, 2,
                                swa_out_cache_loc=np.full(5, 99, np.int64))
    assert out["swa_out_cache_loc"].tolist() == [0] * 5


def test_metadata_full_bs0_writes_nothing():
    r2t = np.zeros((1, 8), np.int32)
    swa_out = np.full(4, 99, np.int64)
    cuq = np.full(1, 55, np.int32)
    oracle.build_metadata(r2t, np.zeros(0, np.int32), np.zeros(0, np.int32), 4, 2, q_mode=2,
                          q_stride=3, cu_seqlens_q=cuq, swa_mapping=np.zeros(8, np.int64),
                          out_cache_loc=np.zeros(4, np.int64), swa_out_cache_loc=swa_out)
    assert swa_out.tolist() == [99] * 4 and cuq.tolist() == [55]


@pytest.mark.parametrize("cfg", [1, 3, 5])
def test_metadata_identity_swa_mapping_reproduces_page_table(cfg):
    """With full_to_swa the identity, every slot the generator placed is >= 0,
    so the sliding-window table must equal the full page table, and the
    translated out_cache_loc must equal out_cache_loc with its zero tail."""
    c = W.make_config(cfg)
    bs, msp = c.batch, c.page_list.shape[1]
    n_slots = c.num_pages * c.page_size
    ident = np.arange(n_slots + c.page_size + 1, dtype=np.int64)
    rng = np.random.default_rng(cfg)
    ocl = rng.integers(0, n_slots, size=bs).astype(np.int64)
    out = oracle.build_metadata(c.req_to_token, c.req_pool_indices, c.seq_lens, c.page_size,
                                msp, swa_mapping=ident, swa_page_table=True, out_cache_loc=ocl,
                                swa_out_cache_loc=np.full(bs + 9, 99, np.int64))
    assert np.array_equal(out["swa_page_table"], out["page_table"])
    assert out["swa_out_cache_loc"].tolist() == ocl.tolist() + [0] * 9


def test_metadata_swa_unmapped_and_negative_slots_give_minus_one():
    """A mapping that evicts every slot gives page -1 everywhere; a negative
    slot gives -1 without reading the mapping."""
    r2t = np.array([[-3, -3, -3, -3, 7, 7, 7, 7]], np.int32)
    out = oracle.build_metadata(r2t, np.array([0, 0], np.int32), np.array([1, 1], np.int32), 4,
                                2, swa_mapping=np.full(8, -9, np.int64), swa_page_table=True,
                                out_cache_loc=np.array([-1, 3], np.int64),
                                swa_out_cache_loc=np.zeros(2, np.int64))
    assert out["swa_page_table"].tolist() == [[-1, -1], [-1, -1]]
    assert out["page_table"].tolist() == [[-1, 1], [-1, 1]]
    # any negative mapped slot is the sentinel -1, not floor(-9 / 4) = -3 ...
    # ... but swa_out_cache_loc passes the mapped value through unchanged
    assert out["swa_out_cache_loc"].tolist() == [-1, -9]


def test_metadata_q_modes_agree_and_wrap_int32():
    """Equal qlens make the cumsum mode the strided mode; the cumsum's steps
    give back qlens; both wrap modulo 2^32 like the int32 arithmetic."""
    bs = 37
    r2t = np.zeros((1, 64), np.int32)
    rpi = np.zeros(bs, np.int32)
    sl = np.ones(bs, np.int32)
    for stride in (1, 5, 2**30 + 3):
        a = oracle.build_metadata(r2t, rpi, sl, 64, 1, q_mode=1,
                                  qlens=np.full(bs, stride, np.int32))["cu_seqlens_q"]
        b = oracle.build_metadata(r2t, rpi, sl, 64, 1, q_mode=2, q_stride=stride)["cu_seqlens_q"]
        assert np.array_equal(a, b)
        want = ((np.arange(bs + 1, dtype=np.int64) * stride + 2**31) % 2**32 - 2**31)
        assert a.tolist() == want.tolist()
    ql = np.random.default_rng(5).integers(0, 9, size=bs).astype(np.int32)
    cu = oracle.build_metadata(r2t, rpi, sl, 64, 1, q_mode=1, qlens=ql)["cu_seqlens_q"]
    assert cu[0] == 0 and np.array_equal(np.diff(cu), ql)


# ---------------------------------------------------------------- attention: golden

def _golden_case(c, int8=False):
    Hq, Hkv, D, P = c["num_q_heads"], c["num_kv_heads"], c["head_dim"], c["page_size"]
    q = _bits(c["q"]).reshape(1, Hq, D)
    pt = np.array([c["page_table"]], np.int32)
    sl = np.array([c["seq_len"]], np.int32)
    if int8:
        k = np.array(c["k_pool_q8"], np.int8)
        v = np.array(c["v_pool_q8"], np.int8)
        ks = np.array(c["k_scales"], np.float32).reshape(k.shape[:3])
        vs = np.array(c["v_scales"], np.float32).reshape(v.shape[:3])
        return oracle.paged_attention(q, k, v, pt, sl, num_kv_heads=Hkv, page_size=P,
                                      scale=c["scale"], kv_dtype="int8", k_scales=ks,
                                      v_scales=vs)
    k = _bits(c["k_pool"])
    v = _bits(c["v_pool"])
    return oracle.paged_attention(q, k, v, pt, sl, num_kv_heads=Hkv, page_size=P,
                                  scale=c["scale"])


@pytest.mark.parametrize("idx", range(3))
def test_attention_golden_closed_forms(idx):
    c = json.load(open(os.path.join(GOLDEN, "attention_tiny.json")))["cases"][idx]
    out, lse = _golden_case(c)
    want_o = np.array([[_ev(x) for x in row] for row in c["expect_out"]])
    want_l = np.array([_ev(x) for x in c["expect_lse"]])
    np.testing.assert_allclose(out[0], want_o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], want_l, rtol=0, atol=1e-14)


def test_attention_golden_int8():
    c = json.load(open(os.path.join(GOLDEN, "attention_tiny.json")))["int8_cases"][0]
    out, lse = _golden_case(c, int8=True)
    want_o = np.array([[_ev(x) for x in row] for row in c["expect_out"]])
    np.testing.assert_allclose(out[0], want_o, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[0], [_ev(c["expect_lse"][0])], rtol=0, atol=1e-14)


# ---------------------------------------------------------------- attention: brute force

SMALL = [
    # (seq_lens, Hq, Hkv, D, P, num_pages)
    ([1], 4, 1, 8, 4, 8),
    ([2, 63], 8, 2, 8, 4, 24),
    ([64, 65], 32, 8, 128, 64, 8),
    ([130], 8, 2, 128, 64, 5),
    ([63, 1], 32, 8, 128, 64, 4),
    ([5, 9, 17], 4, 1, 8, 4, 12),
]


@pytest.mark.parametrize("kv", ["bf16", "int8"])
@pytest.mark.parametrize("shape", SMALL)
def test_attention_matches_dense_brute_force(shape, kv):
    lens, Hq, Hkv, D, P, npg = shape
    msp = max(-(-L // P) for L in lens) + 1
    c = W.make_case(seed=11, seq_lens=lens, num_pages=npg, num_splits=2, kv_dtype=kv,
                    num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
                    req_pool_rows=4, req_to_token_stride=msp * P, max_seq_pages=msp)
    out, lse = oracle.case_attention(c)
    bo, bl = dense_attention(c)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_attention_config1_matches_brute_force():
    c = W.make_config(1)
    out, lse = oracle.case_attention(c)
    bo, bl = dense_attention(c)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_attention_via_metadata_page_table_equals_generator_placement():
    c = W.make_config(3)
    pt, _, _ = oracle.case_page_table(c)
    a = oracle.case_attention(c, page_table=pt)
    b = oracle.case_attention(c)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- special cases

def _small(lens, **kw):
    base = dict(seed=5, seq_lens=lens, num_pages=16, num_splits=4, num_q_heads=8,
                num_kv_heads=2, head_dim=16, page_size=8, req_pool_rows=4,
                req_to_token_stride=256, max_seq_pages=16)
    base.update(kw)
    return W.make_case(**base)


def test_single_token_returns_its_value_row():
    c = _small([1, 1])
    out, lse = oracle.case_attention(c)
    qf = W.bf16_bits_to_f32(c.q).astype(np.float64)
    for b in range(c.batch):
        k, v, _, _ = c.dense_kv(b)
        kf = W.bf16_bits_to_f32(k).astype(np.float64)
        vf = W.bf16_bits_to_f32(v).astype(np.float64)
        for h in range(c.num_q_heads):
            g = h // c.group
            assert np.array_equal(out[b, h], vf[0, g])
            assert lse[b, h] == pytest.approx(float(c.scale) * float(qf[b, h] @ kf[0, g]),
                                              abs=1e-12)


def test_zero_query_gives_mean_of_values():
    c = _small([37, 8], q_override=np.zeros((2, 8, 16), np.uint16))
    out, lse = oracle.case_attention(c)
    for b in range(c.batch):
        _, v, _, _ = c.dense_kv(b)
        vf = W.bf16_bits_to_f32(v).astype(np.float64)
        L = vf.shape[0]
        for h in range(c.num_q_heads):
            np.testing.assert_allclose(out[b, h], vf[:, h // c.group].mean(0), atol=1e-14)
            assert lse[b, h] == pytest.approx(math.log(L), abs=1e-14)


def test_constant_value_rows_give_that_constant():
    c = _small([29])
    c.v_pages[...] = _bits(np.float32(0.375))
    out, _ = oracle.case_attention(c)
    assert np.all(np.abs(out - 0.375) < 1e-15)


def test_large_logits_no_overflow():
    qf = np.random.default_rng(3).standard_normal((1, 8, 16)).astype(np.float32) * 30
    c = _small([100], q_override=_bits(qf))
    out, lse = oracle.case_attention(c)
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    bo, bl = dense_attention(c)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=1e-14, atol=1e-12)


def test_empty_request_gives_zero_and_minus_inf():
    c = _small([0, 3])
    out, lse = oracle.case_attention(c)
    assert np.all(out[0] == 0) and np.all(lse[0] == -np.inf)
    assert np.all(np.isfinite(lse[1]))


# ---------------------------------------------------------------- invariances

@pytest.mark.parametrize("S", [1, 2, 3, 4, 16, 128])
def test_split_merge_equals_direct(S):
    c = _small([1, 8, 9, 100], num_pages=40, req_pool_rows=8)
    out, lse = oracle.case_attention(c)
    acc, m, l = oracle.split_partials(c.q, c.k_pages, c.v_pages, c.page_list, c.seq_lens,
                                      num_kv_heads=c.num_kv_heads, page_size=c.page_size,
                                      scale=c.scale, num_splits=S)
    mo, ml = oracle.split_merge(acc, m, l)
    np.testing.assert_allclose(mo, out, rtol=0, atol=1e-14)
    np.testing.assert_allclose(ml, lse, rtol=0, atol=1e-13)


def test_split_partial_contract_single_split_and_empty_splits():
    c = _small([8], num_pages=4)
    acc, m, l = oracle.split_partials(c.q, c.k_pages, c.v_pages, c.page_list, c.seq_lens,
                                      num_kv_heads=2, page_size=8, scale=c.scale, num_splits=3)
    # one page, three splits: split 0 holds everything, splits 1 and 2 are empty
    assert np.all(m[:, :, 1:] == -np.inf) and np.all(l[:, :, 1:] == 0) and np.all(acc[:, :, 1:] == 0)
    out, lse = oracle.case_attention(c)
    np.testing.assert_allclose(acc[:, :, 0] / l[:, :, 0, None], out, atol=1e-15)
    np.testing.assert_allclose(m[:, :, 0] + np.log(l[:, :, 0]), lse, atol=1e-14)


def _repermute(c, seed):
    """Move every physical page to a new slot and update the placement; the
    logical data are unchanged."""
    rng = np.random.default_rng(seed)
    sigma = rng.permutation(c.num_pages)          # old page p -> new page sigma[p]
    k = np.empty_like(c.k_pages); k[sigma] = c.k_pages
    v = np.empty_like(c.v_pages); v[sigma] = c.v_pages
    pl = np.where(c.page_list >= 0, sigma[np.maximum(c.page_list, 0)], -1).astype(np.int32)
    kw = {}
    if c.k_scales is not None:
        ks = np.empty_like(c.k_scales); ks[sigma] = c.k_scales
        vs = np.empty_like(c.v_scales); vs[sigma] = c.v_scales
        kw = dict(k_scales=ks, v_scales=vs)
    return k, v, pl, kw


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_physical_page_permutation_is_bit_identical(kv):
    c = _small([50, 3, 17], num_pages=30, kv_dtype=kv)
    out, lse = oracle.case_attention(c)
    k, v, pl, kw = _repermute(c, 1)
    o2, l2 = oracle.paged_attention(c.q, k, v, pl, c.seq_lens, num_kv_heads=2, page_size=8,
                                    scale=c.scale, kv_dtype=kv, **kw)
    assert np.array_equal(out, o2) and np.array_equal(lse, l2)


def test_logical_key_order_permutation():
    c = _small([40], num_pages=5)
    out, lse = oracle.case_attention(c)
    P = c.page_size
    pages = c.page_list[0, :5]
    rows = np.arange(40)
    perm = np.random.default_rng(2).permutation(40)
    k = c.k_pages.copy(); v = c.v_pages.copy()
    src_k = c.k_pages[pages].reshape(40, 2, 16)
    src_v = c.v_pages[pages].reshape(40, 2, 16)
    k[pages] = src_k[perm].reshape(5, P, 2, 16)
    v[pages] = src_v[perm].reshape(5, P, 2, 16)
    o2, l2 = oracle.paged_attention(c.q, k, v, c.page_list, c.seq_lens, num_kv_heads=2,
                                    page_size=P, scale=c.scale)
    np.testing.assert_allclose(o2, out, atol=1e-14)
    np.testing.assert_allclose(l2, lse, atol=1e-13)
    assert rows.size == 40


def test_gqa_identical_queries_in_group_give_identical_outputs():
    c = _small([33])
    q = c.q.copy()
    q[:, 1:4] = q[:, 0:1]     # heads 0..3 form KV group 0 (group size 4)
    o, l = oracle.paged_attention(q, c.k_pages, c.v_pages, c.page_list, c.seq_lens,
                                  num_kv_heads=2, page_size=8, scale=c.scale)
    for h in range(1, 4):
        assert np.array_equal(o[:, h], o[:, 0]) and np.array_equal(l[:, h], l[:, 0])
    assert not np.array_equal(o[:, 4], o[:, 0])


def _fp8_every_code_case():
    """Two one-token requests whose K and V rows (8 kv heads x 128 dims each)
    hold every finite e4m3 code; NaN codes are replaced by 0."""
    c = _small([1, 1], kv_dtype="fp8", num_q_heads=32, num_kv_heads=8, head_dim=128)
    codes = (np.arange(2 * 8 * 128) % 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    codes = codes.reshape(2, 8, 128)
    for b in range(2):
        page = c.page_list[b, 0]
        c.k_pages[page, 0] = codes[b]
        c.v_pages[page, 0] = np.roll(codes[b], 3, axis=1)
    return c


def test_fp8_value_decoding_of_every_code_matches_torch():
    """One-token context: the output is the dequantised V row itself, so each
    element must equal PyTorch's e4m3 value of the code times sigma_v."""
    c = _fp8_every_code_case()
    out, _ = oracle.case_attention(c)
    for b in range(2):
        _, v, _, vs = c.dense_kv(b)
        want = e4m3_codes_to_f64(v[0]) * vs[0].astype(np.float64)[:, None]   # [Hkv, D]
        for h in range(c.num_q_heads):
            assert np.array_equal(out[b, h], want[h // c.group]), (b, h)


def test_fp8_key_decoding_of_every_code_matches_torch():
    """One-token context with a one-hot query: lse = s = scale * sigma_k *
    e4m3(code) of the selected dimension, for every dimension and head."""
    base = _fp8_every_code_case()
    for d0 in range(0, 128, 4):
        q = np.zeros((2, 32, 128), np.float32)
        for h in range(32):
            q[:, h, (d0 + h % 4) % 128] = 1.0
        qb = W.f32_to_bf16_bits(q)
        _, lse = oracle.paged_attention(qb, base.k_pages, base.v_pages, base.page_list,
                                        base.seq_lens, num_kv_heads=8, page_size=base.page_size,
                                        scale=base.scale, kv_dtype="fp8",
                                        k_scales=base.k_scales, v_scales=base.v_scales)
        for b in range(2):
            k, _, ks, _ = base.dense_kv(b)
            kv = e4m3_codes_to_f64(k[0]) * ks[0].astype(np.float64)[:, None]
            for h in range(32):
                want = float(base.scale) * kv[h // 4, (d0 + h % 4) % 128]
                assert lse[b, h] == pytest.approx(want, rel=1e-15, abs=1e-300), (d0, b, h)


def test_fp8_known_code_values():
    """Values fixed by the e4m3 format: 448 is the largest finite value,
    2^-6 the smallest normal, 2^-9 the smallest subnormal, 1.0 is 0x38, and
    the sign bit negates."""
    c = _small([1], kv_dtype="fp8", num_q_heads=32, num_kv_heads=8, head_dim=128)
    page = c.page_list[0, 0]
    row = np.zeros((8, 128), np.uint8)
    row[0, :6] = [0x7E, 0x08, 0x01, 0x38, 0xB8, 0xFE]
    c.v_pages[page, 0] = row
    c.v_scales[page, 0] = 1.0
    out, _ = oracle.case_attention(c)
    assert out[0, 0, :6].tolist() == [448.0, 2.0**-6, 2.0**-9, 1.0, -1.0, -448.0]


def test_int8_dequantisation_is_exact_product():
    c = _small([20], kv_dtype="int8")
    k, v, ks, vs = c.dense_kv(0)
    # sigma * q8 with |q8| <= 127 is exact in fp64; the brute force agrees
    out, lse = oracle.case_attention(c)
    bo, bl = dense_attention(c)
    np.testing.assert_allclose(out, bo, atol=1e-12)
    np.testing.assert_allclose(lse, bl, atol=1e-12)
    assert np.max(np.abs(k.astype(np.int32))) <= 127


# ---------------------------------------------------------------- multi-token decode

def _verify(c, q_rows, cu):
    return oracle.verify_attention(q_rows, c.k_pages, c.v_pages, c.page_list, c.seq_lens, cu,
                                   num_kv_heads=c.num_kv_heads, page_size=c.page_size,
                                   scale=c.scale, kv_dtype=c.kv_dtype, k_scales=c.k_scales,
                                   v_scales=c.v_scales)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("lens,qlens", [([20, 9, 33], [4, 1, 3]), ([5, 64, 2], [2, 4, 2]),
                                        ([17, 40], [0, 4]),
                                        # 6 rows: a speculative step with 5 draft tokens
                                        ([70, 6, 129], [6, 6, 5]), ([11, 66], [8, 7])])
def test_verify_matches_dense_causal_brute_force(kv, lens, qlens):
    c = _small(lens, kv_dtype=kv, num_pages=40, max_seq_pages=24)
    q_rows, cu = W.verify_queries(c, qlens)
    out, lse = _verify(c, q_rows, cu)
    bo, bl = dense_verify(c, q_rows, cu)
    np.testing.assert_allclose(out, bo, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, bl, rtol=0, atol=1e-12)


def test_verify_query_i_is_decode_over_its_prefix():
    """Query token i of a request with n queries is exactly the one-token
    decode of the same query over the first L - n + i + 1 tokens."""
    c = _small([30, 23, 11, 70], kv_dtype="bf16", num_pages=24)
    qlens = [4, 3, 2, 6]
    q_rows, cu = W.verify_queries(c, qlens)
    out, lse = _verify(c, q_rows, cu)
    for b in range(c.batch):
        n = qlens[b]
        for i in range(n):
            row = cu[b] + i
            sl = c.seq_lens.copy()
            sl[b] = c.seq_lens[b] - n + i + 1
            q1 = np.repeat(q_rows[row][None], c.batch, axis=0)
            o1, l1 = oracle.paged_attention(q1, c.k_pages, c.v_pages, c.page_list, sl,
                                            num_kv_heads=c.num_kv_heads, page_size=c.page_size,
                                            scale=c.scale)
            assert np.array_equal(out[row], o1[b]) and np.array_equal(lse[row], l1[b])


def test_verify_zero_query_closed_form():
    """With q = 0 every visible score is 0: query token i of a request of
    length L with n queries averages the first L - n + i + 1 value rows and
    lse = ln(L - n + i + 1)."""
    c = _small([7, 3], kv_dtype="bf16")
    qlens = [3, 3]
    q_rows, cu = W.verify_queries(c, qlens)
    q_rows[:] = 0
    out, lse = _verify(c, q_rows, cu)
    for b in range(2):
        _, v, _, _ = c.dense_kv(b)
        vf = W.bf16_bits_to_f32(v).astype(np.float64)
        for i in range(3):
            vis = int(c.seq_lens[b]) - 3 + i + 1
            row = cu[b] + i
            for h in range(c.num_q_heads):
                np.testing.assert_allclose(out[row, h], vf[:vis, h // c.group].mean(axis=0),
                                           rtol=0, atol=1e-15)
                assert lse[row, h] == pytest.approx(math.log(vis), abs=1e-15)


def test_verify_single_query_equals_decode():
    c = _small([50, 1, 17], kv_dtype="int8")
    q_rows, cu = W.verify_queries(c, [1, 1, 1])
    out, lse = _verify(c, q_rows, cu)
    o1, l1 = oracle.paged_attention(q_rows, c.k_pages, c.v_pages, c.page_list, c.seq_lens,
                                    num_kv_heads=c.num_kv_heads, page_size=c.page_size,
                                    scale=c.scale, kv_dtype="int8", k_scales=c.k_scales,
                                    v_scales=c.v_scales)
    assert np.array_equal(out, o1) and np.array_equal(lse, l1)
