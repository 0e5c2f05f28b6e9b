"""GPU parity for split-K paged-attention decode against the fp64 oracle,
through the C ABI.  Tolerances: bf16 output max-abs 1e-2, LSE max-abs 1e-3
(tests/gpu_util.py); structural properties (one-token context, fused vs
two-launch, repeat, page permutation, GQA grouping) are checked bit-exactly."""
import numpy as np
import pytest
import torch

import oracle
import split_paged_attention_amd as spa
import workloads as W
from tests.gpu_util import (DevCase, balanced_walk_lens, bf16_dev, bits_host, compare_attention,
                            config_case, counters_view, walks_balanced, COUNTER_REGION_BYTES)

pytestmark = pytest.mark.gpu

PRODUCERS = ["page_split", "head_grouped"]


def small_case(lens, kv="bf16", S=4, seed=21, num_pages=None, q_override=None, Hkv=8):
    P = 64
    need = sum(-(-L // P) for L in lens)
    msp = max(1, max(-(-L // P) for L in lens))
    return W.make_case(seed=seed, seq_lens=lens, num_pages=num_pages or need + 3, num_splits=S,
                       kv_dtype=kv, num_q_heads=4 * Hkv, num_kv_heads=Hkv, head_dim=128,
                       page_size=P, req_pool_rows=max(4, len(lens)),
                       req_to_token_stride=msp * P, max_seq_pages=msp, q_override=q_override,
                       name=f"lens{lens}_{kv}_S{S}")


# ---------------------------------------------------------------- configs

@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_config_parity_full(cfg):
    c = config_case(cfg)
    print(f"[case] attention config {cfg} ({c.name}) full parity", flush=True)
    d = DevCase(c)
    pt, _, _ = d.page_table()
    out, lse = d.attention(page_table=pt)
    pt_o, _, _ = oracle.case_page_table(c)
    o_ref, l_ref = oracle.case_attention(c, page_table=pt_o)
    compare_attention(out, lse, o_ref, l_ref, label=c.name)


def test_config4_headline_parity():
    """Batch 32 / context 8K in the launch configuration the benchmark times
    (library defaults), every output checked (the oracle finishes it in
    seconds); then both producers with both merges, bit-identical per producer."""
    c = config_case(4)
    print(f"[case] attention config 4 ({c.name}) full parity", flush=True)
    d = DevCase(c)
    pt, _, _ = d.page_table()
    out, lse = d.attention(page_table=pt)
    o_ref, l_ref = oracle.case_attention(c)
    compare_attention(out, lse, o_ref, l_ref, label=c.name)
    for producer in PRODUCERS:
        o1, l1 = d.attention(page_table=pt, producer=producer, merge="fused")
        compare_attention(o1, l1, o_ref, l_ref, label=f"{c.name} {producer} fused")
        o2, l2 = d.attention(page_table=pt, producer=producer, merge="separate")
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_config6_fp8_headline_parity():
    """Batch 32 / context 8K with e4m3 KV: library defaults, then both
    producers with both merges (bit-identical per producer), every output."""
    c = config_case(6)
    print(f"[case] attention config 6 ({c.name}) full parity", flush=True)
    d = DevCase(c)
    pt, _, _ = d.page_table()
    out, lse = d.attention(page_table=pt)
    o_ref, l_ref = oracle.case_attention(c)
    compare_attention(out, lse, o_ref, l_ref, label=c.name)
    for producer in PRODUCERS:
        o1, l1 = d.attention(page_table=pt, producer=producer, merge="fused")
        compare_attention(o1, l1, o_ref, l_ref, label=f"{c.name} {producer} fused")
        o2, l2 = d.attention(page_table=pt, producer=producer, merge="separate")
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("producer", PRODUCERS)
def test_fp8_every_code_in_keys_and_values(producer):
    """One-token contexts whose K and V rows hold every finite e4m3 code (the
    hardware conversion of each code meets the oracle's decoding), plus a
    longer context over the same codes."""
    c = small_case([1, 1, 300], kv="fp8", S=4)
    codes = (np.arange(3 * 8 * 128) % 256).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0
    codes = codes.reshape(3, 8, 128)
    for b in range(2):
        page = c.page_list[b, 0]
        c.k_pages[page, 0] = codes[b]
        c.v_pages[page, 0] = np.roll(codes[b], 5, axis=1)
    print(f"[case] fp8 every code {producer}", flush=True)
    out, lse = DevCase(c).attention(producer=producer)
    o_ref, l_ref = oracle.case_attention(c)
    compare_attention(out, lse, o_ref, l_ref, label=f"fp8 codes {producer}")


# ---------------------------------------------------------------- ragged / edges

@pytest.mark.parametrize("producer", PRODUCERS)
@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("lens,S", [
    ([1, 63, 64, 65], 1),
    ([127, 128, 129, 1000], 3),
    ([1, 2, 3, 700], 16),           # splits with no pages
    ([4096, 5, 64, 191], 64),       # many empty splits
    ([8192, 8191, 1], 16),
])
def test_ragged_parity(lens, S, kv, producer):
    c = small_case(lens, kv=kv, S=S)
    print(f"[case] ragged {c.name} {producer}", flush=True)
    out, lse = DevCase(c).attention(producer=producer)
    o_ref, l_ref = oracle.case_attention(c)
    compare_attention(out, lse, o_ref, l_ref, label=c.name)


def test_zero_length_request():
    c = small_case([0, 70, 0], S=4)
    print("[case] zero-length requests", flush=True)
    out, lse = DevCase(c).attention()
    o_ref, l_ref = oracle.case_attention(c)
    compare_attention(out, lse, o_ref, l_ref, label="L=0")
    o = bits_host(out)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert torch.all(torch.isneginf(lse[0])) and torch.all(torch.isneginf(lse[2]))


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_single_token_returns_value_row_bit_exact(kv):
    c = small_case([1, 1, 1], kv=kv, S=4)
    print(f"[case] one-token context {kv}", flush=True)
    out, lse = DevCase(c).attention()
    o_ref, l_ref = oracle.case_attention(c)
    compare_attention(out, lse, o_ref, l_ref, label=f"L=1 {kv}")
    if kv != "bf16":
        return   # int8: the value scale is folded into the bf16 probability, so within tolerance
    got = bits_host(out)
    for b in range(c.batch):
        k, v, _, _ = c.dense_kv(b)
        for h in range(c.num_q_heads):
            assert np.array_equal(got[b, h], v[0, h // c.group])


def test_large_logits():
    qf = np.random.default_rng(4).standard_normal((2, 32, 128)).astype(np.float32) * 30
    c = small_case([900, 77], S=4, q_override=W.f32_to_bf16_bits(qf))
    print("[case] large logits", flush=True)
    out, lse = DevCase(c).attention()
    assert torch.isfinite(lse).all()
    o_ref, l_ref = oracle.case_attention(c)
    compare_attention(out, lse, o_ref, l_ref, label="q*30")


# ---------------------------------------------------------------- structure

@pytest.mark.parametrize("producer", PRODUCERS)
@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_fused_equals_two_launch_bit_exact(kv, producer):
    c = small_case([3000, 64, 1, 777], kv=kv, S=16)
    print(f"[case] fused vs separate merge {kv} {producer}", flush=True)
    d = DevCase(c)
    o1, l1 = d.attention(merge="fused", producer=producer)
    o2, l2 = d.attention(merge="separate", producer=producer)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_default_head_grouped_fused_merge(kv):
    """A head-grouped grid of 4 splits, where the default plan fuses the
    merge into the producer launch (32 ragged requests x 8 kv heads x 4
    splits = 1024 triples): against the oracle, and bit-exactly against the
    two-launch merge."""
    lens = W._gen(32, 5).integers(1, 3000, size=32).tolist()
    lens[:3] = [1, 64, 2999]
    c = small_case(lens, kv=kv, S=4, seed=16)
    assert spa.decode_default_flags(32, 8, 4, kv, c.max_seq_pages) == (
        spa.SPA_DECODE_HEAD_GROUPED | spa.SPA_DECODE_FUSED_MERGE)
    print(f"[case] default head-grouped fused {kv} batch 32 S=4", flush=True)
    d = DevCase(c)
    o1, l1 = d.attention()
    o_ref, l_ref = oracle.case_attention(c)
    compare_attention(o1, l1, o_ref, l_ref, label=f"hg fused default {kv}")
    o2, l2 = d.attention(producer="head_grouped", merge="separate")
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_repeat_bit_identical_and_counters_return_to_zero():
    c = config_case(3)
    print("[case] repeat x20 + counters", flush=True)
    d = DevCase(c)
    B, Hq, D, S = c.batch, c.num_q_heads, c.head_dim, c.num_splits
    ws = spa.new_workspace(B, Hq, c.num_kv_heads, D, S)
    o0, l0 = d.attention(workspace=ws)
    for _ in range(20):
        o, l = d.attention(workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), o0.view(torch.int16)) and torch.equal(l, l0)
    assert int(counters_view(ws).abs().sum()) == 0


def test_alternating_inputs_share_one_workspace():
    """Two different batches of the same shape alternate on one workspace: a
    merge that read partial state left by the previous call (instead of this
    call's) would give the other batch's answer."""
    ca = small_case([3000, 700, 65, 1], S=16, seed=31)
    cb = small_case([3000, 700, 65, 1], S=16, seed=32)
    print("[case] alternating inputs on one workspace", flush=True)
    da, db = DevCase(ca), DevCase(cb)
    ref_a = da.attention(separate_merge=True)
    ref_b = db.attention(separate_merge=True)
    ws = spa.new_workspace(4, 32, 8, 128, 16)
    for it in range(6):
        d, ref = (da, ref_a) if it % 2 == 0 else (db, ref_b)
        o, l = d.attention(workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16), ref[0].view(torch.int16)), it
        assert torch.equal(l, ref[1]), it


def test_one_workspace_serves_every_shape_and_entry_point():
    """One workspace, sized for the largest call, serves in turn fused
    decode calls of two batch sizes, a multi-token decode call and a
    separate-merge call.  The counters sit in a region no call writes partial
    state to, so every fused call still merges exactly once: each output
    equals that of the same call on a fresh workspace, bit for bit, and the
    counters end at zero."""
    ca = small_case([3000, 700, 65, 1], S=8, seed=41)           # 4 requests
    cb = small_case([900, 64, 1, 2500, 130, 7, 4000, 12, 640], S=8, seed=42)   # 9
    print("[case] one workspace: fused decode at two batch sizes + multi-token + separate",
          flush=True)
    da, db = DevCase(ca), DevCase(cb)
    q_rows, cu = W.verify_queries(cb, [3, 1, 1, 4, 2, 0, 4, 1, 2])
    qv, cuv = bf16_dev(q_rows), torch.from_numpy(cu).cuda()
    T = q_rows.shape[0]

    def verify(ws):
        return spa.paged_verify_attention(qv, db.k, db.v, db.page_list, db.seq_lens, cuv, 8,
                                          float(cb.scale), max_q_len=4, workspace=ws)

    calls = [lambda ws: da.attention(merge="fused", producer="page_split", workspace=ws),
             lambda ws: db.attention(merge="fused", producer="page_split", workspace=ws),
             verify,
             lambda ws: da.attention(merge="separate", producer="head_grouped", workspace=ws),
             lambda ws: db.attention(merge="fused", producer="head_grouped", workspace=ws)]
    refs = [f(spa.new_workspace(40, 32, 8, 128, 8)) for f in calls]
    nbytes = max(spa.decode_workspace_bytes(cb.batch, 32, 8, 128, 8),
                 spa.verify_workspace_bytes(T, 32, 8, 128, 8))
    ws = torch.zeros((nbytes,), dtype=torch.uint8, device="cuda")
    for it in range(3):
        for k, f in enumerate(calls):
            o, l = f(ws)
            torch.cuda.synchronize()
            assert torch.equal(o.view(torch.int16), refs[k][0].view(torch.int16)), (it, k)
            assert torch.equal(l, refs[k][1]), (it, k)
    assert int(counters_view(ws).abs().sum()) == 0


def test_nan_poisoned_partials_region_is_never_read_before_write():
    c = small_case([1500, 2, 640], S=8)
    print("[case] NaN-poisoned workspace", flush=True)
    d = DevCase(c)
    B, Hq, D, S = c.batch, c.num_q_heads, c.head_dim, c.num_splits
    ws = spa.new_workspace(B, Hq, c.num_kv_heads, D, S)
    ws[COUNTER_REGION_BYTES:].view(torch.float32).fill_(float("nan"))
    out, lse = d.attention(workspace=ws)
    o_ref, l_ref = oracle.case_attention(c)
    compare_attention(out, lse, o_ref, l_ref, label="poisoned")


def test_physical_page_permutation_bit_identical():
    c = small_case([900, 130, 64, 1], S=4, num_pages=40)
    print("[case] physical page permutation", flush=True)
    d = DevCase(c)
    o1, l1 = d.attention()
    sigma = np.random.default_rng(9).permutation(c.num_pages)
    k = np.empty_like(c.k_pages); k[sigma] = c.k_pages
    v = np.empty_like(c.v_pages); v[sigma] = c.v_pages
    pl = np.where(c.page_list >= 0, sigma[np.maximum(c.page_list, 0)], -1).astype(np.int32)
    o2, l2 = spa.paged_decode_attention(d.q, bf16_dev(k), bf16_dev(v),
                                        torch.from_numpy(pl).cuda(), d.seq_lens, c.num_splits,
                                        float(c.scale))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_gqa_identical_queries_identical_outputs():
    q = np.random.default_rng(5).standard_normal((2, 32, 128)).astype(np.float32)
    q = q.reshape(2, 8, 4, 128)
    q[:, :, 1:] = q[:, :, :1]
    c = small_case([500, 64], S=4, q_override=W.f32_to_bf16_bits(q.reshape(2, 32, 128)))
    print("[case] GQA identical queries", flush=True)
    out, lse = DevCase(c).attention()
    o = bits_host(out).reshape(2, 8, 4, 128)
    l = lse.cpu().numpy().reshape(2, 8, 4)
    for r in range(1, 4):
        assert np.array_equal(o[:, :, r], o[:, :, 0]) and np.array_equal(l[:, :, r], l[:, :, 0])


def test_split_count_changes_little():
    c = small_case([6000, 300], S=1)
    print("[case] split count sweep", flush=True)
    d = DevCase(c)
    o_ref, l_ref = oracle.case_attention(c)
    for S in [1, 2, 5, 16, 94, 128, 1024]:
        out, lse = d.attention(num_splits=S)
        compare_attention(out, lse, o_ref, l_ref, label=f"S={S}")


def test_split_merge_entry_point():
    c = small_case([2000, 1, 300], S=7)
    print("[case] split-merge entry point", flush=True)
    acc, m, l = oracle.split_partials(c.q, c.k_pages, c.v_pages, c.page_list, c.seq_lens,
                                      num_kv_heads=8, page_size=64, scale=c.scale, num_splits=7)
    acc32, m32, l32 = acc.astype(np.float32), m.astype(np.float32), l.astype(np.float32)
    o_ref, l_ref = oracle.split_merge(acc32, m32, l32)
    out, lse = spa.split_merge(torch.from_numpy(acc32).cuda(), torch.from_numpy(m32).cuda(),
                               torch.from_numpy(l32).cuda())
    torch.cuda.synchronize()
    from tests.gpu_util import bf16_to_f64
    o = bf16_to_f64(out)
    # bf16 rounding of the output (half an ulp) plus fp32 arithmetic
    assert np.all(np.abs(o - o_ref) <= np.abs(o_ref) * 2.0 ** -8 + 1e-6)
    fin = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lse.cpu().numpy()), fin)
    assert np.max(np.abs(lse.cpu().numpy()[fin] - l_ref[fin])) <= 1e-5


def test_split_merge_generic_head_dim():
    rng = np.random.default_rng(3)
    print("[case] split-merge head_dim 72, 33 splits, empty splits", flush=True)
    B, Hq, S, D = 3, 5, 33, 72
    acc = rng.standard_normal((B, Hq, S, D)).astype(np.float32)
    m = rng.standard_normal((B, Hq, S)).astype(np.float32) * 5
    l = rng.uniform(0.5, 3, (B, Hq, S)).astype(np.float32)
    m[0, 0, ::2] = -np.inf; l[0, 0, ::2] = 0; acc[0, 0, ::2] = 0
    m[1, 1, :] = -np.inf; l[1, 1, :] = 0; acc[1, 1, :] = 0
    o_ref, l_ref = oracle.split_merge(acc, m, l)
    out, lse = spa.split_merge(torch.from_numpy(acc).cuda(), torch.from_numpy(m).cuda(),
                               torch.from_numpy(l).cuda())
    torch.cuda.synchronize()
    from tests.gpu_util import bf16_to_f64
    o = bf16_to_f64(out)
    assert np.all(np.abs(o - o_ref) <= np.abs(o_ref) * 2.0 ** -8 + 1e-6)
    ln = lse.cpu().numpy()
    assert np.isneginf(ln[1, 1]) and np.all(o[1, 1] == 0)
    fin = np.isfinite(l_ref)
    assert np.max(np.abs(ln[fin] - l_ref[fin])) <= 1e-5


# ---------------------------------------------------------------- full step + graphs

def test_full_step_config5_metadata_then_attention():
    """The whole hot path on the ragged int8 batch: page table, cache_seqlens
    and cu_seqlens_k built on the device (bit-exact) feed the attention."""
    c = config_case(5)
    print("[case] full step config 5", flush=True)
    d = DevCase(c)
    pt, cache, cu = d.page_table()
    pt_o, cache_o, cu_o = oracle.case_page_table(c)
    torch.cuda.synchronize()
    assert np.array_equal(pt.cpu().numpy(), pt_o)
    assert np.array_equal(cache.cpu().numpy(), cache_o)
    assert np.array_equal(cu.cpu().numpy(), cu_o)
    out, lse = d.attention(page_table=pt)
    o_ref, l_ref = oracle.case_attention(c, page_table=pt_o)
    compare_attention(out, lse, o_ref, l_ref, label="config 5 step")


def _walk_case():
    return small_case(balanced_walk_lens(64, 13).tolist(), kv="bf16", S=16, seed=64)


def _int8_hg_case():
    lens = W._gen(32, 17).integers(1, 3000, size=32).tolist()
    return small_case(lens, kv="int8", S=4, seed=32)


def _bf16_hg_small_case():
    lens = W._gen(8, 23).integers(600, 1025, size=8).tolist()
    return small_case(lens, kv="bf16", S=4, seed=8)   # 256 triples, 4-page splits


@pytest.mark.parametrize("make,kw", [
    (lambda: config_case(3), {}),                     # default: page split, fused merge
    (_bf16_hg_small_case, {}),                        # default: head grouped, fused merge
    (_walk_case, dict(producer="head_grouped", merge="fused")),   # fused with split walks
    (_int8_hg_case, {}),                              # default: 4-head 1-byte, fused merge
], ids=["b8_ctx1k_default", "bf16_hg_small_default", "bf16_walks_fused", "int8_hg_fused_default"])
def test_hip_graph_replay_matches_eager(make, kw):
    c = make()
    print(f"[case] HIP graph capture of the decode step {c.name} {kw}", flush=True)
    d = DevCase(c)
    B, Hq, D, S = c.batch, c.num_q_heads, c.head_dim, c.num_splits
    ws = spa.new_workspace(B, Hq, c.num_kv_heads, D, S)
    pt = torch.empty((B, c.max_seq_pages), dtype=torch.int32, device="cuda")
    cache = torch.empty((B,), dtype=torch.int32, device="cuda")
    cu = torch.empty((B + 1,), dtype=torch.int32, device="cuda")
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")

    def step():
        spa.build_page_table(d.r2t, d.rpi, d.seq_lens, c.page_size, c.max_seq_pages,
                             page_table=pt, cache_seqlens=cache, cu_seqlens_k=cu)
        d.attention(page_table=pt, workspace=ws, out=out, lse=lse, **kw)

    step()
    torch.cuda.synchronize()
    o_eager, l_eager = out.clone(), lse.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(4):
        out.zero_(); lse.zero_(); pt.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), o_eager.view(torch.int16))
        assert torch.equal(lse, l_eager)
        step()   # eager work between replays
        torch.cuda.synchronize()
    assert int(counters_view(ws).abs().sum()) == 0


def test_large_grid_walks_whatever_the_lengths():
    """512 ragged requests, 8 splits: the walked grid spans several rounds of
    resident workgroups, so the producer walks without looking at the
    lengths (the dispatcher evens out the workgroups over the rounds).
    Against the oracle, and bit-exactly against four of the requests alone
    (a grid too small to walk)."""
    lens = W._gen(512, 31).integers(1, 321, size=512)
    lens[:4] = [0, 1, 64, 320]
    c = small_case(lens.tolist(), kv="bf16", S=8, seed=512)
    print("[case] walked grid of several rounds, batch 512 ragged", flush=True)
    d = DevCase(c)
    o_ref, l_ref = oracle.case_attention(c)
    o1, l1 = d.attention(producer="head_grouped", merge="separate")
    compare_attention(o1, l1, o_ref, l_ref, label="batch 512 walked")
    rows = slice(0, 4)
    o2, l2 = spa.paged_decode_attention(d.q[rows].contiguous(), d.k, d.v,
                                        d.page_list[rows].contiguous(), d.seq_lens[rows].contiguous(),
                                        8, float(c.scale), kv_dtype="bf16",
                                        producer="head_grouped", merge="separate")
    torch.cuda.synchronize()
    assert torch.equal(o2.view(torch.int16), o1[rows].view(torch.int16))
    assert torch.equal(l2, l1[rows])


@pytest.mark.parametrize("merge", ["fused", "separate"])
def test_graph_replay_follows_walk_choice(merge):
    """One captured bf16 head-grouped call, replayed while the lengths
    alternate in place between a batch balanced enough to walk and a ragged
    one: the kernel chooses per replay, and every replay equals an eager
    call on the same lengths, bit for bit (the fused merge's arrival
    counters, counted per walk or per split, end at zero)."""
    bal = balanced_walk_lens(64, 21)
    rag = bal.copy()
    rag[8:40] = 1
    assert not walks_balanced(rag)
    c = small_case(bal.tolist(), kv="bf16", S=16, seed=121)
    print(f"[case] graph replay, walk chosen per replay, {merge} merge", flush=True)
    d = DevCase(c)
    B, Hq, D, S = c.batch, c.num_q_heads, c.head_dim, c.num_splits
    ws = spa.new_workspace(B, Hq, c.num_kv_heads, D, S)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    sl = d.seq_lens
    cases = [("balanced", torch.tensor(bal, dtype=torch.int32)),
             ("ragged", torch.tensor(rag, dtype=torch.int32))]

    def call():
        spa.paged_decode_attention(d.q, d.k, d.v, d.page_list, sl, S, float(c.scale),
                                   kv_dtype="bf16", workspace=ws, out=out, lse=lse,
                                   producer="head_grouped", merge=merge)

    eager = {}
    for name, host in cases:
        sl.copy_(host)
        call()
        torch.cuda.synchronize()
        eager[name] = (out.clone(), lse.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(6):
        name, host = cases[i % 2]
        sl.copy_(host)
        out.zero_(); lse.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager[name][0].view(torch.int16)), (i, name)
        assert torch.equal(lse, eager[name][1]), (i, name)
    assert int(counters_view(ws).abs().sum()) == 0


# ---------------------------------------------------------------- other batch and head shapes

@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("producer", PRODUCERS)
@pytest.mark.parametrize("batch", [72, 100])
def test_large_ragged_batches(batch, producer, kv):
    """More than 64 requests (natural request order instead of longest
    first); 72 is a multiple of 8 (request-major XCD placement for 1-byte
    codes), 100 is not."""
    lens = W._gen(batch, 99).integers(1, 2001, size=batch).tolist()
    c = small_case(lens, kv=kv, S=8, seed=batch)
    print(f"[case] batch {batch} ragged {kv} {producer}", flush=True)
    out, lse = DevCase(c).attention(producer=producer)
    o_ref, l_ref = oracle.case_attention(c)
    compare_attention(out, lse, o_ref, l_ref, label=f"batch {batch} {kv} {producer}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("S", [16, 8])
def test_split_walk(S, kv):
    """bf16 and e4m3 head-grouped grids large enough that a workgroup walks several
    consecutive splits (states of all but the last kept in LDS until the
    workgroup ends), on a batch balanced enough to walk: empty and one-token
    requests, exact page multiples and splits past the context inside a
    walk.  Checked against the oracle; the fused launch (which walks too, a
    group's splits arriving as its walks) bit-exactly against the separate
    one.  A walk changes no split's arithmetic, so these rows are bit-equal
    to the same requests in calls that do not walk: a batch made ragged by
    cutting other requests to one token, and four requests alone (a grid
    too small to walk)."""
    lens = balanced_walk_lens(64, 7)
    c = small_case(lens.tolist(), kv=kv, S=S, seed=64 + S)
    print(f"[case] split walk S={S} {kv} batch 64 balanced", flush=True)
    d = DevCase(c)
    o_ref, l_ref = oracle.case_attention(c)
    o1, l1 = d.attention(producer="head_grouped", merge="separate")
    compare_attention(o1, l1, o_ref, l_ref, label=f"walk S={S} {kv}")
    o2, l2 = d.attention(producer="head_grouped", merge="fused")
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    ragged = lens.copy()
    ragged[8:40] = 1
    assert not walks_balanced(ragged)
    sl = torch.tensor(ragged, dtype=torch.int32, device="cuda")
    keep = list(range(8)) + list(range(40, 64))
    for merge in ("separate", "fused"):
        o3, l3 = spa.paged_decode_attention(d.q, d.k, d.v, d.page_list, sl, S, float(c.scale),
                                            kv_dtype=kv, k_scales=d.ks, v_scales=d.vs,
                                            producer="head_grouped", merge=merge)
        torch.cuda.synchronize()
        assert torch.equal(o3[keep].view(torch.int16), o1[keep].view(torch.int16)), merge
        assert torch.equal(l3[keep], l1[keep]), merge
    # lengths 65, 4096, 4095, 129: 4 x 4 kv-head blocks x S workgroups (at
    # most 256) is one per CU at most, a grid no walk shortens
    rows = slice(4, 8)
    o3, l3 = spa.paged_decode_attention(d.q[rows].contiguous(), d.k, d.v,
                                        d.page_list[rows].contiguous(), d.seq_lens[rows].contiguous(),
                                        S, float(c.scale), kv_dtype=kv, k_scales=d.ks,
                                        v_scales=d.vs, producer="head_grouped", merge="separate")
    torch.cuda.synchronize()
    assert torch.equal(o3.view(torch.int16), o1[rows].view(torch.int16))
    assert torch.equal(l3, l1[rows])


@pytest.mark.parametrize("S", [16, 8])
def test_ragged_batch_does_not_walk(S):
    """A ragged bf16 batch of the same grid size (the longest request far
    above the mean) takes one split per workgroup: checked against the
    oracle for both merges."""
    rng = W._gen(64, 8)
    lens = rng.integers(1, 4097, size=64)
    lens[:4] = [0, 4096, 64, 65]
    assert not walks_balanced(lens)
    c = small_case(lens.tolist(), kv="bf16", S=S, seed=90 + S)
    print(f"[case] ragged no-walk S={S} batch 64", flush=True)
    d = DevCase(c)
    o_ref, l_ref = oracle.case_attention(c)
    for merge in ("separate", "fused"):
        out, lse = d.attention(producer="head_grouped", merge=merge)
        compare_attention(out, lse, o_ref, l_ref, label=f"ragged S={S} {merge}")


@pytest.mark.parametrize("Hkv", [1, 2, 6, 16])
@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_other_kv_head_counts(Hkv, kv):
    """Group size 4 with 1, 2, 6 or 16 kv heads (head-grouped needs an even
    count; one kv head takes the page-split producer)."""
    c = small_case([700, 64, 1500, 9], kv=kv, S=4, Hkv=Hkv)
    print(f"[case] Hkv={Hkv} {kv}", flush=True)
    d = DevCase(c)
    o_ref, l_ref = oracle.case_attention(c)
    for producer in (["page_split"] if Hkv % 2 else PRODUCERS):
        for merge in ("fused", "separate"):
            out, lse = d.attention(producer=producer, merge=merge)
            compare_attention(out, lse, o_ref, l_ref, label=f"Hkv {Hkv} {kv} {producer} {merge}")
