"""GPU parity for multi-token query decode (target verify / draft extend)
against the fp64 oracle, through the C ABI; same tolerances as the one-token
decode (tests/gpu_util.py)."""
import numpy as np
import pytest
import torch

import oracle
import split_paged_attention_amd as spa
import workloads as W
from tests.gpu_util import (DevCase, balanced_walk_lens, bf16_dev, compare_attention, config_case,
                            walks_balanced)

pytestmark = pytest.mark.gpu


def small_case(lens, kv="bf16", S=4, seed=31, Hkv=8):
    P = 64
    need = sum(-(-L // P) for L in lens)
    msp = max(1, max(-(-L // P) for L in lens))
    return W.make_case(seed=seed, seq_lens=lens, num_pages=need + 3, num_splits=S, kv_dtype=kv,
                       num_q_heads=4 * Hkv, num_kv_heads=Hkv, head_dim=128, page_size=P,
                       req_pool_rows=max(4, len(lens)), req_to_token_stride=msp * P,
                       max_seq_pages=msp, name=f"verify{lens}_{kv}_S{S}")


def run_verify(c, q_rows, cu, S=None, page_table=None, cu_dev=None, max_q_len=4):
    d = DevCase(c)
    pt = d.page_list if page_table is None else page_table
    cu_d = torch.from_numpy(cu).cuda() if cu_dev is None else cu_dev
    out, lse = spa.paged_verify_attention(
        bf16_dev(q_rows), d.k, d.v, pt, d.seq_lens, cu_d, c.num_splits if S is None else S,
        float(c.scale), max_q_len=max_q_len, kv_dtype=c.kv_dtype, k_scales=d.ks, v_scales=d.vs)
    torch.cuda.synchronize()
    return out, lse


def oracle_verify(c, q_rows, cu):
    return oracle.verify_attention(q_rows, c.k_pages, c.v_pages, c.page_list, c.seq_lens, cu,
                                   num_kv_heads=c.num_kv_heads, page_size=c.page_size,
                                   scale=c.scale, kv_dtype=c.kv_dtype, k_scales=c.k_scales,
                                   v_scales=c.v_scales)


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("lens,qlens,S", [
    ([20, 9, 33, 300, 1000], [4, 1, 3, 2, 4], 4),
    ([64, 65, 128, 2000], [4, 4, 4, 4], 16),       # draft rows across page / split edges
    ([1, 4, 700, 5], [1, 4, 2, 0], 3),             # a request with no query rows
    ([4096, 3, 129], [3, 3, 1], 64),               # many empty splits
])
def test_verify_parity(kv, lens, qlens, S):
    c = small_case(lens, kv=kv, S=S)
    q_rows, cu = W.verify_queries(c, qlens)
    print(f"[case] verify {kv} lens={lens} qlens={qlens} S={S}", flush=True)
    out, lse = run_verify(c, q_rows, cu)
    o_ref, l_ref = oracle_verify(c, q_rows, cu)
    compare_attention(out, lse, o_ref, l_ref, label=f"verify {kv} {lens}")


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
@pytest.mark.parametrize("lens,qlens,S", [
    ([70, 6, 1290, 4000], [6, 6, 5, 6], 4),        # 6 rows: a step with 5 draft tokens
    ([64, 65, 2000, 8], [8, 7, 8, 8], 16),         # two row blocks across page / split edges
    ([4096, 3, 129, 700], [5, 3, 8, 0], 64),       # many empty splits; a request with no rows
])
def test_verify_parity_up_to_eight_rows(kv, lens, qlens, S):
    """5 to 8 query rows per request: one workgroup takes 8 query tokens (two
    row blocks sharing every K and V operand)."""
    c = small_case(lens, kv=kv, S=S, seed=57)
    q_rows, cu = W.verify_queries(c, qlens)
    print(f"[case] verify {kv} lens={lens} qlens={qlens} S={S} max_q_len 8", flush=True)
    out, lse = run_verify(c, q_rows, cu, max_q_len=8)
    o_ref, l_ref = oracle_verify(c, q_rows, cu)
    compare_attention(out, lse, o_ref, l_ref, label=f"verify8 {kv} {lens}")


@pytest.mark.parametrize("Hkv", [2, 6, 4])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_verify_kv_head_counts(kv, Hkv):
    """Workgroups of 2 kv heads (2 or 6 kv heads) and of 4 (4 kv heads),
    with 4 and with 6 query rows per request."""
    c = small_case([700, 64, 1500, 9], kv=kv, S=4, seed=61, Hkv=Hkv)
    for qlens, mq in (([4, 2, 3, 1], 4), ([6, 5, 2, 6], 8)):
        q_rows, cu = W.verify_queries(c, qlens)
        print(f"[case] verify Hkv={Hkv} {kv} qlens={qlens}", flush=True)
        out, lse = run_verify(c, q_rows, cu, max_q_len=mq)
        o_ref, l_ref = oracle_verify(c, q_rows, cu)
        compare_attention(out, lse, o_ref, l_ref, label=f"verify Hkv={Hkv} {kv} {qlens}")


@pytest.mark.parametrize("kv", ["bf16", "int8", "fp8"])
def test_verify_more_rows_than_one_workgroup_takes(kv):
    """Up to 20 query rows per request: chunks of 8 tokens, each chunk a grid
    slice of its own reading the request's K and V."""
    c = small_case([300, 40, 2000, 20], kv=kv, S=8, seed=58)
    qlens = [20, 9, 13, 17]
    q_rows, cu = W.verify_queries(c, qlens)
    print(f"[case] verify {kv} qlens={qlens} max_q_len 20 (chunks)", flush=True)
    out, lse = run_verify(c, q_rows, cu, max_q_len=20)
    o_ref, l_ref = oracle_verify(c, q_rows, cu)
    compare_attention(out, lse, o_ref, l_ref, label=f"verify chunks {kv}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("max_q_len,qlens", [(4, [6, 2, 4]), (8, [10, 8, 3]), (3, [5, 3, 1])])
def test_verify_rows_past_max_q_len(kv, max_q_len, qlens):
    """A request with more query rows in the device data than the declared
    max_q_len: its first max_q_len rows are computed with the causal limits
    of all its rows (they match the oracle's), the rest get out = 0 and
    lse = -inf."""
    c = small_case([500, 90, 1400], kv=kv, S=4, seed=59)
    q_rows, cu = W.verify_queries(c, qlens)
    print(f"[case] verify {kv} qlens={qlens} past max_q_len {max_q_len}", flush=True)
    d = DevCase(c)
    T = q_rows.shape[0]
    ws = torch.empty(spa.verify_workspace_bytes(T, 32, 8, 128, 4), dtype=torch.uint8,
                     device="cuda")
    ws.view(torch.float32).fill_(float("nan"))     # stale state must not be what is read
    out, lse = spa.paged_verify_attention(
        bf16_dev(q_rows), d.k, d.v, d.page_list, d.seq_lens, torch.from_numpy(cu).cuda(), 4,
        float(c.scale), max_q_len=max_q_len, kv_dtype=c.kv_dtype, k_scales=d.ks, v_scales=d.vs,
        workspace=ws)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle_verify(c, q_rows, cu)
    inside = np.concatenate([np.arange(n) < max_q_len for n in qlens])
    compare_attention(out[torch.from_numpy(inside).cuda()], lse[torch.from_numpy(inside).cuda()],
                      o_ref[inside], l_ref[inside], label=f"verify rows <= max_q_len {kv}")
    past = torch.from_numpy(~inside).cuda()
    assert torch.isneginf(lse[past]).all() and (out[past].float() == 0).all()


def test_verify_headline_shape_six_query_tokens():
    """Batch 32, context 8K, 6 query tokens per request (a speculative step
    with 5 draft tokens): every output against the oracle."""
    c = config_case(4)
    q_rows, cu = W.verify_queries(c, [6] * c.batch)
    print("[case] verify batch 32 / 8K / 6 tokens", flush=True)
    d = DevCase(c)
    pt, _, _ = d.page_table()
    out, lse = run_verify(c, q_rows, cu, page_table=pt, max_q_len=6)
    o_ref, l_ref = oracle_verify(c, q_rows, cu)
    compare_attention(out, lse, o_ref, l_ref, label="verify b32 8K q6")


def test_verify_headline_shape_four_draft_tokens():
    """Batch 32, context 8K, 4 query tokens per request (draft rows at the end
    of each context): every output against the oracle."""
    c = config_case(4)
    q_rows, cu = W.verify_queries(c, [4] * c.batch)
    print("[case] verify batch 32 / 8K / 4 tokens", flush=True)
    d = DevCase(c)
    pt, _, _ = d.page_table()
    out, lse = run_verify(c, q_rows, cu, page_table=pt)
    o_ref, l_ref = oracle_verify(c, q_rows, cu)
    compare_attention(out, lse, o_ref, l_ref, label="verify b32 8K q4")


def test_verify_consumes_metadata_cu_seqlens_q():
    """The metadata build's strided and cumsum modes produce the
    cu_seqlens_q the verify call reads, on the device."""
    c = small_case([200, 77, 513, 64], kv="bf16", S=4)
    d = DevCase(c)
    print("[case] verify with cu_seqlens_q from the metadata kernel", flush=True)
    for mode, qlens in ((spa.Q_MODE_STRIDED, [3, 3, 3, 3]), (spa.Q_MODE_CUMSUM, [4, 1, 2, 3])):
        q_rows, cu = W.verify_queries(c, qlens)
        md = spa.build_metadata(d.r2t, d.rpi, d.seq_lens, c.page_size, c.max_seq_pages,
                                q_mode=mode, q_stride=3,
                                qlens=torch.tensor(qlens, dtype=torch.int32, device="cuda"))
        out, lse = run_verify(c, q_rows, cu, page_table=md["page_table"],
                              cu_dev=md["cu_seqlens_q"])
        assert np.array_equal(md["cu_seqlens_q"].cpu().numpy(), cu)
        o_ref, l_ref = oracle_verify(c, q_rows, cu)
        compare_attention(out, lse, o_ref, l_ref, label=f"verify q_mode {mode}")


def test_verify_queries_with_nothing_visible():
    """A request shorter than its query count: its first rows see no token
    (out 0, lse -inf)."""
    c = small_case([2, 40], kv="bf16", S=2)
    c.seq_lens[0] = 2
    q_rows, cu = W.verify_queries(c, [2, 4])
    cu = np.array([0, 4, 8], np.int32)              # request 0 claims 4 rows, 2 tokens
    q_rows = np.concatenate([q_rows[:2], q_rows[:2], q_rows[2:]])
    print("[case] verify rows with no visible token", flush=True)
    out, lse = run_verify(c, q_rows, cu)
    o_ref, l_ref = oracle_verify(c, q_rows, cu)
    assert np.isneginf(l_ref[:2]).all()
    compare_attention(out, lse, o_ref, l_ref, label="verify empty rows")
    assert torch.isneginf(lse[:2]).all() and (out[:2].float() == 0).all()


def test_verify_single_token_rows_match_decode_within_tolerance():
    c = small_case([900, 33, 4000], kv="int8", S=8)
    q_rows, cu = W.verify_queries(c, [1, 1, 1])
    print("[case] verify q_len 1 vs decode", flush=True)
    out, lse = run_verify(c, q_rows, cu, max_q_len=1)
    o_ref, l_ref = oracle_verify(c, q_rows, cu)
    compare_attention(out, lse, o_ref, l_ref, label="verify q1")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("batch", [72, 37])
def test_verify_large_batches(batch, kv):
    rng = W._gen(batch, 98)
    lens = rng.integers(4, 1500, size=batch).tolist()
    qlens = rng.integers(0, 5, size=batch).tolist()
    c = small_case(lens, kv=kv, S=6, seed=batch)
    q_rows, cu = W.verify_queries(c, qlens)
    print(f"[case] verify batch {batch} {kv}", flush=True)
    out, lse = run_verify(c, q_rows, cu)
    o_ref, l_ref = oracle_verify(c, q_rows, cu)
    compare_attention(out, lse, o_ref, l_ref, label=f"verify batch {batch} {kv}")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("S", [16, 8])
def test_verify_split_walk(S, kv):
    """bf16 and e4m3 grids large enough that a workgroup walks several
    consecutive splits (states of all but the last held in LDS until the
    workgroup ends), on 64 requests balanced enough to walk, with 0-4 query rows, an
    empty context, exact page multiples and splits past the context inside
    a walk; then the same queries over a ragged batch (other requests cut
    short), which takes one split per workgroup: the rows of the requests
    both calls share are bit-equal."""
    rng = W._gen(64, 11)
    lens = balanced_walk_lens(64, 12)
    lens[0] = 4            # (an empty context would leave no room for query rows)
    qlens = rng.integers(0, 5, size=64)
    qlens[:4] = [4, 0, 1, 4]
    qlens = np.minimum(qlens, lens).tolist()
    c = small_case(lens.tolist(), kv=kv, S=S, seed=80 + S)
    q_rows, cu = W.verify_queries(c, qlens)
    print(f"[case] verify split walk S={S} {kv} batch 64 balanced", flush=True)
    out, lse = run_verify(c, q_rows, cu)
    o_ref, l_ref = oracle_verify(c, q_rows, cu)
    compare_attention(out, lse, o_ref, l_ref, label=f"verify walk S={S} {kv}")
    ragged = lens.copy()
    ragged[8:40] = np.maximum(np.asarray(qlens[8:40]), 1)
    assert not walks_balanced(ragged)
    d = DevCase(c)
    out2, lse2 = spa.paged_verify_attention(
        bf16_dev(q_rows), d.k, d.v, d.page_list, torch.tensor(ragged, dtype=torch.int32).cuda(),
        torch.from_numpy(cu).cuda(), S, float(c.scale), max_q_len=4, kv_dtype=kv,
        k_scales=d.ks, v_scales=d.vs)
    torch.cuda.synchronize()
    cu_h = np.asarray(cu)
    keep = np.concatenate([np.arange(cu_h[b], cu_h[b + 1]) for b in list(range(8)) + list(range(40, 64))])
    keep = torch.from_numpy(keep).cuda()
    assert torch.equal(out2[keep].view(torch.int16), out[keep].view(torch.int16))
    assert torch.equal(lse2[keep], lse[keep])


def test_verify_large_grid_walks_whatever_the_lengths():
    """1024 ragged bf16 requests with 1-4 query rows, 8 splits: the walked
    grid spans several rounds of resident workgroups, so the kernel walks
    without looking at the lengths.  Against the oracle on every output."""
    rng = W._gen(1024, 41)
    lens = rng.integers(4, 321, size=1024)
    lens[:3] = [4, 64, 320]
    qlens = np.minimum(rng.integers(1, 5, size=1024), lens).tolist()
    c = small_case(lens.tolist(), kv="bf16", S=8, seed=1024)
    q_rows, cu = W.verify_queries(c, qlens)
    print("[case] verify walked grid of several rounds, batch 1024 ragged", flush=True)
    out, lse = run_verify(c, q_rows, cu)
    o_ref, l_ref = oracle_verify(c, q_rows, cu)
    compare_attention(out, lse, o_ref, l_ref, label="verify batch 1024 walked")


def test_verify_graph_replay_matches_eager():
    """Captured once, replayed with the query rows changed in place: every
    replay equals an eager call on the same inputs, bit for bit."""
    c = small_case([300, 1200, 64, 900], kv="bf16", S=4)
    q_rows, cu = W.verify_queries(c, [4, 2, 3, 1])
    d = DevCase(c)
    q = bf16_dev(q_rows)
    cu_d = torch.from_numpy(cu).cuda()
    T = q.shape[0]
    ws = torch.empty(spa.verify_workspace_bytes(T, 32, 8, 128, 4), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, 32, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((T, 32), dtype=torch.float32, device="cuda")

    def call(o, l):
        spa.paged_verify_attention(q, d.k, d.v, d.page_list, d.seq_lens, cu_d, 4, float(c.scale),
                                   workspace=ws, out=o, lse=l)

    print("[case] verify graph replay", flush=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(out, lse)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse)
    rng = np.random.default_rng(3)
    for rep in range(3):
        new = W.f32_to_bf16_bits(rng.standard_normal(q_rows.shape).astype(np.float32))
        q.copy_(bf16_dev(new))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_g, l_g = out.clone(), lse.clone()
        o_e = torch.empty_like(out)
        l_e = torch.empty_like(lse)
        call(o_e, l_e)
        torch.cuda.synchronize()
        assert torch.equal(o_g.view(torch.int16), o_e.view(torch.int16)) and torch.equal(l_g, l_e)
