"""GPU parity for the full metadata update (cu_seqlens_q modes, sliding-window
page table, swa_out_cache_loc): bit-exact against the oracle on every
output, including the entries a call must leave untouched."""
import numpy as np
import pytest
import torch

import oracle
import split_paged_attention_amd as spa
from tests.gpu_util import config_case

pytestmark = pytest.mark.gpu

PRESET = -7


def swa_mapping(n_slots, page_size, resident, swa_slots, seed):
    """full_to_swa of length n_slots + page_size + 1: a random `resident`
    fraction of slots maps to distinct sliding-window slots, the rest to -1."""
    rng = np.random.default_rng(seed)
    m = np.full(n_slots + page_size + 1, -1, np.int64)
    live = rng.random(n_slots) < resident
    idx = np.flatnonzero(live)
    m[idx] = rng.choice(swa_slots, size=idx.size, replace=idx.size > swa_slots)
    return m


def run_both(r2t, rpi, sl, P, msp, *, off=0, pt_cols=None, q_mode=0, qlens=None, q_stride=0,
             swa=None, swa_table=False, ocl=None, swa_out_len=None):
    bs = rpi.shape[0]
    cols = max(msp if pt_cols is None else pt_cols, 1)
    pt_h = np.full((bs, cols), PRESET, np.int32)
    spt_h = np.full((bs, cols + 3), PRESET, np.int32) if swa_table else None
    cuq_h = np.full(bs + 1, PRESET, np.int32)
    sout_h = None if swa_out_len is None else np.full(swa_out_len, PRESET, np.int64)
    ref = oracle.build_metadata(
        r2t, rpi, sl, P, msp, seqlen_offset=off, page_table=pt_h.copy(), q_mode=q_mode,
        qlens=qlens, q_stride=q_stride, cu_seqlens_q=cuq_h.copy(), swa_mapping=swa,
        swa_page_table=None if spt_h is None else spt_h.copy(), out_cache_loc=ocl,
        swa_out_cache_loc=None if sout_h is None else sout_h.copy())

    def dev(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda()

    got = spa.build_metadata(
        dev(r2t), dev(rpi), dev(sl), P, msp, seqlen_offset=off, page_table=dev(pt_h),
        cache_seqlens=dev(np.full(bs, PRESET, np.int32)),
        cu_seqlens_k=dev(np.full(bs + 1, PRESET, np.int32)), q_mode=q_mode, qlens=dev(qlens),
        q_stride=q_stride, cu_seqlens_q=dev(cuq_h), full_to_swa=dev(swa),
        swa_page_table=dev(spt_h), out_cache_loc=dev(ocl), swa_out_cache_loc=dev(sout_h))
    torch.cuda.synchronize()
    for k in ("page_table", "cache_seqlens", "cu_seqlens_k", "cu_seqlens_q", "swa_page_table",
              "swa_out_cache_loc"):
        r, g = ref[k], got[k]
        if r is None:
            assert g is None, k
            continue
        g = g.cpu().numpy()
        assert np.array_equal(r, g), (k, np.flatnonzero(r.ravel() != g.ravel())[:8])
    return ref


@pytest.mark.parametrize("cfg", [1, 3, 4, 5])
@pytest.mark.parametrize("q_mode", [0, 1, 2])
def test_metadata_configs_all_outputs_bit_exact(cfg, q_mode):
    c = config_case(cfg)
    print(f"[case] metadata config {cfg} q_mode {q_mode}", flush=True)
    rng = np.random.default_rng(100 * cfg + q_mode)
    n_slots = c.num_pages * c.page_size
    swa = swa_mapping(n_slots, c.page_size, 0.5, n_slots // 4, seed=cfg)
    qlens = rng.integers(1, 8, size=c.batch).astype(np.int32)
    ocl = rng.integers(-1, n_slots, size=c.batch * 3).astype(np.int64)
    ref = run_both(c.req_to_token, c.req_pool_indices, c.seq_lens, c.page_size,
                   c.max_seq_pages, off=1, q_mode=q_mode, qlens=qlens, q_stride=3, swa=swa,
                   swa_table=True, ocl=ocl, swa_out_len=c.batch * 4 + 5)
    # the sliding-window table must actually hold both kinds of entry
    spt = ref["swa_page_table"][:, :c.max_seq_pages]
    assert (spt == -1).any() and (spt >= 0).any()


def test_metadata_swa_out_multi_tile_and_negative_locs():
    print("[case] metadata swa_out 5000 entries, 3333 real, negative locs", flush=True)
    rng = np.random.default_rng(3)
    swa = swa_mapping(1 << 16, 64, 0.7, 1 << 14, seed=3)
    ocl = rng.integers(-50, 1 << 16, size=3333).astype(np.int64)
    r2t = rng.integers(0, 1 << 16, size=(4, 512), dtype=np.int64).astype(np.int32)
    rpi = np.array([3, 1], np.int32)
    sl = np.array([100, 200], np.int32)
    ref = run_both(r2t, rpi, sl, 64, 8, swa=swa, ocl=ocl, swa_out_len=5000)
    s = ref["swa_out_cache_loc"]
    assert (s[:3333][ocl < 0] == -1).all() and (s[3333:] == 0).all()


def test_metadata_out_cache_loc_longer_than_swa_out():
    print("[case] metadata out_cache_loc longer than swa_out_cache_loc", flush=True)
    rng = np.random.default_rng(4)
    swa = swa_mapping(4096, 16, 0.5, 1024, seed=4)
    r2t = rng.integers(0, 4096, size=(2, 64), dtype=np.int64).astype(np.int32)
    ocl = rng.integers(0, 4096, size=1500).astype(np.int64)
    run_both(r2t, np.array([1], np.int32), np.array([7], np.int32), 16, 4, swa=swa, ocl=ocl,
             swa_out_len=1030)


def test_metadata_swa_out_without_out_cache_loc_zero_pads():
    print("[case] metadata swa_out without out_cache_loc", flush=True)
    r2t = np.arange(128, dtype=np.int32).reshape(2, 64)
    ref = run_both(r2t, np.array([0, 1], np.int32), np.array([3, 9], np.int32), 16, 4,
                   swa_out_len=2049)
    assert (ref["swa_out_cache_loc"] == 0).all()


def test_metadata_negative_slots_and_mapped_negatives():
    print("[case] metadata negative slots and negative mapped slots", flush=True)
    rng = np.random.default_rng(5)
    r2t = rng.integers(-300, 3000, size=(8, 2048), dtype=np.int64).astype(np.int32)
    swa = rng.integers(-20, 999, size=3000 + 64 + 1).astype(np.int64)
    rpi = rng.integers(0, 8, size=13).astype(np.int32)
    sl = rng.integers(0, 2048, size=13).astype(np.int32)
    for P, msp, cols in [(64, 32, 40), (48, 40, 40), (1, 600, 700), (7, 250, 260)]:
        run_both(r2t, rpi, sl, P, msp, off=-2, pt_cols=cols, swa=swa, swa_table=True)


def test_metadata_large_batch_cumsum_and_wrap():
    print("[case] metadata bs=1000 cumsum; strided wrap", flush=True)
    rng = np.random.default_rng(6)
    r2t = rng.integers(0, 1 << 20, size=(1024, 256), dtype=np.int64).astype(np.int32)
    rpi = rng.integers(0, 1024, size=1000).astype(np.int32)
    sl = rng.integers(0, 1 << 20, size=1000).astype(np.int32)
    qlens = rng.integers(0, 1 << 22, size=1000).astype(np.int32)   # cumsum wraps int32
    run_both(r2t, rpi, sl, 16, 16, off=5, q_mode=1, qlens=qlens)
    run_both(r2t, rpi, sl, 16, 16, q_mode=2, q_stride=2**30 + 7)


def test_metadata_bs0_writes_nothing():
    print("[case] metadata bs=0", flush=True)
    z = torch.zeros(0, dtype=torch.int32, device="cuda")
    sout = torch.full((9,), 99, dtype=torch.int64, device="cuda")
    cuq = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    spa.build_metadata(torch.zeros((4, 64), dtype=torch.int32, device="cuda"), z, z, 16, 4,
                       q_mode=2, q_stride=4, cu_seqlens_q=cuq,
                       full_to_swa=torch.zeros(64, dtype=torch.int64, device="cuda"),
                       out_cache_loc=torch.zeros(9, dtype=torch.int64, device="cuda"),
                       swa_out_cache_loc=sout)
    torch.cuda.synchronize()
    assert (sout == 99).all() and cuq.item() == 99


def test_metadata_graph_replay_tracks_new_inputs():
    """The update exists to run inside a replayed graph: capture it once on
    fixed buffers, then change the inputs in place between replays (with
    eager work in between) and check every replay against the oracle."""
    c = config_case(3)
    print("[case] metadata graph replay x4, config 3 shapes", flush=True)
    P, msp, bs = c.page_size, c.max_seq_pages, c.batch
    n_slots = c.num_pages * P
    rng = np.random.default_rng(9)
    r2t = torch.from_numpy(c.req_to_token).cuda()
    rpi = torch.from_numpy(c.req_pool_indices).cuda()
    sl = torch.from_numpy(c.seq_lens).cuda()
    qlens = torch.ones(bs, dtype=torch.int32, device="cuda")
    swa = torch.from_numpy(swa_mapping(n_slots, P, 0.5, n_slots // 4, seed=9)).cuda()
    ocl = torch.zeros(bs * 2, dtype=torch.int64, device="cuda")
    outs = dict(page_table=torch.zeros((bs, msp), dtype=torch.int32, device="cuda"),
                cache_seqlens=torch.zeros(bs, dtype=torch.int32, device="cuda"),
                cu_seqlens_k=torch.zeros(bs + 1, dtype=torch.int32, device="cuda"),
                cu_seqlens_q=torch.zeros(bs + 1, dtype=torch.int32, device="cuda"),
                swa_page_table=torch.zeros((bs, msp), dtype=torch.int32, device="cuda"),
                swa_out_cache_loc=torch.zeros(bs * 3, dtype=torch.int64, device="cuda"))

    def call():
        spa.build_metadata(r2t, rpi, sl, P, msp, seqlen_offset=2, q_mode=1, qlens=qlens,
                           full_to_swa=swa, out_cache_loc=ocl, **outs)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for rep in range(4):
        rpi.copy_(torch.from_numpy(rng.permutation(c.req_pool_indices)))
        sl.copy_(torch.from_numpy(rng.integers(1, 1024, size=bs).astype(np.int32)))
        qlens.copy_(torch.from_numpy(rng.integers(1, 6, size=bs).astype(np.int32)))
        swa.copy_(torch.from_numpy(swa_mapping(n_slots, P, 0.3 + 0.1 * rep, n_slots // 4,
                                               seed=rep)))
        ocl.copy_(torch.from_numpy(rng.integers(-1, n_slots, size=bs * 2).astype(np.int64)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = oracle.build_metadata(
            c.req_to_token, rpi.cpu().numpy(), sl.cpu().numpy(), P, msp, seqlen_offset=2,
            q_mode=1, qlens=qlens.cpu().numpy(), swa_mapping=swa.cpu().numpy(),
            swa_page_table=True, out_cache_loc=ocl.cpu().numpy(),
            swa_out_cache_loc=np.zeros(bs * 3, np.int64))
        for k, t in outs.items():
            assert np.array_equal(ref[k], t.cpu().numpy()), (rep, k)
