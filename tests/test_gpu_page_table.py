"""GPU parity for the metadata build: bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import split_paged_attention_amd as spa
from tests.gpu_util import DevCase, config_case

pytestmark = pytest.mark.gpu


def _run_both(r2t, rpi, sl, P, msp, off=0, pt_cols=None, preset=-7):
    bs = rpi.shape[0]
    cols = msp if pt_cols is None else pt_cols
    pt_h = np.full((bs, max(cols, 1)), preset, np.int32)
    pt_o, cache_o, cu_o = oracle.build_page_table(r2t, rpi, sl, P, msp, seqlen_offset=off,
                                                  page_table=pt_h.copy())
    pt_d = torch.from_numpy(pt_h.copy()).cuda()
    cache_d = torch.full((bs,), -7, dtype=torch.int32, device="cuda")
    cu_d = torch.full((bs + 1,), -7, dtype=torch.int32, device="cuda")
    spa.build_page_table(torch.from_numpy(r2t).cuda(), torch.from_numpy(rpi).cuda(),
                         torch.from_numpy(sl).cuda(), P, msp, seqlen_offset=off,
                         page_table=pt_d, cache_seqlens=cache_d, cu_seqlens_k=cu_d)
    torch.cuda.synchronize()
    return (pt_o, cache_o, cu_o), (pt_d.cpu().numpy(), cache_d.cpu().numpy(), cu_d.cpu().numpy())


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_page_table_configs_bit_exact(cfg):
    c = config_case(cfg)
    print(f"[case] page_table config {cfg}", flush=True)
    ref, got = _run_both(c.req_to_token, c.req_pool_indices, c.seq_lens, c.page_size,
                         c.max_seq_pages)
    for r, g in zip(ref, got):
        assert np.array_equal(r, g)


def test_page_table_edge_maps():
    rng = np.random.default_rng(7)
    print("[case] page_table edges: negative slots, offset, wide stride, P=48", flush=True)
    # negative slots (floor division), seqlen_offset, untouched columns past max_seq_pages
    r2t = rng.integers(-500, 5000, size=(16, 4096), dtype=np.int64).astype(np.int32)
    rpi = rng.choice(16, 11, replace=False).astype(np.int32)
    sl = rng.integers(0, 4000, size=11).astype(np.int32)
    for P, msp, cols, off in [(64, 60, 64, 0), (48, 80, 100, 3), (1, 600, 700, -2),
                              (7, 500, 500, 1)]:
        ref, got = _run_both(r2t, rpi, sl, P, msp, off=off, pt_cols=cols)
        for r, g in zip(ref, got):
            assert np.array_equal(r, g), (P, msp, cols, off)


def test_page_table_large_batch_scan():
    rng = np.random.default_rng(8)
    print("[case] page_table bs=1000 (multi-chunk scan)", flush=True)
    r2t = rng.integers(0, 1 << 20, size=(1024, 256), dtype=np.int64).astype(np.int32)
    rpi = rng.integers(0, 1024, size=1000).astype(np.int32)
    sl = rng.integers(0, 1 << 20, size=1000).astype(np.int32)
    ref, got = _run_both(r2t, rpi, sl, 16, 16, off=5)
    for r, g in zip(ref, got):
        assert np.array_equal(r, g)


def test_page_table_bs0_writes_nothing():
    print("[case] page_table bs=0", flush=True)
    r2t = torch.zeros((4, 64), dtype=torch.int32, device="cuda")
    cu = torch.full((1,), 99, dtype=torch.int32, device="cuda")
    pt = torch.full((0, 4), 99, dtype=torch.int32, device="cuda")
    spa.build_page_table(r2t, torch.zeros(0, dtype=torch.int32, device="cuda"),
                         torch.zeros(0, dtype=torch.int32, device="cuda"), 16, 4,
                         page_table=pt, cu_seqlens_k=cu)
    torch.cuda.synchronize()
    assert cu.item() == 99


def test_page_table_matches_generator_placement_on_device():
    c = config_case(5)
    print("[case] page_table vs generator placement, config 5", flush=True)
    pt, cache, cu = DevCase(c).page_table()
    pt = pt.cpu().numpy()
    for b in range(c.batch):
        npg = -(-int(c.seq_lens[b]) // c.page_size)
        assert np.array_equal(pt[b, :npg], c.page_list[b, :npg])
