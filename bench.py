"""Benchmark of the split-K paged-attention decode step on one MI355X.

One step = the whole hot path on one batch: the page table / cache_seqlens /
cu_seqlens_k build (one launch) followed by split-K paged-attention decode
(one launch, producer + fused log-sum-exp merge).  Default workload: batch 32,
context 8192, 32 query / 8 KV heads, head_dim 128, bf16 K/V in 64-token pages
scattered over a 4096-page pool, 16 splits -- lmdeploy's headline H200 shape.

Timing: W untimed warm-up steps, then exactly K steps between two device
synchronisations; HIP events on the launch stream bracket every attention
launch, giving the attention kernel's average duration.  Two copies of the KV
pool alternate so that consecutive steps do not read the same addresses.  A
HIP-graph replay of the step is timed as well (the pages quote CUDA-graph
latency).  The fp64 CPU oracle is timed on the host beside it.

Prints ONE JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E peak, GB/s


def _traffic_for(kernel_file: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        src = open(os.path.join(ROOT, "split_paged_attention_amd", "csrc", kernel_file), "rb").read()
        if rec.get("kernel_source_sha256") != hashlib.sha256(src).hexdigest():
            return None
        return int(rec["hbm_bytes_per_launch"])
    except Exception:
        return None


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=4, help="workload 1..5 (4 = headline)")
    ap.add_argument("--graph-replays", type=int, default=200)
    ap.add_argument("--cpu-reps", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(batch rows and KV heads shard with no exchange; see DESIGN.md).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import split_paged_attention_amd as spa
    import workloads as W

    torch.cuda.set_device(0)
    spa.lib()  # fail loudly if the HIP library is missing
    t_gen = time.time()
    case = W.make_config(args.config)
    gen_s = time.time() - t_gen
    dev = "cuda:0"

    def bf16(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
            torch.bfloat16)

    q = bf16(case.q)
    if case.kv_dtype == "bf16":
        k0, v0 = bf16(case.k_pages), bf16(case.v_pages)
        ks0 = vs0 = None
    else:
        k0 = torch.from_numpy(case.k_pages).to(dev)
        v0 = torch.from_numpy(case.v_pages).to(dev)
        ks0 = torch.from_numpy(case.k_scales).to(dev)
        vs0 = torch.from_numpy(case.v_scales).to(dev)
    copies = [(k0, v0, ks0, vs0),
              (k0.clone(), v0.clone(), None if ks0 is None else ks0.clone(),
               None if vs0 is None else vs0.clone())]
    r2t = torch.from_numpy(case.req_to_token).to(dev)
    rpi = torch.from_numpy(case.req_pool_indices).to(dev)
    sl = torch.from_numpy(case.seq_lens).to(dev)
    B, Hq, D, S = case.batch, case.num_q_heads, case.head_dim, case.num_splits
    Hkv, P, msp = case.num_kv_heads, case.page_size, case.max_seq_pages
    pt = torch.empty((B, msp), dtype=torch.int32, device=dev)
    cache = torch.empty((B,), dtype=torch.int32, device=dev)
    cu = torch.empty((B + 1,), dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    ws = spa.new_workspace(B, Hq, Hkv, D, S, device=dev)
    scale = float(case.scale)

    def k1():
        spa.build_page_table(r2t, rpi, sl, P, msp, page_table=pt, cache_seqlens=cache,
                             cu_seqlens_k=cu)

    def attn(i):
        k, v, ks, vs = copies[i % 2]
        spa.paged_decode_attention(q, k, v, pt, sl, S, scale, kv_dtype=case.kv_dtype,
                                   k_scales=ks, v_scales=vs, workspace=ws, out=out, lse=lse)

    for i in range(args.warmup):
        k1()
        attn(i)
    torch.cuda.synchronize()

    K = args.steps
    ev_s = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev_e = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(K):
        k1()
        ev_s[i].record()
        attn(i)
        ev_e[i].record()
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / K
    attn_us = [ev_s[i].elapsed_time(ev_e[i]) * 1e3 for i in range(K)]
    attn_us_mean = float(np.mean(attn_us))

    # HIP-graph replay of the whole step (both KV copies, alternating)
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(2):
            k1()
            attn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(2):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            k1()
            attn(i)
        graphs.append(g)
    for i in range(20):
        graphs[i % 2].replay()
    torch.cuda.synchronize()
    R = args.graph_replays
    gs = [torch.cuda.Event(enable_timing=True) for _ in range(R)]
    ge = [torch.cuda.Event(enable_timing=True) for _ in range(R)]
    for i in range(R):
        gs[i].record()
        graphs[i % 2].replay()
        ge[i].record()
    torch.cuda.synchronize()
    graph_us = np.array([gs[i].elapsed_time(ge[i]) * 1e3 for i in range(R)])

    nbytes = W.algorithmic_bytes(case)
    achieved = nbytes / (attn_us_mean * 1e-6) / 1e9
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    workload = case.name
    traffic = _traffic_for("decode_attention.hip", workload)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
        oracle.case_attention(case)           # untimed (page-in)
        ts = []
        for _ in range(max(1, args.cpu_reps)):
            t0 = time.perf_counter()
            oracle.case_attention(case)
            ts.append(time.perf_counter() - t0)
        t_med = float(np.median(ts))
        cpu = {"value": round(nbytes / t_med / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": f"whole {workload} decode-attention call (fp64 C oracle, OpenMP), "
                         f"median of {len(ts)} reps, {t_med * 1e6:.0f} us per call"}

    rec = {
        "metric": "decode-attn us/call + achieved HBM GB/s (% of peak), B=32 ctx=8K",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.kv_dtype,
        "data": "synthetic (seeded N(0,1) K/V/Q, random page placement)",
        "config": {"workload": workload, "batch": B, "context": int(case.seq_lens.max()),
                   "ragged": bool(np.any(case.seq_lens != case.seq_lens[0])),
                   "num_q_heads": Hq, "num_kv_heads": Hkv, "head_dim": D, "page_size": P,
                   "num_pages": case.num_pages, "num_splits": S, "kv_dtype": case.kv_dtype,
                   "step": "page-table build + fused split-K decode attention"},
        "us_per_call": round(attn_us_mean, 3),
        "pct_of_peak": round(100.0 * achieved / PEAK_HBM_GBS, 2),
        "graph_step_us": {"p10": round(float(np.percentile(graph_us, 10)), 3),
                          "p50": round(float(np.percentile(graph_us, 50)), 3),
                          "p90": round(float(np.percentile(graph_us, 90)), 3)},
        "algorithmic_bytes": int(nbytes),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic},
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
        "gen_s": round(gen_s, 2),
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
