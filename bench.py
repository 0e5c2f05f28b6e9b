"""Benchmark of the split-K paged-attention decode step on one MI355X.

One step = the whole hot path on one batch: the page table / cache_seqlens /
cu_seqlens_k build (one launch) followed by one split-K paged-attention decode
with the library's default choices (producer plus log-sum-exp merge).  Where
the default plan is two launches (at the default workload: the head-grouped
producer, then the merge), the step makes them through the producer entry
point and the merge entry point, which launch exactly those kernels.
Default workload: batch 32, context 8192, 32 query / 8 KV heads, head_dim 128,
bf16 K/V in 64-token pages scattered over a 4096-page pool, 16 splits --
lmdeploy's headline H200 shape.

Timing: W untimed warm-up steps, then untimed steps until --settle-ms have
passed (the GPU's clocks settle after about 10 ms of sustained work), then
exactly K steps between two device synchronisations (events on the launch
stream bracket the run; `value` and ms_per_step come from them).  Then K
more of the same steps with HIP events around every attention call (both
launches and the gap between them fall inside) and, for a two-launch plan,
around the producer launch alone: the roofline figure is the algorithmic
bytes over the producer's average duration.  These events are kept out of
the timed steps because an event between two launches idles the GPU for
about 4 us.  The KV pool holds R >= 2 copies of the batch's pages, R * (bytes
of one copy) >= 1 GiB, and step i reads copy i % R, so no step finds its
pages in the 256 MB Infinity Cache.  HIP graphs of R steps and of R calls
are timed as well (the pages quote CUDA-graph latency), p10 / p50 / p90 per
call over the replays.  The fp64 CPU oracle is timed on the host beside it.

Prints ONE JSON line.  --summarize-pmc turns two rocprofv3 counter runs
(FETCH_SIZE, WRITE_SIZE) into the HBM-traffic record the bench reports.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0   # MI355X HBM3E peak, GB/s

# Context only (another machine): split-K paged-attention CUDA-graph latency on
# H200 before PDL, from the lmdeploy PR "use PDL for paged attention",
# Performance table.  Not a target and not used for vs_baseline, whose unit
# (GB/s) the page does not report.
H200_GRAPH_US = {"b1_ctx1k_s4_bf16": 12.096, "b1_ctx8k_s16_bf16": 22.080,
                 "b8_ctx1k_s4_bf16": 21.376, "b32_ctx8k_s16_bf16": 260.384}


# Sources of the kernels one call runs (the merge kernel lives with the decode).
KERNEL_SOURCES = {
    "decode": ["decode_attention.hip", "kernel_common.h"],
    "verify": ["verify_attention.hip", "decode_attention.hip", "kernel_common.h"],
}


def _source_hash(kind: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(open(os.path.join(ROOT, "split_paged_attention_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def _traffic_for(kind: str, workload: str, producer_only: bool = False):
    """HBM bytes per call (or per producer launch) from the committed
    rocprofv3 counter summary, if it was taken on the current kernel sources;
    else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("kernel_source_sha256") != _source_hash(kind):
            return None
        if producer_only:
            k = rec["kernels"]["verify" if kind == "verify" else "decode"]
            return int(k["fetch_bytes"]) + int(k["write_bytes"])
        return int(rec["hbm_bytes_per_launch"])
    except Exception:
        return None


def _pmc_rows(d: str):
    """Rows of every rocprofv3 counter_collection.csv under directory d."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _per_dispatch(rows, counter: str, match) -> list:
    """Counter value per dispatch (summed over its dimension rows) for kernels
    whose name satisfies match()."""
    acc = {}
    for r in rows:
        if r.get("Counter_Name") != counter or not match(r.get("Kernel_Name", "")):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    return list(acc.values())


def summarize_pmc(fetch_dir: str, write_dir: str, out_path: str, copy_mib: int, workload: str,
                  commands: list, kind: str = "decode") -> dict:
    """HBM bytes per decode call from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE, both in KiB per dispatch), each scaled by what the same counter
    reads for a device copy of copy_mib MiB (which moves exactly that many bytes
    each way)."""
    import statistics
    fr, wr = _pmc_rows(fetch_dir), _pmc_rows(write_dir)
    is_copy = lambda k: "copyBuffer" in k or "elementwise" in k or "copy" in k.lower()
    rec = {"workload": workload, "commands": commands, "copy_reference_bytes": copy_mib << 20,
           "kernels": {}}
    nbytes = copy_mib << 20
    cf = [v for v in _per_dispatch(fr, "FETCH_SIZE", is_copy) if v > 0]
    cw = [v for v in _per_dispatch(wr, "WRITE_SIZE", is_copy) if v > 0]
    fscale = nbytes / (1024.0 * max(cf)) if cf else None
    wscale = nbytes / (1024.0 * max(cw)) if cw else None
    rec["fetch_scale"] = fscale
    rec["write_scale"] = wscale
    total = 0.0
    producer = ("verify", "verify_kernel") if kind == "verify" else ("decode", "decode_kernel")
    for short, pat in (producer, ("split_merge", "split_merge"),
                       ("metadata", "build_metadata_kernel")):
        f = _per_dispatch(fr, "FETCH_SIZE", lambda k, pat=pat: pat in k)
        w = _per_dispatch(wr, "WRITE_SIZE", lambda k, pat=pat: pat in k)
        if not f or not w or fscale is None or wscale is None:
            continue
        fb = statistics.median(f) * 1024.0 * fscale
        wb = statistics.median(w) * 1024.0 * wscale
        rec["kernels"][short] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                                 "dispatches": len(f)}
        if short in (producer[0], "split_merge"):
            total += fb + wb
    rec["kernel_source_sha256"] = _source_hash(kind)
    rec["hbm_bytes_per_launch"] = round(total)
    with open(out_path, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def summarize_trace(trace_dir: str, warmup: int, steps: int) -> dict:
    """Per-kernel durations from a rocprofv3 --kernel-trace run of this bench:
    the average over the K timed steps (decode dispatches warmup ..
    warmup + steps - 1, in start order), over the K steps that follow them
    with per-launch events, and over all dispatches."""
    import csv
    import glob
    import statistics
    rows = []
    for f in glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    out = {}
    for short, pat in (("producer", "decode_kernel"), ("verify_producer", "verify_kernel"),
                       ("split_merge", "split_merge_kernel"),
                       ("metadata", "build_metadata_kernel")):
        d = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
             for r in rows if pat in r["Kernel_Name"]]
        if not d:
            continue
        names = sorted(set(r["Kernel_Name"] for r in rows if pat in r["Kernel_Name"]))
        o = 1 if short == "metadata" else 0     # the rig's own first page-table build
        timed = d[o + warmup:o + warmup + steps]
        evented = d[o + warmup + steps:o + warmup + 2 * steps]
        out[short] = {"kernel": names, "dispatches": len(d),
                      "timed_steps_avg_us": round(statistics.mean(timed), 3) if timed else None,
                      "event_steps_avg_us": round(statistics.mean(evented), 3) if evented else None,
                      "all_avg_us": round(statistics.mean(d), 3)}
    return out


class HipEvents:
    """Timing events of the HIP runtime torch has loaded, created with
    hipEventDisableSystemFence: recording one then costs no system-scope cache
    writeback and invalidation, which with torch's default events slowed the
    next kernel (the producer by about 5% at batch 32 / 8K).  Elapsed times
    are read only after a device synchronisation."""

    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        path = None
        with open("/proc/self/maps") as fh:
            for line in fh:
                if "libamdhip64.so" in line:
                    path = line.split()[-1]
                    break
        if path is None:
            raise RuntimeError("the HIP runtime is not loaded (import torch and use the GPU first)")
        self.ct = ctypes
        self.hip = ctypes.CDLL(path)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.events = []

    def new(self):
        ev = self.ct.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.ct.byref(ev), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        self.events.append(ev)
        return ev

    def record(self, ev):
        import torch
        rc = self.hip.hipEventRecord(ev, self.ct.c_void_p(torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def ms(self, a, b) -> float:
        f = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(f.value)

    def close(self):
        for ev in self.events:
            self.hip.hipEventDestroy(ev)
        self.events = []


# Timing loops rotate over copies of the batch's pages so that consecutive
# calls read different addresses: with at least this many bytes of distinct
# K/V between two reads of the same page, the 256 MB Infinity Cache (MALL)
# cannot serve them.
ROTATION_BYTES = 1 << 30


def rotation_copies(case, min_bytes: int = ROTATION_BYTES) -> int:
    """Copies of the batch's used pages (at least 2) whose K/V (+ scales)
    bytes together reach min_bytes."""
    import numpy as np
    P = case.page_size
    used = int(sum(-(-int(L) // P) for L in case.seq_lens))
    per = used * P * case.kv_bytes_per_token()
    return max(2, -(-min_bytes // max(per, 1))), per


class Rig:
    """Device copies of one workload and the calls of one step on them.

    The KV pool holds R copies of the pages the batch uses (R from
    rotation_copies), each in its own random placement; call i reads copy
    i % R, through a req_to_token map whose rows c*B .. c*B+B-1 are the
    batch's requests in copy c.  Step i builds copy i % R's page table with
    the metadata kernel and decodes from it; attention-only calls use the
    page tables built once at set-up."""

    def __init__(self, case, qlen: int = 0):
        import numpy as np
        import torch

        import split_paged_attention_amd as spa
        import workloads as W
        self.case = case
        self.qlen = qlen
        dev = "cuda:0"

        def bf16(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(
                torch.bfloat16)

        self.R, self.copy_bytes = rotation_copies(case)
        src, r2t, rpi = W.rotation_layout(case, self.R)
        src = torch.from_numpy(src).to(dev)
        self.q = bf16(case.q)
        if case.kv_dtype == "bf16":
            k0, v0 = bf16(case.k_pages), bf16(case.v_pages)
            ks0 = vs0 = None
        else:
            k0 = torch.from_numpy(case.k_pages).to(dev)
            v0 = torch.from_numpy(case.v_pages).to(dev)
            ks0 = torch.from_numpy(case.k_scales).to(dev)
            vs0 = torch.from_numpy(case.v_scales).to(dev)
        # the rotated pool: page n holds the case's page src[n]
        self.k = k0.index_select(0, src)
        self.v = v0.index_select(0, src)
        self.ks = None if ks0 is None else ks0.index_select(0, src)
        self.vs = None if vs0 is None else vs0.index_select(0, src)
        del k0, v0, ks0, vs0
        self.r2t = torch.from_numpy(r2t).to(dev)
        self.rpi = torch.from_numpy(rpi).to(dev)          # [R, B]
        self.sl = torch.from_numpy(case.seq_lens).to(dev)
        B, Hq, D, S = case.batch, case.num_q_heads, case.head_dim, case.num_splits
        self.pt = torch.empty((self.R, B, case.max_seq_pages), dtype=torch.int32, device=dev)
        self.cache = torch.empty((B,), dtype=torch.int32, device=dev)
        self.cu = torch.empty((B + 1,), dtype=torch.int32, device=dev)
        self.out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        self.ws = spa.new_workspace(B, Hq, case.num_kv_heads, D, S, device=dev)
        if qlen:
            # multi-token decode: qlen query rows per request; cu_seqlens_q
            # comes from the metadata build (strided mode)
            q_rows, _ = W.verify_queries(case, [qlen] * B)
            self.q_rows = bf16(q_rows)
            self.cu_q = torch.empty((B + 1,), dtype=torch.int32, device=dev)
            T = B * qlen
            self.ws = torch.empty(spa.verify_workspace_bytes(T, Hq, case.num_kv_heads, D, S),
                                  dtype=torch.uint8, device=dev)
            self.out = torch.empty((T, Hq, D), dtype=torch.bfloat16, device=dev)
            self.lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
        self.spa = spa
        self.merge = None
        self.producer = None
        # one-token decode with a two-launch default plan: the step can run
        # the producer and the merge as two entry points (same kernels as
        # the one call), so that events can bracket the producer alone
        self.two_launch = (not qlen and spa.decode_default_flags(
            B, case.num_kv_heads, S, case.kv_dtype, case.max_seq_pages)
            & spa.SPA_DECODE_SEPARATE_MERGE) != 0
        if self.two_launch:
            self.p_acc = torch.empty((B, Hq, S, D), dtype=torch.float32, device=dev)
            self.p_max = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
            self.p_sum = torch.empty((B, Hq, S), dtype=torch.float32, device=dev)
        for c in range(self.R):
            self.k1(c)                # every copy's page table, for attention-only calls
        torch.cuda.synchronize()

    def k1(self, i):
        """The metadata build of call i (copy i % R's page table)."""
        c = self.case
        r = i % self.R
        if self.qlen:
            self.spa.build_metadata(self.r2t, self.rpi[r], self.sl, c.page_size, c.max_seq_pages,
                                    page_table=self.pt[r], cache_seqlens=self.cache,
                                    cu_seqlens_k=self.cu, q_mode=self.spa.Q_MODE_STRIDED,
                                    q_stride=self.qlen, cu_seqlens_q=self.cu_q)
            return
        self.spa.build_page_table(self.r2t, self.rpi[r], self.sl, c.page_size, c.max_seq_pages,
                                  page_table=self.pt[r], cache_seqlens=self.cache,
                                  cu_seqlens_k=self.cu)

    def attn(self, i):
        c = self.case
        pt = self.pt[i % self.R]
        if self.qlen:
            self.spa.paged_verify_attention(self.q_rows, self.k, self.v, pt, self.sl, self.cu_q,
                                            c.num_splits, float(c.scale), max_q_len=self.qlen,
                                            kv_dtype=c.kv_dtype, k_scales=self.ks,
                                            v_scales=self.vs, workspace=self.ws, out=self.out,
                                            lse=self.lse)
            return
        self.spa.paged_decode_attention(self.q, self.k, self.v, pt, self.sl, c.num_splits,
                                        float(c.scale), kv_dtype=c.kv_dtype, k_scales=self.ks,
                                        v_scales=self.vs, workspace=self.ws, out=self.out,
                                        lse=self.lse, merge=self.merge,
                                        producer=self.producer)

    def producer_pass(self, i):
        """spa_paged_decode_partials: the producer launch of a two-launch call."""
        c = self.case
        self.spa.paged_decode_partials(self.q, self.k, self.v, self.pt[i % self.R], self.sl,
                                       c.num_splits, float(c.scale), kv_dtype=c.kv_dtype,
                                       k_scales=self.ks, v_scales=self.vs,
                                       partial_acc=self.p_acc, partial_max=self.p_max,
                                       partial_sum=self.p_sum)

    def merge_pass(self):
        """spa_split_merge over the producer's split states."""
        self.spa.split_merge(self.p_acc, self.p_max, self.p_sum, out=self.out, lse=self.lse)


def capture(fn, n):
    """A HIP graph of fn(0), fn(1), ..., fn(n - 1), after a warm-up of the
    same calls on a side stream."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n):
            fn(i)
    return g


def time_graph(g, calls: int, replays: int, warm_ms: float = 50.0):
    """Microseconds per call of a graph of `calls` calls: replays back to
    back until warm_ms have passed (the clocks settle after about 10 ms of
    sustained work), then `replays` replays, each between two events.
    Returns (mean, p10, p50, p90) over the replays."""
    import numpy as np
    import torch
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            g.replay()
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= warm_ms:
            break
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(replays)]
    for a, b in ev:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 / calls for a, b in ev])
    return (float(us.mean()), float(np.percentile(us, 10)), float(np.percentile(us, 50)),
            float(np.percentile(us, 90)))


def time_eager(fn, K, warmup=200):
    """Per-call microseconds (mean, median) from events around each of K calls."""
    import numpy as np
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i in range(K):
        ev[i][0].record()
        fn(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    return float(np.mean(us)), float(np.median(us))


def ablation(args) -> int:
    """Launch-gap ablation: every workload, eager (events around each call)
    and HIP-graph replay, merge fused into the producer launch vs a second
    launch, for each producer shape the workload supports.  One JSON line."""
    import workloads as W
    cfgs = [int(x) for x in args.ablation_configs.split(",")]
    rows = []
    for cfg in cfgs:
        case = W.make_config(cfg)
        rig = Rig(case)
        for producer in ("head_grouped", "page_split"):
            for merge in ("fused", "separate"):
                rig.producer, rig.merge = producer, merge
                e_mean, e_med = time_eager(rig.attn, args.steps)
                # one call per graph (the graph launch paid per call), and a
                # graph of R calls over the R page copies (paid once per R)
                g1 = [capture(lambda i, c=c: rig.attn(c), 1) for c in range(2)]
                g1_us = min(time_graph(g, 1, max(1, args.graph_replays // 2))[2] for g in g1)
                gr = time_graph(capture(rig.attn, rig.R), rig.R, max(1, args.graph_replays // 4))
                rows.append({"workload": case.name, "producer": producer, "merge": merge,
                             "eager_us_mean": round(e_mean, 3), "eager_us_median": round(e_med, 3),
                             "graph_1_call_us": round(g1_us, 3), "graph_us_p50": round(gr[2], 3),
                             "graph_us_p10": round(gr[1], 3), "graph_us_p90": round(gr[3], 3),
                             "graph_calls": rig.R,
                             "h200_graph_us_pre_pdl": H200_GRAPH_US.get(case.name)})
                print(f"[ablation] {rows[-1]}", file=sys.stderr, flush=True)
        del rig
    print(json.dumps({"ablation": "launch gap: eager vs graph x fused vs two-launch merge",
                      "rows": rows}), flush=True)
    return 0


def policy_sweep(args) -> int:
    """Producer x merge choice across decode shapes (batch 1-32, context
    1K-8K, 4/8/16 splits, equal lengths; then ragged batches of 8-32
    requests with lengths U[1, 2K or 8K] and 8/16 splits; 32 query / 8 KV
    heads, head_dim 128, 64-token pages
    drawn at random from a 4096-page pool): microseconds per call from HIP
    graphs of R calls, for both producers with both merges and for the
    library's default.  The R calls of a graph read disjoint page sets that
    together cover the pool (R = pool pages // pages per call), so every
    call reads pages the Infinity Cache has not held since the pool's last
    pass.  One JSON line; a progress line per shape on stderr."""
    import itertools

    import numpy as np
    import torch

    import split_paged_attention_amd as spa
    kv = args.policy_sweep
    dev = "cuda:0"
    g = torch.Generator(device=dev)
    g.manual_seed(3)
    P, Hq, Hkv, D, pool = 64, 32, 8, 128, 4096
    if kv == "bf16":
        k = torch.randn(pool, P, Hkv, D, device=dev, generator=g).to(torch.bfloat16)
        ks = vs = None
    else:
        k = torch.randint(-127, 128, (pool, P, Hkv, D), device=dev, generator=g,
                          dtype=torch.int8)
        if kv == "fp8":
            k = k.view(torch.uint8) & 0xF7   # finite e4m3 codes (no NaN pattern)
        ks = torch.rand(pool, P, Hkv, device=dev, generator=g) * 0.02 + 0.001
        vs = ks.clone()
    v = k.clone()
    variants = [("page_split", "fused"), ("page_split", "separate"),
                ("head_grouped", "fused"), ("head_grouped", "separate"), (None, None)]
    rows = []
    # equal lengths, then ragged batches (lengths U[1, L], seeded per shape)
    shapes = [(B, L, S, False) for B, L, S in
              itertools.product([1, 2, 4, 8, 16, 32], [1024, 2048, 4096, 8192], [4, 8, 16])]
    shapes += [(B, L, S, True) for B, L, S in itertools.product([8, 16, 32], [2048, 8192], [8, 16])]
    for B, L, S, ragged in shapes:
        npg = B * (L // P)
        R = max(1, pool // npg)
        q = torch.randn(B, Hq, D, device=dev, generator=g).to(torch.bfloat16)
        pts = torch.randperm(pool, device=dev, generator=g)[:R * npg].to(torch.int32)
        pts = pts.view(R, B, L // P).contiguous()
        if ragged:
            lens = np.random.default_rng(1000 * B + S).integers(1, L + 1, size=B)
            sl = torch.tensor(lens, dtype=torch.int32, device=dev)
        else:
            sl = torch.full((B,), L, dtype=torch.int32, device=dev)
        ws = spa.new_workspace(B, Hq, Hkv, D, S, device=dev)
        out = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
        us = []
        for prod, merge in variants:
            def call(i, prod=prod, merge=merge):
                spa.paged_decode_attention(q, k, v, pts[i % R], sl, S, 0.0884, kv_dtype=kv,
                                           k_scales=ks, v_scales=vs, workspace=ws, out=out,
                                           lse=lse, producer=prod, merge=merge)

            us.append(time_graph(capture(call, R), R, max(2, 40 // R), warm_ms=10.0)[0])
        best = min(range(4), key=lambda i: us[i])
        rows.append({"batch": B, "context": L, "ragged": ragged, "splits": S,
                     "waves": B * Hkv * S, "calls": R,
                     "page_split_fused_us": round(us[0], 2),
                     "page_split_separate_us": round(us[1], 2),
                     "head_grouped_fused_us": round(us[2], 2),
                     "head_grouped_separate_us": round(us[3], 2),
                     "default_us": round(us[4], 2),
                     "best": "/".join(variants[best])})
        print(f"[policy] {rows[-1]}", file=sys.stderr, flush=True)
    print(json.dumps({"policy_sweep": kv, "unit": "us per call (graph replay)", "rows": rows}),
          flush=True)
    return 0


TIMELINE_NAMES = ["entry", "length known", "first page id", "first scores", "pages done",
                  "states issued", "states in memory", "arrival counted", "merge done", "end"]


def timeline(args) -> int:
    """Per-wave timeline of one decode call from the diagnostics build
    libspa_timeline.so (include/spa_timeline.h): warm-up calls on the rotated
    pool, then --timeline-calls single calls, each on the next page copy,
    stamped and read back.  Prints one JSON line: the last call's per-link
    durations (between consecutive steps each wave reached) and, per page
    count of a wave's workgroup, when its waves started and ended.  The
    stamps themselves cost time: spans are longer than the library's."""
    import ctypes

    import numpy as np
    import torch

    import split_paged_attention_amd as spa
    from split_paged_attention_amd import build as spa_build
    import workloads as W

    if not os.path.exists(spa_build.TIMELINE_LIB):
        print(f"{spa_build.TIMELINE_LIB} is missing: build it first "
              "(python split_paged_attention_amd/build.py --timeline)", file=sys.stderr)
        return 2
    spa.LIB_PATH = spa_build.TIMELINE_LIB
    L = spa.lib()
    L.spa_timeline_clear.argtypes = []
    L.spa_timeline_clear.restype = ctypes.c_int
    L.spa_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    L.spa_timeline_read.restype = ctypes.c_int
    SLOTS, WAVES = 16, 65536
    torch.cuda.set_device(0)
    case = W.make_config(args.config)
    rig = Rig(case)
    i = 0
    t_end = time.time() + max(args.settle_ms, 30.0) / 1e3
    while i < args.warmup or time.time() < t_end:
        rig.attn(i)
        i += 1
        if i % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    spans, t = [], None
    for _ in range(args.timeline_calls):
        if L.spa_timeline_clear() != 0:
            raise RuntimeError("spa_timeline_clear failed")
        rig.attn(i)
        i += 1
        torch.cuda.synchronize()
        buf = np.zeros(WAVES * SLOTS, dtype=np.uint64)
        if L.spa_timeline_read(buf.ctypes.data, buf.nbytes) != 0:
            raise RuntimeError("spa_timeline_read failed")
        t = buf.reshape(WAVES, SLOTS)[:, :].astype(np.int64)
        t = t[t[:, 0] != 0]
        # waves of workgroups past a walked grid stamp only their entry (they
        # exit at once); they are counted, not charted
        exited = int((t[:, 1] == 0).sum())
        t = t[t[:, 1] != 0]
        spans.append(float((t[:, 9].max() - t[:, 0].min()) / 100.0))
    base = t[:, 0].min()
    us = lambda x: (x - base) / 100.0     # 100 MHz clock -> us
    links = {}
    for k in range(1, 9):
        ok = (t[:, k] != 0) & (t[:, k - 1] != 0)
        if ok.any():
            d = (t[ok, k] - t[ok, k - 1]) / 100.0
            links[f"{TIMELINE_NAMES[k - 1]} -> {TIMELINE_NAMES[k]}"] = {
                "waves": int(ok.sum()), "min_us": round(float(d.min()), 3),
                "median_us": round(float(np.median(d)), 3),
                "p90_us": round(float(np.percentile(d, 90)), 3), "max_us": round(float(d.max()), 3)}
    at = {TIMELINE_NAMES[k]: round(float(np.median(us(t[t[:, k] != 0, k]))), 3)
          for k in range(10) if (t[:, k] != 0).any()}
    st, en, npg = us(t[:, 0]), us(t[:, 9]), t[:, 11]
    by_pages = {}
    for k in sorted(set(npg.tolist())):
        m = npg == k
        by_pages[str(k)] = {"waves": int(m.sum()), "start_median_us": round(float(np.median(st[m])), 2),
                            "end_median_us": round(float(np.median(en[m])), 2),
                            "end_max_us": round(float(en[m].max()), 2),
                            "life_median_us": round(float(np.median(en[m] - st[m])), 2)}
    flags = spa.decode_default_flags(case.batch, case.num_kv_heads, case.num_splits, case.kv_dtype,
                                     case.max_seq_pages)
    rec = {"timeline": case.name, "library": os.path.basename(spa.LIB_PATH),
           "default_flags": int(flags), "waves": int(t.shape[0]),
           "waves_exited_at_once": exited, "calls": len(spans),
           "span_us": [round(x, 2) for x in spans],
           "wave_start_us_pct": [round(float(x), 2) for x in np.percentile(st, [0, 50, 90, 100])],
           "wave_end_us_pct": [round(float(x), 2) for x in np.percentile(en, [0, 50, 90, 100])],
           "step_median_us": at, "links": links, "by_workgroup_pages": by_pages,
           "rotation": {"page_copies": rig.R}}
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200,
                    help="untimed steps first: the GPU clocks settle after about 10 ms of "
                         "sustained work (durations rise about 12%% after an idle period, "
                         "then recover)")
    ap.add_argument("--config", type=int, default=4, help="workload 1..5 (4 = headline)")
    ap.add_argument("--graph-replays", type=int, default=200)
    ap.add_argument("--settle-ms", type=float, default=30.0,
                    help="untimed steps after the warm-up until this much time has passed, "
                         "whatever --warmup is (reported as settle_ms / settle_steps)")
    ap.add_argument("--cpu-reps", type=int, default=40,
                    help="timed oracle calls for cpu_baseline (about 10 s of host work at the "
                         "headline shape)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-ref-mib", type=int, default=0,
                    help="after timing, run device copies of this size (counter scaling)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="turn two rocprofv3 --pmc runs into a traffic record and exit")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR", default=None,
                    help="per-kernel averages over the timed steps of a rocprofv3 "
                         "--kernel-trace run of this bench (same --steps/--warmup), then exit")
    ap.add_argument("--pmc-out", default=None)
    ap.add_argument("--pmc-commands", nargs="*", default=[])
    ap.add_argument("--ablation", action="store_true",
                    help="launch-gap ablation over workloads instead of the bench line")
    ap.add_argument("--ablation-configs", default="1,2,3,4,5")
    ap.add_argument("--policy-sweep", choices=["bf16", "int8", "fp8"], default=None,
                    help="time both producers and merges over a grid of decode shapes")
    ap.add_argument("--verify-qlen", type=int, default=0,
                    help="multi-token decode with this many query tokens per request (1..64)")
    ap.add_argument("--timeline", action="store_true",
                    help="per-wave timeline of the one-token decode producer (diagnostics "
                         "build libspa_timeline.so) instead of the bench line")
    ap.add_argument("--timeline-calls", type=int, default=5)
    args = ap.parse_args()

    if args.summarize_trace:
        print(json.dumps(summarize_trace(args.summarize_trace, args.warmup, args.steps)),
              flush=True)
        return 0

    if args.summarize_pmc:
        import workloads as W
        name = W.CONFIGS[args.config]["name"] + (f"_q{args.verify_qlen}" if args.verify_qlen else "")
        out = args.pmc_out or os.path.join(ROOT, "profiles", f"traffic_{name}.json")
        rec = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], out,
                            args.copy_ref_mib or 1024, name, args.pmc_commands,
                            kind="verify" if args.verify_qlen else "decode")
        print(json.dumps(rec), flush=True)
        return 0

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this decode path has no multi-GPU mode "
              "(batch rows and KV heads would shard across GPUs with no exchange).",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import split_paged_attention_amd as spa
    import workloads as W

    if args.timeline:
        return timeline(args)
    torch.cuda.set_device(0)
    spa.lib()  # fail loudly if the HIP library is missing
    if args.ablation:
        return ablation(args)
    if args.policy_sweep:
        return policy_sweep(args)
    t_gen = time.time()
    case = W.make_config(args.config)
    gen_s = time.time() - t_gen
    Q = args.verify_qlen
    if Q < 0 or Q > 64:
        print("--verify-qlen must be 0..64", file=sys.stderr)
        return 2
    rig = Rig(case, qlen=Q)
    dev = "cuda:0"
    B, Hq, D, S = case.batch, case.num_q_heads, case.head_dim, case.num_splits
    Hkv, P = case.num_kv_heads, case.page_size
    k1, attn = rig.k1, rig.attn

    # One step: the metadata build, then the decode call.  Where the
    # library's default plan is two launches (producer, then merge), the step
    # makes them as the two entry points that launch exactly those kernels,
    # and an event between them times the producer -- the dominant kernel --
    # on its own; otherwise the call is one launch and its events time it.
    two = rig.two_launch

    hev = HipEvents()

    def step(i, ev=None):
        k1(i)
        if ev is not None:
            hev.record(ev[0])
        if two:
            rig.producer_pass(i)
            if ev is not None:
                hev.record(ev[1])
            rig.merge_pass()
        else:
            attn(i)
        if ev is not None:
            hev.record(ev[2])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # Settle: after an idle period the GPU's clocks take about 10 ms of
    # sustained work to settle (durations rise ~12% and recover), so untimed
    # steps continue until settle_ms have passed, however few warm-up steps
    # were asked for.  The timed steps below are unaffected in number.
    settle0 = time.perf_counter()
    settle_steps = 0
    while (time.perf_counter() - settle0) * 1e3 < args.settle_ms:
        for _ in range(8):
            step(args.warmup + settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    settle_ms = (time.perf_counter() - settle0) * 1e3

    # The K timed steps: events only around the whole run (an event between
    # two launches leaves the GPU idle for about 4 us, so per-launch events
    # would inflate the step time).
    K = args.steps
    t_start, t_end = hev.new(), hev.new()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    hev.record(t_start)
    for i in range(K):
        step(i)
    hev.record(t_end)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = hev.ms(t_start, t_end) / K
    # Then K more of the same steps with events around each decode call and
    # around its producer launch: the per-call and per-kernel durations.
    evs = [[hev.new() for _ in range(3)] for _ in range(K)]
    for i in range(K):
        step(K + i, evs[i])
    torch.cuda.synchronize()
    attn_us = np.array([hev.ms(e[0], e[2]) * 1e3 for e in evs])
    kernel_us = np.array([hev.ms(e[0], e[1]) * 1e3 for e in evs]) if two else attn_us
    attn_us_mean, kernel_us_mean = float(attn_us.mean()), float(kernel_us.mean())
    hev.close()

    def pct(x):
        return {"p10": round(float(np.percentile(x, 10)), 3),
                "p50": round(float(np.percentile(x, 50)), 3),
                "p90": round(float(np.percentile(x, 90)), 3)}

    if args.copy_ref_mib > 0:
        # device copies of a known size, for scaling the memory counters
        src_buf = torch.empty(args.copy_ref_mib << 20, dtype=torch.uint8, device=dev)
        dst_buf = torch.empty_like(src_buf)
        for _ in range(2):
            dst_buf.copy_(src_buf)
        torch.cuda.synchronize()
        del src_buf, dst_buf

    # HIP-graph replays (the pages quote CUDA-graph latency): graphs of R
    # steps and of R attention calls, call i on page copy i % R, so no call
    # finds its pages in the Infinity Cache; per call, p10 / p50 / p90 over
    # the replays (the graph launch, about 8 us, is paid once per R calls).
    def step_fn(i):
        k1(i)
        attn(i)

    reps = max(4, args.graph_replays)
    gs = time_graph(capture(step_fn, rig.R), rig.R, max(4, reps // max(1, rig.R // 16)))
    ga = time_graph(capture(attn, rig.R), rig.R, max(4, reps // max(1, rig.R // 16)))

    nbytes = W.verify_algorithmic_bytes(case, [Q] * B) if Q else W.algorithmic_bytes(case)
    achieved = nbytes / (kernel_us_mean * 1e-6) / 1e9
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    workload = case.name + (f"_q{Q}" if Q else "")
    traffic = _traffic_for("verify" if Q else "decode", workload, producer_only=two)

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cores = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
        if Q:
            q_rows, cu_q = W.verify_queries(case, [Q] * B)
            pt_o, _, _ = oracle.case_page_table(case)

            def run_oracle():
                oracle.verify_attention(q_rows, case.k_pages, case.v_pages, pt_o, case.seq_lens,
                                        cu_q, num_kv_heads=Hkv, page_size=P, scale=case.scale,
                                        kv_dtype=case.kv_dtype, k_scales=case.k_scales,
                                        v_scales=case.v_scales)
        else:
            def run_oracle():
                oracle.case_attention(case)
        run_oracle()                          # untimed (page-in)
        ts = []
        for _ in range(max(1, args.cpu_reps)):
            t0 = time.perf_counter()
            run_oracle()
            ts.append(time.perf_counter() - t0)
        t_med = float(np.median(ts))
        what = f"{Q}-token decode" if Q else "decode-attention"
        cpu = {"value": round(nbytes / t_med / 1e9, 4), "unit": "GB/s", "cores": cores,
               "kind": "oracle",
               "sample": f"whole {workload} {what} call (fp64 C oracle, OpenMP), "
                         f"median of {len(ts)} reps, {t_med * 1e6:.0f} us per call"}

    rec = {
        "metric": ("decode-attn us/call + achieved HBM GB/s (% of peak), B=32 ctx=8K" if not Q else
                   f"{Q}-token verify decode us/call + achieved HBM GB/s (% of peak)"),
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
                   "query_tokens_per_request": Q or 1,
                   "step": (("page-table build + split-K decode attention (library default "
                             "plan: producer launch, then merge launch)") if two else
                            "page-table build + split-K decode attention (library defaults)"
                            if not Q else "metadata build (page table, cu_seqlens_q) + "
                            "multi-token split-K decode attention")},
        "us_per_call": round(attn_us_mean, 3),
        "us_per_call_pct": pct(attn_us),
        "producer_us": round(kernel_us_mean, 3) if two else None,
        "producer_us_pct": pct(kernel_us) if two else None,
        "pct_of_peak": round(100.0 * achieved / PEAK_HBM_GBS, 2),
        "graph_step_us": round(gs[2], 3),
        "graph_step_us_pct": {"p10": round(gs[1], 3), "p50": round(gs[2], 3),
                              "p90": round(gs[3], 3)},
        "graph_attn_us": round(ga[2], 3),
        "graph_attn_us_pct": {"p10": round(ga[1], 3), "p50": round(ga[2], 3),
                              "p90": round(ga[3], 3)},
        "rotation": {"page_copies": rig.R, "bytes_per_copy": int(rig.copy_bytes),
                     "bytes_rotated": int(rig.R * rig.copy_bytes),
                     "note": "call i reads copy i % page_copies (distinct addresses), so "
                             "the 256 MB Infinity Cache cannot hold the pages between reads"},
        "settle_ms": round(settle_ms, 1),
        "settle_steps": settle_steps,
        "context_h200_graph_attn_us": None if Q else H200_GRAPH_US.get(case.name),
        "algorithmic_bytes": int(nbytes),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                     "traffic": traffic,
                     "kernel": ("producer launch (events around spa_paged_decode_partials)"
                                if two else "the call's launches (events around the call)")},
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 4),
        "gen_s": round(gen_s, 2),
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
