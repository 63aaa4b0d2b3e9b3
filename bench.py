#!/usr/bin/env python3
"""Benchmark of the multi-LoRA batched layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is one pass of the layer over one synthetic batch (lora_layer_apply's
launch sequence): for the decode batch, a stream launch (split-K partial
products of x W and the BGMV shrink partials x A[ids]) and a finish launch
(sum of partials plus the scaled expand, y rounded once).  The headline workload is the decode batch: one 4096->4096
q projection, rank 16, a uniform pool of 250 adapters, 32 single-token rows
on 20 distinct adapters plus 3 base-only rows, bf16 inputs with fp32
accumulation.  Successive steps rotate over 8 replicas of the layer
(different weights and pools, ~800 MB in all, more than the 256 MB
Infinity Cache) so that every step reads its weights from HBM, as the
layers of a model would.  Steps are captured in HIP graphs and replayed.

The JSON line carries:
  value        tokens/s of the whole step (wall clock around exactly K steps)
  roofline     the dominant kernel (the stream launch) against HBM peak, from
               its average launch duration (HIP events)
  adapter_term the adapter overhead fraction (step time minus base-only step
               time) and the standalone BGMV shrink's algorithmic bytes/s
  cpu_baseline the fp64 oracle on the host cores, on a bounded sample
  workloads    the other four workloads (skewed 8B decode, 70B prefill,
               mixed-rank 70B ragged and padded), measured the same way
  merge        the merge kernel's HBM GB/s (W += s A B in place)
  q4_decode    the headline decode batch over a 4-bit base weight
  adapter_term_prefill  the SGMV shrink and expand of the 70B prefill batch
               on their own: algorithmic HBM GB/s against the 8 TB/s peak
  paging       the adapter slot cache: cold-load latency and H2D GB/s of
               whole 8B-shaped adapters, decode step time with loads in flight
  serving      a Zipf decode serving loop through the admission scheduler and
               the slot cache: distinct adapters per step, adapter overhead
               fraction, hit rate and queue waits, locality weight vs FIFO
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--replicas", type=int, default=8)
    ap.add_argument("--kernel-reps", type=int, default=50, help="graph replays per kernel timing")
    ap.add_argument("--workloads", default="skewed,prefill,mixed",
                    help="comma list of extra workloads to measure (empty: none)")
    ap.add_argument("--extra-steps", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-paging", action="store_true", help="skip the adapter-paging measurements")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the merge, 4-bit and standalone SGMV legs (profiling runs of the workloads)")
    ap.add_argument("--comparators", action="store_true",
                    help="also time the vendor GEMM on the decode base product and a device copy of the "
                         "decode stream's bytes")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB read + 256 MiB write kernel (counter calibration)")
    return ap.parse_args()


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def profiled_traffic(kernel, sources, profile):
    """HBM bytes per launch from a committed counter summary, or None when the
    kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", profile)
    if not os.path.exists(path):
        return None
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    fields = {}
    for line in open(path).read().splitlines():
        if ":" in line and line.split(":")[0] in ("traffic_kernel", "traffic_bytes_per_launch", "source_hash"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("traffic_kernel") != kernel or fields.get("source_hash") != h.hexdigest()[:16]:
        return None
    return int(fields["traffic_bytes_per_launch"])


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def make_pool(b, p):
    from lora_bgmv_shrink_amd import workloads as wl
    if p.layout == wl.UNIFORM:
        return b.lora_pool_create(b.LORA_LAYOUT_UNIFORM, p.A, p.B, p.n_adapters, p.d_in, p.d_out, p.r_max,
                                  p.scales)
    return b.lora_pool_create(b.LORA_LAYOUT_RAGGED, p.A, p.B, p.n_adapters, p.d_in, p.d_out, p.r_max,
                              p.scales, ranks=p.ranks, a_off=p.a_off, b_off=p.b_off)


def capture(torch, fn):
    """Capture fn() into a HIP graph (after one eager run)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graph(torch, g, reps):
    """Average GPU time of one replay, from HIP events on the replay stream."""
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    g.replay()
    torch.cuda.synchronize()
    e0.record(s)
    for _ in range(reps):
        g.replay()
    e1.record(s)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e-3   # seconds


def distinct_bytes(p, ids, which):
    """Bytes of the A (or B) blocks of the distinct adapters the batch uses."""
    import numpy as np
    us = sorted(set(int(a) for a in ids.tolist() if 0 <= a < p.n_adapters))
    eb = p.A.element_size()
    if which == "A":
        return sum(int(p.ranks[u]) * p.d_in * eb for u in us), len(us)
    return sum(int(p.ranks[u]) * p.d_out * eb for u in us), len(us)


# ---------------------------------------------------------------------------
# headline: decode q_proj
# ---------------------------------------------------------------------------

def bench_decode(torch, args):
    import numpy as np

    from lora_bgmv_shrink_amd import binding as b
    from lora_bgmv_shrink_amd import workloads as wl

    dev = torch.device("cuda:0")
    R = args.replicas
    reps = []
    for r in range(R):
        w = wl.decode_q_proj(device=dev, value_seed=None if r == 0 else 1 + 1000 * r)
        p = w.projections[0]
        pool = make_pool(b, p.pool)
        Wt = p.W.t().contiguous()
        p.W = None
        n = w.n_rows
        ids = torch.as_tensor(w.ids, device=dev)
        y = torch.zeros((n, p.d_out), dtype=torch.bfloat16, device=dev)
        yb = torch.zeros_like(y)
        ws = torch.zeros(b.lora_decode_workspace(pool, n, True), dtype=torch.uint8, device=dev)
        wsb = torch.zeros(b.lora_decode_workspace(pool, n, False), dtype=torch.uint8, device=dev)
        reps.append(dict(w=w, p=p, pool=pool, Wt=Wt, ids=ids, y=y, yb=yb, ws=ws, wsb=wsb))
    w0, p0 = reps[0]["w"], reps[0]["p"]
    n = w0.n_rows

    def stream(r):
        b.lora_decode_stream(r["pool"], r["p"].x, r["Wt"], r["ids"], r["ws"], True)

    def finish(r):
        b.lora_decode_finish(r["pool"], r["ids"], r["ws"], r["y"], True)

    def base_stream(r):
        b.lora_decode_stream(r["pool"], r["p"].x, r["Wt"], r["ids"], r["wsb"], False)

    def base_finish(r):
        b.lora_decode_finish(r["pool"], r["ids"], r["wsb"], r["yb"], False)

    def base_step(r):
        base_stream(r)
        base_finish(r)

    def step(r):
        stream(r)
        finish(r)

    # the step is lora_layer_apply's launch sequence; check it gives the same bits
    r0 = reps[0]
    step(r0)
    y_ref = b.lora_layer_apply(r0["pool"], r0["p"].x, r0["Wt"], r0["ids"], w_layout=b.LORA_W_OUT_IN,
                               mode=b.LORA_MODE_BGMV)
    torch.cuda.synchronize()
    assert torch.equal(y_ref, r0["y"]), "step differs from lora_layer_apply"

    K, W = args.steps, args.warmup
    g_full = capture(torch, lambda: [step(r) for r in reps])
    rem = K % R
    g_rem = capture(torch, lambda: [step(r) for r in reps[:rem]]) if rem else None
    for _ in range(max(1, W // R)):
        g_full.replay()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps ----
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K // R):
        g_full.replay()
    if g_rem is not None:
        g_rem.replay()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    sec_step = (t1 - t0) / K

    # ---- per-kernel launch durations (graphs of R back-to-back launches) ----
    kr = args.kernel_reps
    g_stream = capture(torch, lambda: [stream(r) for r in reps])
    g_finish = capture(torch, lambda: [finish(r) for r in reps])
    g_base = capture(torch, lambda: [base_step(r) for r in reps])
    d_stream = time_graph(torch, g_stream, kr) / R
    d_finish = time_graph(torch, g_finish, kr) / R
    d_base = time_graph(torch, g_base, kr) / R
    d_bstream = time_graph(torch, capture(torch, lambda: [base_stream(r) for r in reps]), kr) / R
    d_bfinish = time_graph(torch, capture(torch, lambda: [base_finish(r) for r in reps]), kr) / R
    d_step = time_graph(torch, g_full, max(1, kr // 2)) / R
    decode_graph = g_full

    # the standalone BGMV shrink entry point on the same batch
    for r in reps:
        r["t"] = torch.zeros((n, r["p"].pool.r_max), dtype=torch.float32, device=dev)
    g_shr = capture(torch, lambda: [b.lora_bgmv_shrink(r["pool"], r["p"].x, r["ids"], t=r["t"]) for r in reps])
    d_shr = time_graph(torch, g_shr, kr) / R

    # diversity sweep: 32 rows on 1, 2, 4, ... 32 distinct adapters (each used
    # round-robin), same replicas and launches as the headline step
    sweep = []
    for U_s in (1, 2, 4, 8, 16, 32):
        ids_s = torch.as_tensor(((np.arange(n) % U_s) * 7) % 250, dtype=torch.int32, device=dev)
        for r in reps:
            r["ids_s"] = ids_s

        def step_s(r):
            b.lora_decode_stream(r["pool"], r["p"].x, r["Wt"], r["ids_s"], r["ws"], True)
            b.lora_decode_finish(r["pool"], r["ids_s"], r["ws"], r["y"], True)

        d_s = time_graph(torch, capture(torch, lambda: [step_s(r) for r in reps]), kr) / R
        sweep.append(dict(distinct_adapters=U_s, step_us=round(d_s * 1e6, 3),
                          adapter_bytes=U_s * 16 * (4096 + 4096) * 2))
    for r in reps:
        del r["ids_s"]

    pool = p0.pool
    bA, U = distinct_bytes(pool, w0.ids, "A")
    bB, _ = distinct_bytes(pool, w0.ids, "B")
    eb = 2
    x_b = n * pool.d_in * eb
    y_b = n * pool.d_out * eb
    t_b = n * pool.r_max * 4
    w_b = pool.d_in * pool.d_out * eb
    stream_bytes = w_b + bA + x_b + n * 4
    shrink_bytes = bA + x_b + t_b + n * 4
    achieved = stream_bytes / d_stream / 1e9
    comparators = None
    if args.comparators:
        # context, not part of the layer: the vendor GEMM on the bare base
        # product of the same batch, and a plain device copy that moves the
        # stream launch's algorithmic bytes (half read, half written)
        half = (stream_bytes // 4) * 2
        pool_dout = p0.pool.d_out
        for r in reps:
            r["y_mm"] = torch.empty((n, pool_dout), dtype=torch.bfloat16, device=dev)
            r["cp_src"] = torch.ones(half // 2, dtype=torch.bfloat16, device=dev)
            r["cp_dst"] = torch.empty_like(r["cp_src"])
        g_mm = capture(torch, lambda: [torch.mm(r["p"].x, r["Wt"].t(), out=r["y_mm"]) for r in reps])
        g_cp = capture(torch, lambda: [r["cp_dst"].copy_(r["cp_src"]) for r in reps])
        d_mm = time_graph(torch, g_mm, kr) / R
        d_cp = time_graph(torch, g_cp, kr) / R
        mm_bytes = p0.pool.d_in * pool_dout * 2 + n * p0.pool.d_in * 2 + n * pool_dout * 2
        comparators = dict(
            vendor_base_product=dict(call="torch.mm (hipBLASLt): x[32,4096] times W^T, W stored [d_out, d_in], bf16",
                                     us=round(d_mm * 1e6, 3), GBps=round(mm_bytes / d_mm / 1e9, 1)),
            device_copy_same_bytes=dict(bytes=2 * half, us=round(d_cp * 1e6, 3),
                                        GBps=round(2 * half / d_cp / 1e9, 1)),
            decode_stream_rate_over_copy_rate=round(d_cp / d_stream, 3),
            layer_step_over_vendor_base_product=round(d_step / d_mm, 3),
        )
        del g_mm, g_cp
        for r in reps:
            del r["y_mm"], r["cp_src"], r["cp_dst"]
    out = dict(
        sec_step=sec_step,
        tokens_per_s=n / sec_step,
        gpu_step_s=d_step,
        kernels_us=dict(decode_stream=round(d_stream * 1e6, 3), decode_finish=round(d_finish * 1e6, 3),
                        base_only_step=round(d_base * 1e6, 3), base_only_stream=round(d_bstream * 1e6, 3),
                        base_only_finish=round(d_bfinish * 1e6, 3),
                        bgmv_shrink_standalone=round(d_shr * 1e6, 3)),
        roofline=dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBS, 4),
                      traffic=profiled_traffic("k_decode_stream",
                                               ["lora_bgmv_shrink_amd/csrc/decode.hip",
                                                "lora_bgmv_shrink_amd/csrc/lora_internal.hpp"],
                                               "decode_q4096_r16_rows32_traffic.md"),
                      kernel="k_decode_stream (split-K base partials + BGMV shrink partials)",
                      what="the stream launch: the base weight W (92% of its bytes) and the distinct "
                           "adapters' A blocks; the adapter term alone is adapter_term.bgmv_shrink_frac_hbm",
                      bytes_per_launch=stream_bytes, avg_launch_us=round(d_stream * 1e6, 3)),
        adapter_term=dict(
            distinct_adapters=U,
            adapter_bytes=bA + bB,
            step_us=round(d_step * 1e6, 3), base_only_step_us=round(d_base * 1e6, 3),
            overhead_fraction=round(max(0.0, (d_step - d_base) / d_step), 4),
            layer_GBps=round((w_b + bA + bB + x_b + y_b) / d_step / 1e9, 1),
            bgmv_shrink_bytes=shrink_bytes, bgmv_shrink_us=round(d_shr * 1e6, 3),
            bgmv_shrink_GBps=round(shrink_bytes / d_shr / 1e9, 1),
            bgmv_shrink_frac_hbm=round(shrink_bytes / d_shr / 1e9 / HBM_PEAK_GBS, 4),
        ),
        comparators=comparators,
        diversity_sweep=sweep,
        # the graph replays launches over reps' tensors and pools: whoever
        # replays it must hold reps too
        _decode_graph=(decode_graph, reps),
    )
    return out, w0


# ---------------------------------------------------------------------------
# other workloads
# ---------------------------------------------------------------------------

def bench_multi(torch, args, name):
    """Seven projections per step through lora_layer_apply (AUTO mode)."""
    from lora_bgmv_shrink_amd import binding as b
    from lora_bgmv_shrink_amd import workloads as wl

    dev = torch.device("cuda:0")
    if name == "skewed":
        w = wl.skewed_decode_8b(device=dev)
        pools = [("uniform", [pp.pool for pp in w.projections])]
    elif name == "prefill":
        w = wl.prefill_70b(device=dev)
        pools = [("uniform", [pp.pool for pp in w.projections])]
    else:
        w = wl.mixed_rank_70b(device=dev)
        pools = [("ragged", [pp.pool for pp in w.projections]),
                 ("padded", [pp.pool_padded for pp in w.projections])]
    n = w.n_rows
    ids = torch.as_tensor(w.ids, device=dev)
    projs = []
    for pp in w.projections:
        Wt = pp.W.t().contiguous()
        pp.W = None
        projs.append(dict(p=pp, Wt=Wt, y=torch.empty((n, pp.d_out), dtype=torch.bfloat16, device=dev)))
    res = dict(workload=w.name, rows=n, distinct_adapters=int(len(set(w.ids[w.ids >= 0].tolist()))))
    for label, plist in pools:
        hs = [make_pool(b, pl) for pl in plist]
        wss = [torch.zeros(b.lora_layer_workspace(h, n), dtype=torch.uint8, device=dev) for h in hs]
        # one batch, one group-by: the segments are built once per step and
        # handed to every projection (a layer that picks BGMV ignores them)
        seg = b.segments_alloc(n, plist[0].n_adapters, dev)

        def step():
            b.lora_segments_build(ids, plist[0].n_adapters, seg=seg)
            for pr, h, ws in zip(projs, hs, wss):
                b.lora_layer_apply(h, pr["p"].x, pr["Wt"], ids, w_layout=b.LORA_W_OUT_IN, seg=seg, y=pr["y"],
                                   ws=ws)

        # base-only: the same calls with every row base-only (the adapter term
        # drops out; the kernels are the same)
        ids_base = torch.full_like(ids, -1)
        seg_base = b.lora_segments_build(ids_base, plist[0].n_adapters)

        def base_step():
            for pr, h, ws in zip(projs, hs, wss):
                b.lora_layer_apply(h, pr["p"].x, pr["Wt"], ids_base, w_layout=b.LORA_W_OUT_IN, seg=seg_base,
                                   y=pr["y"], ws=ws)

        g = capture(torch, step)
        gb = capture(torch, base_step)
        for _ in range(2):
            g.replay()
        torch.cuda.synchronize()
        K = args.extra_steps
        t0 = time.perf_counter()
        for _ in range(K):
            g.replay()
        torch.cuda.synchronize()
        sec = (time.perf_counter() - t0) / K
        d_base = time_graph(torch, gb, 3)
        flops = 0
        abytes = 0
        wbytes = 0
        for pr, pl in zip(projs, plist):
            pp = pr["p"]
            flops += 2 * n * pp.d_in * pp.d_out
            bA, _ = distinct_bytes(pl, w.ids, "A")
            bB, _ = distinct_bytes(pl, w.ids, "B")
            abytes += bA + bB
            wbytes += pp.d_in * pp.d_out * 2
            r_true = [int(pl.ranks[a]) if a >= 0 else 0 for a in w.ids.tolist()]
            flops += 2 * sum(r_true) * (pp.d_in + pp.d_out)
        res[label] = dict(
            tokens_per_s_per_projection=round(n * len(projs) / sec, 1),
            tokens_per_s_seven_projections=round(n / sec, 1),
            ms_per_step=round(sec * 1e3, 4),
            tflops=round(flops / sec / 1e12, 1), mfma_frac=round(flops / sec / 1e12 / BF16_PEAK_TFLOPS, 4),
            weight_plus_adapter_GBps=round((wbytes + abytes) / sec / 1e9, 1),
            weight_plus_adapter_frac_hbm=round((wbytes + abytes) / sec / 1e9 / HBM_PEAK_GBS, 4),
            adapter_bytes=abytes,
            overhead_fraction=round(max(0.0, (sec - d_base) / sec), 4),
        )
        res[label]["base_only_ms"] = round(d_base * 1e3, 4)
        for h in hs:
            h.destroy()
    if args.comparators:
        # context: the vendor GEMM (hipBLASLt through torch.mm) on the same
        # seven base products, W stored [d_out, d_in], no adapter term
        g_mm = capture(torch, lambda: [torch.mm(pr["p"].x, pr["Wt"].t(), out=pr["y"]) for pr in projs])
        res["vendor_base_product_ms"] = round(time_graph(torch, g_mm, 3) * 1e3, 4)
        del g_mm
    return res


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands
# ---------------------------------------------------------------------------

def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(w, seconds):
    """The fp64 oracle on the host cores: the full decode batch (base + LoRA)
    at all cores and at one thread, and the LoRA term alone (x A then
    s t B, no base product).  The oracle is rebuilt here for this host
    (-O3 -march=native, OpenMP, no fast-math) into a temporary file; the
    in-tree build stays portable."""
    import tempfile

    import numpy as np

    import oracle

    p = w.projections[0]
    pool = p.pool
    used = sorted(set(int(a) for a in w.ids.tolist() if a >= 0))
    # marshal the batch to fp64 (outside the timed loop)
    A, B, a_off, b_off = [], [], [], []
    pa = pb = 0
    for u in used:
        a = pool.a_block(u).float().cpu().double().numpy().reshape(-1)
        bb = pool.b_block(u).float().cpu().double().numpy().reshape(-1)
        a_off.append(pa)
        b_off.append(pb)
        pa += a.size
        pb += bb.size
        A.append(a)
        B.append(bb)
    mp = {u: i for i, u in enumerate(used)}
    ids = np.array([mp.get(int(a), -1) for a in w.ids.tolist()], np.int32)
    op = oracle.OraclePool(len(used), pool.d_in, pool.d_out, pool.r_max,
                           np.array([pool.ranks[u] for u in used], np.int32), np.array(a_off, np.int64),
                           np.array(b_off, np.int64), np.concatenate(A), np.concatenate(B),
                           pool.scales[used].astype(np.float64))
    x = p.x.float().cpu().double().numpy()
    Wm = p.W.float().cpu().double().numpy()
    lib = None
    native = False
    try:
        tmp = os.path.join(tempfile.gettempdir(), f"liboracle_native_{os.getpid()}.so")
        oracle.build(out=tmp, extra=("-march=native",))
        lib = oracle.load(tmp)
        native = True
    except Exception as e:   # no compiler: the in-tree build
        log(f"cpu baseline: native oracle build failed ({e}); using the in-tree build")
        lib = oracle.load()
    threads = oracle.max_threads(lib)

    def rate(fn, budget, min_passes=1):
        n_done = 0
        t0 = time.perf_counter()
        while True:
            fn()
            n_done += 1
            el = time.perf_counter() - t0
            if el >= budget and n_done >= min_passes:
                return n_done, el

    n_all, el_all = rate(lambda: oracle.layer(x, Wm, ids, op, threads=threads, lib=lib), 0.5 * seconds)
    n_one, el_one = rate(lambda: oracle.layer(x, Wm, ids, op, threads=1, lib=lib), 0.35 * seconds)
    n_lo, el_lo = rate(lambda: oracle.layer(x, None, ids, op, want=("lora",), threads=1, lib=lib),
                       0.15 * seconds)
    rows = w.n_rows
    return dict(value=round(n_all * rows / el_all, 2), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"full decode batch ({rows} rows, q 4096->4096, r16, 20 adapters, base + LoRA) "
                       f"x{n_all} passes, {el_all:.1f} s, fp64, {threads} threads",
                one_thread=dict(value=round(n_one * rows / el_one, 2), unit="tokens/s", cores=1,
                                sample=f"same batch x{n_one} passes, {el_one:.1f} s"),
                lora_term_one_thread=dict(value=round(n_lo * rows / el_lo, 2), unit="tokens/s", cores=1,
                                          sample=f"LoRA term alone (x A, s t B; no x W) x{n_lo} passes, "
                                                 f"{el_lo:.1f} s"),
                cpu_model=_cpu_model(), build="gcc -O3 -march=native -fopenmp" if native else "gcc -O3 -fopenmp")


def bench_paging(torch, args, decode, R):
    """Adapter slot cache: cold-load latency and host-to-device GB/s of whole
    8B-shaped adapters (32 layers x 7 projections; rank 8 is about the 40 MB
    hot adapter of the paging page, rank 16 twice that), and the decode step
    time while loads are in flight on the cache's stream versus idle (a
    fetch must not stall the decode loop).  Blobs are pinned host memory."""
    from lora_bgmv_shrink_amd import binding as b
    from lora_bgmv_shrink_amd import workloads as wl

    decode_graph, decode_reps = decode   # the replica tensors stay referenced while the graph replays
    assert len(decode_reps) == R
    dev = torch.device("cuda:0")
    parts = wl.eight_b_parts(32)
    n_ad, n_slots = 8, 4
    c = b.Cache(torch.bfloat16, parts, 16, n_ad, n_slots, 4, device=dev)
    ranks = [8, 16] * (n_ad // 2)
    blob_bytes = {}
    g = wl._gen(dev, 9100)
    for a, r in enumerate(ranks):
        n_el = c.blob_layout(r)[2]
        blob = torch.empty(n_el, dtype=torch.bfloat16, pin_memory=True)
        blob.copy_((torch.randn(n_el, generator=g, device=dev) / 64).to(torch.bfloat16))
        c.register_blob(a, r, 2.0, blob)
        blob_bytes[r] = n_el * 2
    torch.cuda.synchronize()

    # cold loads one at a time: request (miss) then wait
    lat = {8: [], 16: []}
    for _ in range(3):
        for a in range(n_ad):
            if c.slot_of(a) >= 0:
                continue
            t0 = time.perf_counter()
            st = c.request(a)
            assert st == b.LORA_CACHE_LOADING, st
            c.wait()
            lat[ranks[a]].append(time.perf_counter() - t0)
    # back-to-back loads (cap 4 in flight) of 4 adapters not resident
    miss = [a for a in range(n_ad) if c.slot_of(a) < 0][:4]
    t0 = time.perf_counter()
    for a in miss:
        assert c.request(a) == b.LORA_CACHE_LOADING
    c.wait()
    burst_s = time.perf_counter() - t0
    burst_bytes = sum(blob_bytes[ranks[a]] for a in miss)

    # decode steps with and without loads in flight
    reps = 50
    for _ in range(5):
        decode_graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        decode_graph.replay()
    torch.cuda.synchronize()
    idle_s = (time.perf_counter() - t0) / (reps * R)
    miss = [a for a in range(n_ad) if c.slot_of(a) < 0][:4]
    t0 = time.perf_counter()
    for a in miss:
        assert c.request(a) == b.LORA_CACHE_LOADING
    for _ in range(reps):
        decode_graph.replay()
    torch.cuda.synchronize()
    busy_s = (time.perf_counter() - t0) / (reps * R)
    n_done = c.poll()
    c.wait()
    st = c.stats()
    c.destroy()
    pct = lambda v, q: float(sorted(v)[min(len(v) - 1, int(round(q * (len(v) - 1))))])
    out = dict(adapter="8B-shaped, 32 layers x 7 projections, bf16", slots=n_slots,
               blob_MB={str(r): round(v / 1e6, 2) for r, v in blob_bytes.items()})
    for r in (8, 16):
        v = lat[r]
        out[f"rank{r}"] = dict(loads=len(v), cold_load_ms_p50=round(pct(v, 0.5) * 1e3, 3),
                               cold_load_ms_p95=round(pct(v, 0.95) * 1e3, 3),
                               h2d_GBps_p50=round(blob_bytes[r] / pct(v, 0.5) / 1e9, 1))
    out["burst"] = dict(loads=len(miss), MB=round(burst_bytes / 1e6, 1), ms=round(burst_s * 1e3, 3),
                        h2d_GBps=round(burst_bytes / burst_s / 1e9, 1))
    out["decode_step_us_idle"] = round(idle_s * 1e6, 3)
    out["decode_step_us_while_loading"] = round(busy_s * 1e6, 3)
    out["loads_completed_during_decode"] = n_done
    out["evictions"] = st["evictions"]
    return out


def bench_serving(torch, args):
    """A decode serving loop on one q projection (4096 -> 4096, rank 16):
    single-token requests with adapter ids ~ Zipf(1.1) over 1000 adapters
    kept on the host, a standing backlog of 256 requests plus Poisson(32)
    arrivals per step (the queue is saturated, so admission has a choice);
    each step the admission scheduler forms a batch of at most 32 rows, the
    slot cache (250 slots) maps it to slots, and lora_layer_apply runs it.
    A load started in a step completes before the next step (the cache
    completes loads only where the loop waits), so the run depends on the
    seed alone.
    Reported per policy (the page's locality weight 0.35; 0 = first come
    first served; a strong weight of 8; 0.35 with a cap of 8 adapters per
    batch): distinct
    adapters per step (the cost driver), cache hit rate, queue waits in
    steps (overall and for the less popular half of the adapters), and the
    GPU time of the last 64 batches the loop formed, graph-replayed over
    eight copies of W in turn, against the base-only decode of the same rows
    and weights (adapter overhead fraction)."""
    from lora_bgmv_shrink_amd import binding as b
    from lora_bgmv_shrink_amd import workloads as wl

    dev = torch.device("cuda:0")
    d, r, n_ad, n_slots, rows_max = 4096, 16, 1000, 250, 32
    g = wl._gen(dev, 9200)
    W = wl._randn(g, (d, d), wl.W_DIV, torch.bfloat16, dev)          # stored [d_out, d_in]
    x = wl._randn(g, (rows_max, d), 1.0, torch.bfloat16, dev)
    out = {}
    for label, w_local, cap in (("locality_0.35", 0.35, rows_max), ("fifo", 0.0, rows_max),
                                ("locality_8", 8.0, rows_max), ("locality_0.35_cap8", 0.35, 8)):
        # loads complete only where the loop waits for them (after each
        # step's batch), so one seed always forms the same batches
        c = b.Cache(torch.bfloat16, [(d, d)], r, n_ad, n_slots, 8, device=dev, explicit_poll=True)
        n_el = c.blob_layout(r)[2]
        blobs = torch.empty(n_ad * n_el, dtype=torch.bfloat16, pin_memory=True)
        blobs.copy_((torch.randn(n_ad * n_el, generator=g, device=dev) / 32).to(torch.bfloat16))
        for a in range(n_ad):
            c.register_blob(a, r, 2.0, blobs[a * n_el:(a + 1) * n_el])
        sch = b.Scheduler(n_ad, 1.0, w_local, max_adapters=cap, max_rows=rows_max, cache=c)
        rng = np.random.default_rng(77)
        p = wl.zipf_probs(n_ad, 1.1)
        steps, warm = 1500, 300
        distinct, waits_all, waits_tail, last, n_rows = [], [], [], [], []
        rid = 0
        stats0 = None
        for step in range(steps):
            k = int(rng.poisson(32)) + (256 if step == 0 else 0)
            ids = rng.choice(n_ad, size=k, p=p)
            for j, a in enumerate(ids):
                sch.submit(rid, int(a), 1, step + (j + 0.5) / max(k, 1))
                rid += 1
            (req, ad, rw, wt), info = sch.step(float(step + 1), rows_max)
            if step == warm:
                stats0 = c.stats()
            n = len(ad)
            if n == 0:
                c.wait()
                continue
            slots = c.map(ad)
            b.lora_layer_apply(c.pool(0), x[:n], W, torch.as_tensor(slots, device=dev), w_layout=b.LORA_W_OUT_IN,
                               mode=b.LORA_MODE_BGMV)
            c.release()
            c.wait()   # the loads this step started are resident from the next step on
            if step >= warm:
                n_rows.append(n)
                distinct.append(info["distinct_adapters"])
                waits_all.extend(wt.tolist())
                waits_tail.extend(wt[ad >= n_ad // 2].tolist())
            if step >= steps - 64:
                last.append(slots.copy())
        torch.cuda.synchronize()
        c.wait()                      # no copy in flight while the batches are timed
        st = c.stats()
        # GPU time of the last batches (their slots are still those adapters'
        # or others of the same rank; the time does not depend on the values)
        pool = c.pool(0)
        ids_l = [torch.as_tensor(sl, device=dev) for sl in last]
        ys = [torch.empty((len(sl), d), dtype=torch.bfloat16, device=dev) for sl in last]
        ws = torch.zeros(b.lora_layer_workspace(pool, rows_max, b.LORA_MODE_BGMV), dtype=torch.uint8, device=dev)
        wsb = torch.zeros(b.lora_decode_workspace(pool, rows_max, False), dtype=torch.uint8, device=dev)
        # batch i runs on weight copy i % 8: eight 33.5 MB copies outgrow the
        # 256 MB last-level cache, so each batch reads its W from HBM as a
        # layer of a real model would (one W would stay cached across batches)
        Ws = [W] + [W.clone() for _ in range(7)]
        g_lora = capture(torch, lambda: [b.lora_layer_apply(pool, x[:len(sl)], Ws[i % 8], ii,
                                                            w_layout=b.LORA_W_OUT_IN,
                                                            mode=b.LORA_MODE_BGMV, y=yy, ws=ws)
                                         for i, (sl, ii, yy) in enumerate(zip(last, ids_l, ys))])
        g_base = capture(torch, lambda: [(b.lora_decode_stream(pool, x[:len(sl)], Ws[i % 8], ii, wsb, False),
                                          b.lora_decode_finish(pool, ii, wsb, yy, False))
                                         for i, (sl, ii, yy) in enumerate(zip(last, ids_l, ys))])
        lora_us = time_graph(torch, g_lora, 20) / len(last) * 1e6
        base_us = time_graph(torch, g_base, 20) / len(last) * 1e6
        hits = st["hits"] - stats0["hits"]
        loads = st["loads_started"] - stats0["loads_started"]
        q = lambda v, f: round(float(np.quantile(np.asarray(v, np.float64), f)), 3) if len(v) else None
        out[label] = dict(
            w_local=w_local, max_adapters=cap, steps=len(distinct), rows_per_step=round(float(np.mean(n_rows)), 2),
            distinct_adapters_per_step=dict(p10=q(distinct, .1), p50=q(distinct, .5), p90=q(distinct, .9),
                                            max=int(max(distinct))),
            gpu_step_us=round(lora_us, 3), base_only_step_us=round(base_us, 3),
            adapter_overhead_fraction=round(max(0.0, (lora_us - base_us) / lora_us), 4),
            cache_hit_rate=round(hits / max(1, hits + loads), 4), loads=loads,
            wait_steps=dict(p50=q(waits_all, .5), p99=q(waits_all, .99)),
            wait_steps_less_popular_half=dict(p50=q(waits_tail, .5), p99=q(waits_tail, .99), n=len(waits_tail)))
        del g_lora, g_base
        sch.destroy()
        c.destroy()
        del blobs
    return out


def bench_q4_decode(torch, args):
    """The headline decode batch (q 4096 -> 4096, rank 16, 32 rows on 20
    adapters of a pool of 250) over a 4-bit base weight with bf16 adapters:
    lora_decode_stream_q4 + lora_decode_finish, graph-replayed over 24
    replicas (each its own weight, pool and x; the step's working set times
    24 exceeds the Infinity Cache).  The stream launch's algorithmic bytes:
    the 4-bit weight, its scales, the distinct adapters' A blocks, x and the
    ids."""
    from lora_bgmv_shrink_amd import binding as b
    from lora_bgmv_shrink_amd import workloads as wl

    dev = torch.device("cuda:0")
    R = 24
    reps = []
    for r in range(R):
        w = wl.decode_q_proj(device=dev, value_seed=None if r == 0 else 7 + 1000 * r)
        p = w.projections[0]
        p.W = None
        pool = make_pool(b, p.pool)
        Wq, sc = wl.q4_weight(100 + r, 4096, 4096, dev)
        n = w.n_rows
        ids = torch.as_tensor(w.ids, device=dev)
        reps.append(dict(w=w, p=p, pool=pool, Wq=Wq, sc=sc, ids=ids,
                         y=torch.zeros((n, 4096), dtype=torch.bfloat16, device=dev),
                         ws=torch.zeros(b.lora_decode_workspace(pool, n, True), dtype=torch.uint8, device=dev),
                         wsb=torch.zeros(b.lora_decode_workspace(pool, n, False), dtype=torch.uint8, device=dev)))
    n = reps[0]["w"].n_rows

    def stream(r, lora=True):
        b.lora_decode_stream_q4(r["pool"], r["p"].x, r["Wq"], r["sc"], r["ids"], r["ws" if lora else "wsb"], lora)

    def finish(r, lora=True):
        b.lora_decode_finish(r["pool"], r["ids"], r["ws" if lora else "wsb"], r["y"], lora)

    g_step = capture(torch, lambda: [(stream(r), finish(r)) for r in reps])
    g_stream = capture(torch, lambda: [stream(r) for r in reps])
    g_base = capture(torch, lambda: [(stream(r, False), finish(r, False)) for r in reps])
    kr = max(4, args.kernel_reps // 2)
    d_step = time_graph(torch, g_step, kr) / R
    d_stream = time_graph(torch, g_stream, kr) / R
    d_base = time_graph(torch, g_base, kr) / R
    pool = reps[0]["p"].pool
    bA, U = distinct_bytes(pool, reps[0]["w"].ids, "A")
    wbytes = 4096 * 4096 // 2 + 4096 * (4096 // 128) * 4
    stream_bytes = wbytes + bA + n * 4096 * 2 + n * 4
    out = dict(workload="decode_q4base_q4096_r16_pool250_rows32", replicas=R, distinct_adapters=U,
               step_us=round(d_step * 1e6, 3), tokens_per_s=round(n / d_step, 1),
               base_only_step_us=round(d_base * 1e6, 3),
               overhead_fraction=round(max(0.0, (d_step - d_base) / d_step), 4),
               stream_us=round(d_stream * 1e6, 3), stream_bytes=stream_bytes,
               stream_GBps=round(stream_bytes / d_stream / 1e9, 1),
               stream_frac_hbm=round(stream_bytes / d_stream / 1e9 / HBM_PEAK_GBS, 4))
    del g_step, g_stream, g_base, reps
    torch.cuda.empty_cache()
    return out


def bench_q4_prefill(torch, args):
    """The 70B prefill batch (13,894 rows in arrival order, 8 rank-64
    adapters, seven projections) over 4-bit base weights with bf16 adapters:
    lora_layer_apply_q4 per projection, segments built once per step,
    graph-replayed.  MFMA fraction against the bf16 peak (the 4-bit weights
    are widened to bf16 for the matrix cores)."""
    from lora_bgmv_shrink_amd import binding as b
    from lora_bgmv_shrink_amd import workloads as wl

    dev = torch.device("cuda:0")
    w = wl.prefill_70b(device=dev)
    n = w.n_rows
    ids = torch.as_tensor(w.ids, device=dev)
    projs, flops, wbytes = [], 0, 0
    for i, pp in enumerate(w.projections):
        pp.W = None
        Wq, sc = wl.q4_weight(200 + i, pp.d_in, pp.d_out, dev)
        h = make_pool(b, pp.pool)
        projs.append(dict(p=pp, Wq=Wq, sc=sc, h=h, y=torch.empty((n, pp.d_out), dtype=torch.bfloat16, device=dev)))
        flops += 2 * n * pp.d_in * pp.d_out + 2 * n * 64 * (pp.d_in + pp.d_out)
        wbytes += pp.d_in * pp.d_out // 2 + pp.d_out * (pp.d_in // 128) * 4
    ws = torch.zeros(max(b.lora_layer_q4_workspace(pr["h"], n) for pr in projs), dtype=torch.uint8, device=dev)
    seg = b.segments_alloc(n, 64, dev)

    def step():
        b.lora_segments_build(ids, 64, seg=seg)
        for pr in projs:
            b.lora_layer_apply_q4(pr["h"], pr["p"].x, pr["Wq"], pr["sc"], ids, seg=seg, y=pr["y"], ws=ws)

    g = capture(torch, step)
    d = time_graph(torch, g, max(2, args.extra_steps // 2))
    out = dict(workload="prefill_q4base_70b_r64_pool64", rows=n, ms_per_step=round(d * 1e3, 4),
               tokens_per_s_seven_projections=round(n / d, 1), tflops=round(flops / d / 1e12, 1),
               mfma_frac=round(flops / d / 1e12 / BF16_PEAK_TFLOPS, 4), weight_bytes=wbytes)
    for pr in projs:
        pr["h"].destroy()
    del g, projs, ws
    torch.cuda.empty_cache()
    return out


def bench_sgmv_adapter_term(torch, args):
    """The adapter term of the 70B prefill batch on its own (13,894 rows in
    arrival order, 8 rank-64 adapters, q and o projections 8192 -> 8192):
    lora_sgmv_shrink (t = x A per segment, K split over its workspace) and
    lora_sgmv_expand accumulating
    s t B into y, each graph-replayed alternately over the two projections
    (x and y of one are 228 MB, so the pair exceeds the Infinity Cache).
    Algorithmic bytes: shrink = x + the distinct A blocks + t; expand = t +
    the distinct B blocks + y read and written."""
    from lora_bgmv_shrink_amd import binding as b
    from lora_bgmv_shrink_amd import workloads as wl

    dev = torch.device("cuda:0")
    w = wl.prefill_70b(device=dev, projections=["q", "o"])
    n = w.n_rows
    ids = torch.as_tensor(w.ids, device=dev)
    pr = []
    for pp in w.projections:
        pp.W = None
        h = make_pool(b, pp.pool)
        pr.append(dict(p=pp, h=h, t=torch.zeros((n, pp.pool.r_max), dtype=torch.float32, device=dev),
                       y=torch.zeros((n, pp.d_out), dtype=torch.bfloat16, device=dev)))
    seg = b.lora_segments_build(ids, pr[0]["p"].pool.n_adapters)
    for r in pr:   # K-split partial sums of the shrink (no zeroing needed)
        r["ws"] = torch.empty(max(1, b.lora_sgmv_shrink_workspace(r["h"], n)), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    g_shr = capture(torch, lambda: [b.lora_sgmv_shrink(r["h"], r["p"].x, seg, t=r["t"], ws=r["ws"]) for r in pr])
    g_exp = capture(torch, lambda: [b.lora_sgmv_expand(r["h"], r["t"], seg, y=r["y"], accumulate=True) for r in pr])
    reps = max(4, args.extra_steps)
    d_shr = time_graph(torch, g_shr, reps) / len(pr)
    d_exp = time_graph(torch, g_exp, reps) / len(pr)
    pool = pr[0]["p"].pool
    bA, U = distinct_bytes(pool, w.ids, "A")
    bB, _ = distinct_bytes(pool, w.ids, "B")
    d_in, d_out, r = pool.d_in, pool.d_out, pool.r_max
    shr_bytes = n * d_in * 2 + bA + n * r * 4
    exp_bytes = n * r * 4 + bB + 2 * n * d_out * 2
    out = dict(workload="prefill_sgmv_70b_q_o_r64_rows%d" % n, rows=n, distinct_adapters=U,
               sgmv_shrink=dict(us=round(d_shr * 1e6, 2), bytes=shr_bytes, GBps=round(shr_bytes / d_shr / 1e9, 1),
                                frac_hbm=round(shr_bytes / d_shr / 1e9 / HBM_PEAK_GBS, 4)),
               sgmv_expand=dict(us=round(d_exp * 1e6, 2), bytes=exp_bytes, GBps=round(exp_bytes / d_exp / 1e9, 1),
                                frac_hbm=round(exp_bytes / d_exp / 1e9 / HBM_PEAK_GBS, 4)))
    del g_shr, g_exp, pr
    torch.cuda.empty_cache()
    return out


def bench_merge(torch, args):
    """lora_merge_adapter (W += s A_a B_a in place) on 8B and 70B q_proj
    shapes: merges then unmerges over 4 weight replicas (more than the
    Infinity Cache holds), captured in a graph; HBM GB/s of the algorithmic
    bytes (W read and written once, A_a and B_a read once)."""
    from lora_bgmv_shrink_amd import binding as b
    from lora_bgmv_shrink_amd import workloads as wl

    dev = torch.device("cuda:0")
    out = {}
    for label, d, r in (("q_proj_8b_r16", 4096, 16), ("q_proj_70b_r64", 8192, 64)):
        g = wl._gen(dev, 7000 + d + r)
        pool_w = wl.make_uniform_pool(g, dev, torch.bfloat16, 8, d, d, r)
        h = make_pool(b, pool_w)
        Ws = [wl._randn(g, (d, d), wl.W_DIV, torch.bfloat16, dev) for _ in range(4)]

        def step():
            for Wt in Ws:
                b.lora_merge_adapter(h, Wt, 3, w_layout=b.LORA_W_OUT_IN, sign=1.0)
            for Wt in Ws:
                b.lora_merge_adapter(h, Wt, 3, w_layout=b.LORA_W_OUT_IN, sign=-1.0)

        gr = capture(torch, step)
        sec = time_graph(torch, gr, max(2, args.extra_steps)) / (2 * len(Ws))
        nbytes = 2 * d * d * 2 + r * (d + d) * 2
        out[label] = dict(d_in=d, d_out=d, rank=r, us_per_merge=round(sec * 1e6, 2),
                          GBps=round(nbytes / sec / 1e9, 1), frac_hbm=round(nbytes / sec / 1e9 / HBM_PEAK_GBS, 4),
                          bytes_per_merge=nbytes)
        del Ws, gr
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this layer is built and measured on a single MI355X; "
              f"--gpus {args.gpus} (WORLD_SIZE={world}) is not supported.", file=sys.stderr)
        sys.exit(2)
    import torch

    log("bench: decode q_proj (BGMV) ...")
    dec, w0 = bench_decode(torch, args)
    if args.copy_probe:
        # a plain elementwise kernel of known size: reads 256 MiB, writes 256 MiB
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    extra = {}
    for name in [s for s in args.workloads.split(",") if s]:
        log(f"bench: workload {name} ...")
        extra[name] = bench_multi(torch, args, name)
        torch.cuda.empty_cache()
    merge = q4 = sgmv = q4p = None
    if not args.no_extras:
        log("bench: merge kernel ...")
        merge = bench_merge(torch, args)
        log("bench: 4-bit base decode ...")
        q4 = bench_q4_decode(torch, args)
        log("bench: SGMV adapter term (prefill) ...")
        sgmv = bench_sgmv_adapter_term(torch, args)
        if "prefill" in args.workloads.split(","):
            log("bench: 4-bit base prefill ...")
            q4p = bench_q4_prefill(torch, args)
    decode = dec.pop("_decode_graph")
    paging = serving = None
    if not args.no_paging:
        log("bench: adapter paging ...")
        paging = bench_paging(torch, args, decode, args.replicas)
        log("bench: serving loop (admission + cache + layer) ...")
        serving = bench_serving(torch, args)
    del decode
    cpu = None
    if not args.no_cpu:
        log("bench: cpu baseline (oracle) ...")
        # the oracle needs W in [d_in, d_out]; regenerate replica 0's values
        from lora_bgmv_shrink_amd import workloads as wl
        wc = wl.decode_q_proj(device=torch.device("cuda:0"))
        cpu = cpu_baseline(wc, args.cpu_seconds)

    line = {
        "metric": "LoRA-layer tokens/s; adapter-term HBM GB/s (% peak), BGMV decode + SGMV prefill",
        "value": round(dec["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(dec["sec_step"] * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_bgmv_q4096_r16_pool250_rows32", "rows": 32, "d_in": 4096,
                   "d_out": 4096, "rank": 16, "pool": 250, "distinct_adapters": 20, "base_only_rows": 3,
                   "w_layout": "out_in", "replicas": args.replicas, "graph": True},
        "roofline": dec["roofline"],
        "cpu_baseline": cpu,
        "kernels_us": dec["kernels_us"],
        "adapter_term": dec["adapter_term"],
        "comparators": dec["comparators"],
        "diversity_sweep_rows32": dec["diversity_sweep"],
        "gpu_step_us": round(dec["gpu_step_s"] * 1e6, 3),
        "workloads": extra,
        "merge": merge,
        "q4_decode": q4,
        "q4_prefill": q4p,
        "adapter_term_prefill": sgmv,
        "paging": paging,
        "serving": serving,
    }
    if cpu:
        line["gpu_over_cpu"] = round(line["value"] / cpu["value"], 1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
