"""Benchmark of the DSA indexer hot path on one MI355X.

A step is one pass of the whole path over one batch of synthetic input:
    xk_indexer_logits -> xk_indexer_topk -> xk_mxfp4_paged_gather
Prints ONE JSON line. The headline workload is the long-context fp8 chunked
prefill (T=2048 queries at causal offset 96256 against K=98304 OCP-e4m3
keys, top-1024), the largest single-GPU shape. `value` is the indexer-logits
throughput of the whole step (algorithmic logits FLOPs / step wall time),
`topk_gather_GBps` the algorithmic bytes of top-k + gather over their kernel
time; `stages` has every kernel's average duration against its roof (plus
per-dispatch percentiles, warm and after a 512 MiB cache flush), and
`roofline` repeats the dominant kernel. Prefill configs also time the fused
step (xk_indexer_logits_topk -> gather, no score matrix) under `fused`, and
the sparse attention that consumes the selection under `consumer` (not part
of the step). `other_configs` gives the stage table of the Flash decode,
Flash prefill and Pro decode workloads measured in the same run.

Steps are replayed from HIP graphs: one graph holds a round of steps, one
per input copy, so the timed loop measures the GPU rather than Python's or
the graph launch's cost; before timing, replays are checked bit for bit
against an eager step, and `ms_per_step_eager` reports eager launches too.
A kernel's average duration is timed with HIP events on the launch stream
around replays of a graph of 20 back-to-back launches of that kernel alone
(rotating the input copies), so no launch gap is counted.

Inputs are resident in HBM before timing starts. Several identical copies of
q/k/w are rotated across steps so that a decode-sized working set cannot be
served from the 256 MB last-level cache instead of HBM.

    python bench.py [--steps K] [--warmup W] [--config long_fp8_prefill]
    python bench.py --kernel logits [--config C] [--steps N]   (one stage only, for profilers)
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer logits TFLOP/s & top-k+mxfp4 gather GB/s, % of MI355X roofline"
PEAK = {"hbm": 8000.0, "mfma_bf16": 2500.0, "mfma_fp8": 5000.0}   # GB/s, TFLOP/s (dense)
FLOP_PER_PAIR = 2 * 64 * 128
DEFAULT_CONFIG = "long_fp8_prefill"
EXTRA_CONFIGS = "flash_decode,flash_prefill,pro_decode"
FLUSH_BYTES = 512 << 20   # written before each cold dispatch: twice the 256 MB last-level cache


def algorithmic_work(x, sel_pos=None):
    """Per-step algorithmic FLOPs and bytes of each stage (what the method must move)."""
    cfg = x["cfg"]
    eb = 2 if cfg.dtype == "bf16" else 1
    lim = x["limit"].astype(np.int64)
    n_valid = np.clip(lim + 1, 0, cfg.K)                      # [B,T]
    pairs = int(n_valid.sum())
    keys_read = int(n_valid.max(axis=1).sum())                # distinct valid key rows
    if cfg.kcache == "mxfp4":
        key_bytes = keys_read * (64 + 4)                       # E2M1 nibbles + E8M0 bytes
    elif cfg.kcache == "fp8":
        key_bytes = keys_read * (128 + 4)                      # e4m3 + fp32 scale
    else:
        key_bytes = keys_read * 128 * eb + (keys_read * 4 if cfg.dtype == "fp8" else 0)
    if cfg.kcache is not None:                                 # block-table entries read
        key_bytes += int(((n_valid.max(axis=1) + x["block_size"] - 1) // x["block_size"]).sum()) * 4
    logits_bytes = key_bytes + cfg.rows * 64 * 128 * eb + cfg.rows * 64 * 4 + pairs * 4
    if cfg.dtype == "fp8":
        logits_bytes += cfg.rows * 64 * 4                      # q scales
    topk_bytes = pairs * 4 + cfg.rows * cfg.topk * 4
    slots = cfg.rows * cfg.topk
    distinct = slots
    if sel_pos is not None:
        seq = np.repeat(x["row_seq"].astype(np.int64), cfg.topk)
        p = sel_pos.reshape(-1).astype(np.int64)
        ok = p >= 0
        distinct = int(np.unique(seq[ok] * (1 << 32) + p[ok]).size)
    gather_bytes = slots * (256 + 4) + distinct * 68
    return {"pairs": pairs, "logits_flops": pairs * FLOP_PER_PAIR, "logits_bytes": logits_bytes,
            "topk_bytes": topk_bytes, "gather_bytes": gather_bytes, "distinct_rows": distinct}


# the sources each stage's kernel is built from (a byte-counter summary is
# valid only for the sources it was taken on)
STAGE_SOURCES = {
    "logits": ("logits.hip", "tile16.h", "xk_internal.h"),
    "topk": ("topk.hip", "tile16.h", "xk_internal.h"),
    "gather": ("gather.hip", "mxfp4.h", "xk_internal.h"),
}


def source_hash(stage=None):
    """sha256 prefix of one stage's kernel sources (all of csrc/ without a stage)."""
    csrc = os.path.join(ROOT, "sparse_attention_indexer_logits_amd", "csrc")
    files = ([os.path.join(csrc, f) for f in STAGE_SOURCES[stage]] if stage
             else sorted(glob.glob(os.path.join(csrc, "*"))))
    h = hashlib.sha256()
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(config, kernel_stage):
    """HBM bytes per launch of a stage's kernel from a committed rocprofv3
    --pmc summary (profiles/traffic_<config>.txt), if it was taken on the
    stage's current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{config}.txt")
    if not os.path.exists(path):
        return None
    src, vals = {}, {}
    for line in open(path):
        parts = line.split()
        if len(parts) == 3 and parts[0] == "kernel_source_sha":
            src[parts[1]] = parts[2]
        elif len(parts) == 3 and parts[0] == "traffic_bytes_per_launch":
            vals[parts[1]] = float(parts[2])
    if kernel_stage not in vals or src.get(kernel_stage) != source_hash(kernel_stage):
        return None
    return vals[kernel_stage]


def host_cores():
    """Threads the numpy oracle runs on (its BLAS pool; the rest of numpy is
    single-threaded) next to the host's cores: those this process may run
    on, and the machine's count."""
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        blas = 1
    return {"threads_used": int(min(blas, affinity)), "blas_threads": int(blas), "affinity": affinity,
            "cpu_count": os.cpu_count()}


def cpu_baseline(x, work, budget_s):
    """The oracle as it stands, on a bounded sample of the step's query rows."""
    import oracle
    cores = host_cores()
    cfg = x["cfg"]
    R = cfg.rows
    order = np.random.default_rng(0).permutation(R)

    def run(n):
        rows = np.sort(order[:n])
        pairs = [(int(r) // cfg.T, int(r) % cfg.T) for r in rows]
        t0 = time.perf_counter()
        if cfg.kcache is None:
            L = oracle.indexer_logits(x["q"], x["k"], x["w"], x["limit"], x["q_scale"],
                                      x["k_scale"], cfg.dtype, rows=pairs)
        else:
            L = oracle.indexer_logits_paged(x["q"], x["q_scale"], x["w"], x["limit"], x["kc"],
                                            x["kc_scale"], x["block_table"], x["block_size"],
                                            cfg.K, cfg.kcache, rows=pairs)
        L = L.reshape(R, cfg.K)
        idx = oracle.indexer_topk(L, x["limit"].reshape(-1), cfg.topk, rows=rows)
        oracle.mxfp4_paged_gather(x["kv_fp4"], x["kv_scale"], x["block_table"], idx,
                                  x["row_seq"], x["block_size"], rows=rows)
        return time.perf_counter() - t0, rows

    # the first row also pays one-time costs (dequantizing the sequence's
    # keys), so the sample grows until it fills about the budget
    t1, _ = run(1)
    n = int(min(R, max(1, budget_s / max(t1, 1e-6))))
    tn, rows = run(n)
    while tn < 0.5 * budget_s and n < R:
        n = int(min(R, max(n + 1, n * 0.8 * budget_s / max(tn, 1e-6))))
        tn, rows = run(n)
    if n < R:
        frac = float(np.clip(x["limit"].reshape(-1)[rows] + 1, 0, cfg.K).sum()) / max(work["pairs"], 1)
        step_s = tn / max(frac, 1e-12)          # scale by the share of the step's pairs done
        sample = (f"{n} of {R} query rows (logits + top-k + gather, float64 numpy), {tn:.1f} s, "
                  "scaled by their share of the step's valid pairs")
    else:
        total, reps = 0.0, 0
        while total < budget_s or reps == 0:    # whole steps, repeated to fill the budget
            t, _ = run(R)
            total, reps = total + t, reps + 1
        step_s = total / reps
        sample = (f"{reps} whole steps ({R} query rows each: logits + top-k + gather, float64 "
                  f"numpy), {total:.1f} s")
    return {"value": work["logits_flops"] / step_s / 1e12, "unit": "TFLOP/s", "cores": cores["threads_used"],
            "host_cores": cores["affinity"], "host_cpu_count": cores["cpu_count"],
            "blas_threads": cores["blas_threads"], "kind": "oracle", "sample": sample,
            "ms_per_step": step_s * 1e3}


def cpu_table(args):
    """The CPU oracle per stage on the host's cores and on one thread, for the
    tiny, Flash decode and Flash prefill workloads: whole steps where they
    take seconds, else a bounded sample of query rows scaled by its share of
    the step's valid pairs. One JSON line."""
    import oracle
    import workloads
    from threadpoolctl import threadpool_limits

    cores = host_cores()
    table = {}
    for name in ("tiny", "flash_decode", "flash_prefill"):
        x = workloads.inputs(name)
        cfg = x["cfg"]
        R = cfg.rows
        lim = x["limit"].reshape(-1)
        n_valid = np.clip(lim.astype(np.int64) + 1, 0, cfg.K)
        order = np.random.default_rng(0).permutation(R)
        row = {}
        n = None  # sample size, fixed by the all-cores run and reused on one thread
        for threads in (cores["threads_used"], 1):
            with threadpool_limits(limits=threads):
                def run(n):
                    rows = np.sort(order[:n])
                    pairs = [(int(r) // cfg.T, int(r) % cfg.T) for r in rows]
                    t = {}
                    t0 = time.perf_counter()
                    L = oracle.indexer_logits(x["q"], x["k"], x["w"], x["limit"], x["q_scale"], x["k_scale"],
                                              cfg.dtype, rows=pairs).reshape(R, cfg.K)
                    t["logits"] = time.perf_counter() - t0
                    t0 = time.perf_counter()
                    idx = oracle.indexer_topk(L, lim, cfg.topk, rows=rows)
                    t["topk"] = time.perf_counter() - t0
                    t0 = time.perf_counter()
                    oracle.mxfp4_paged_gather(x["kv_fp4"], x["kv_scale"], x["block_table"], idx, x["row_seq"],
                                              x["block_size"], rows=rows)
                    t["gather"] = time.perf_counter() - t0
                    return t, rows
                if n is None:
                    t1, _ = run(1)
                    n = int(min(R, max(1, args.cpu_budget / 3 / max(sum(t1.values()), 1e-6))))
                t, rows = run(n)
                share = float(n_valid[rows].sum()) / max(float(n_valid.sum()), 1.0)
                row[f"threads_{threads}"] = {
                    "ms_per_step": {k: v / share * 1e3 for k, v in t.items()},
                    "sample": f"{n} of {R} query rows" + ("" if n == R else ", scaled by their share of the valid pairs")}
        table[name] = row
    print(json.dumps({"cpu_oracle_per_stage": table, "host_cores": cores["affinity"],
                      "host_cpu_count": cores["cpu_count"], "blas_threads": cores["blas_threads"],
                      "kind": "oracle (float64 numpy)"}), flush=True)


def producers(args):
    """The producers of the path's quantized inputs on a config's shapes: q
    (B*T*64 rows) and k (the valid keys) quantized per row to OCP fp8, and k
    written into the paged mxfp4 cache. Inputs are bf16 rows resident in HBM,
    drawn N(0,1) with a per-row power-of-two spread; one JSON line."""
    import torch
    import oracle
    import workloads
    import sparse_attention_indexer_logits_amd as xk

    cfg = workloads.CONFIGS[args.config]
    rng = np.random.default_rng(cfg.seed)
    nq = cfg.rows * 64
    nk = int(workloads.seq_lengths(cfg).sum())
    bs = workloads.BLOCK_SIZE
    NB = (nk + bs - 1) // bs

    def draw(n):
        x = rng.standard_normal((n, 128), dtype=np.float32) * np.exp2(rng.integers(-4, 4, (n, 1)))
        return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)

    qx, kx = draw(nq), draw(nk)
    slots = torch.from_numpy(rng.permutation(NB * bs)[:nk].astype(np.int64))
    dq, dk, ds = qx.cuda(), kx.cuda(), slots.cuda()
    q8 = torch.empty((nq, 128), dtype=torch.uint8, device="cuda")
    qs = torch.empty((nq,), dtype=torch.float32, device="cuda")
    k8 = torch.empty((nk, 128), dtype=torch.uint8, device="cuda")
    ks = torch.empty((nk,), dtype=torch.float32, device="cuda")
    kv = torch.zeros((NB, bs, 64), dtype=torch.uint8, device="cuda")
    kvs = torch.zeros((NB, bs, 4), dtype=torch.uint8, device="cuda")
    runs = {
        "quant_fp8_q": (lambda: xk.xk_quant_fp8_rows(dq, out=q8, scale=qs), nq * (256 + 128 + 4)),
        "quant_fp8_k": (lambda: xk.xk_quant_fp8_rows(dk, out=k8, scale=ks), nk * (256 + 128 + 4)),
        "mxfp4_write_k": (lambda: xk.xk_mxfp4_cache_write(dk, ds, kv, kvs), nk * (256 + 8 + 68)),
    }
    # checked pass: the GPU results against the oracle on the first rows
    for f, _ in runs.values():
        f()
    torch.cuda.synchronize()
    n_chk = min(4096, nk)
    c, s_ = oracle.quant_fp8_rows(kx[:n_chk].float().numpy())
    if not (np.array_equal(k8[:n_chk].cpu().numpy(), c) and np.array_equal(ks[:n_chk].cpu().numpy(), s_)):
        raise RuntimeError("fp8 quantizer differs from the oracle")
    stages = {}
    total_bytes, total_s = 0, 0.0
    n_in_graph = 20
    for name, (f, nbytes) in runs.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n_in_graph):
                f()
        for _ in range(max(1, args.warmup // n_in_graph)):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, args.steps // n_in_graph)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        sec = e0.elapsed_time(e1) / 1e3 / (reps * n_in_graph)
        ach = nbytes / sec / 1e9
        stages[name] = {"bound": "hbm", "us": sec * 1e6, "achieved": ach, "peak": PEAK["hbm"],
                        "unit": "GB/s", "frac": ach / PEAK["hbm"], "bytes": nbytes}
        total_bytes += nbytes
        total_s += sec
    dom = max(stages, key=lambda k: stages[k]["us"])
    roof = {k: stages[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    roof["kernel"], roof["traffic"] = dom, None
    line = {
        "metric": "indexer input producers GB/s (fp8 row quantizer, mxfp4 cache writer)",
        "value": total_bytes / total_s / 1e9, "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": total_s * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16->fp8/mxfp4",
        "data": "synthetic: seeded N(0,1) bf16 rows with a per-row power-of-two spread",
        "config": {"workload": f"{cfg.name} producers", "q_rows": nq, "k_rows": nk, "D": 128,
                   "cache": "mxfp4 E2M1+E8M0, block 64"},
        "stages": stages, "roofline": roof,
    }
    if not args.no_cpu_baseline:
        cores = host_cores()
        n = min(nk, 65536)
        xs = kx[:n].float().numpy()
        t0 = time.perf_counter()
        oracle.quant_fp8_rows(xs)
        t_q = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.mxfp4_encode_rows(xs)
        t_e = time.perf_counter() - t0
        step_s = (nq + nk) * t_q / n + nk * t_e / n
        line["cpu_baseline"] = {"value": total_bytes / step_s / 1e9, "unit": "GB/s", "cores": cores["threads_used"],
                                "host_cores": cores["affinity"], "host_cpu_count": cores["cpu_count"],
                                "kind": "oracle",
                                "sample": f"{n} k rows quantized to fp8 ({t_q:.1f} s) and encoded to mxfp4 "
                                          f"({t_e:.1f} s), numpy, scaled to the step's q and k rows",
                                "ms_per_step": step_s * 1e3}
    print(json.dumps(line), flush=True)


def step_graphs(torch, steps, run):
    """One captured graph per step (input copy) and one holding a round of
    all of them in order."""
    graphs = []
    for s in steps:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            run(s)
        graphs.append(g)
    round_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(round_graph):
        for s in steps:
            run(s)
    torch.cuda.synchronize()
    return graphs, round_graph


def time_steps(torch, graphs, round_graph, n_steps, warmup):
    """Wall ms per step over exactly n_steps steps: whole rounds from the round
    graph (one launch per len(graphs) steps), the rest from single-step
    graphs; warm-up the same way, untimed."""
    n = len(graphs)

    def run(count):
        for _ in range(count // n):
            round_graph.replay()
        for i in range(count % n):
            graphs[i].replay()

    run(warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(n_steps)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / n_steps


def _graph_us(torch, launches, reps):
    """Average duration of one launch in a graph of back-to-back launches,
    timed with events on the launch stream."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in launches:
            f()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * len(launches))


def fused_timing(args, cfg, steps, n_sets, eager_out, ms):
    """Prefill shapes: the step with the fused logits -> top-k call in place of
    the two kernels (xk_indexer_logits_topk, then the gather). Its indices and
    gathered rows must equal the eager three-kernel step's bit for bit."""
    import torch
    ws = None
    for s in steps:
        ws = s.enable_fused(ws)
    base = steps[0]
    base.idx.fill_(-7)
    base.gathered.fill_(-7)
    base.run_fused()
    torch.cuda.synchronize()
    if not (torch.equal(base.idx, eager_out[1]) and torch.equal(base.gathered, eager_out[2])):
        raise RuntimeError("fused logits -> top-k differs from the three-kernel step")
    graphs, round_graph = step_graphs(torch, steps, lambda s: s.run_fused())
    ms_step = time_steps(torch, graphs, round_graph, args.steps, args.warmup)
    if not (torch.equal(base.idx, eager_out[1]) and torch.equal(base.gathered, eager_out[2])):
        raise RuntimeError("fused graph replays differ from the three-kernel step")
    n_in_graph = 20
    us = _graph_us(torch, [steps[i % n_sets].run_logits_topk for i in range(n_in_graph)],
                   max(1, args.steps // n_in_graph))
    unfused = (ms["logits"] + ms["topk"]) * 1e3
    return {"ms_per_step": ms_step, "logits_topk_us": us, "unfused_logits_plus_topk_us": unfused,
            "speedup_vs_unfused": unfused / us,
            "workspace_MiB": ws.numel() * ws.element_size() / 2 ** 20,
            "score_matrix_MiB": cfg.B * cfg.T * cfg.K * 4 / 2 ** 20,
            "note": "xk_indexer_logits_topk + gather; same indices and rows as the step"}


def consumer_timing(args, x, d, steps, n_sets):
    """The sparse attention that consumes the step's selection
    (xk_sparse_attention_mxfp4 on the top-k indices and the mxfp4 cache),
    timed like the step's kernels. Algorithmic work per valid slot: the
    cache row (64 B nibbles + 4 B scales) and its sel_pos entry, and
    4*H*128 FLOPs (scores and weighted sum); per row: q (bf16) and out
    (fp32)."""
    import torch
    import workloads
    import sparse_attention_indexer_logits_amd as xk
    cfg = x["cfg"]
    a = workloads.attention_inputs(cfg)
    H = a["q"].shape[1]
    q = torch.from_numpy(a["q"].view(np.int16)).cuda().view(torch.bfloat16)
    sink = torch.from_numpy(a["sink"]).cuda()
    idx = steps[0].idx
    n_valid = int((idx >= 0).sum().item())
    calls, outs = [], []  # outs keeps every output alive while launches hold its pointer
    for s in steps[:n_sets]:
        cargs, out = xk.attention_args(q, d["kv_fp4"], d["kv_scale"], d["block_table"], s.idx, d["row_seq"],
                                       sink, a["scale"])
        outs.append(out)
        calls.append(lambda c=cargs: xk._check(xk.lib().xk_sparse_attention_mxfp4(*c, xk._stream(None))))
    n_in_graph = 20
    us = _graph_us(torch, [calls[i % len(calls)] for i in range(n_in_graph)], max(1, args.steps // n_in_graph))
    torch.cuda.synchronize()
    del calls, outs
    nbytes = n_valid * (68 + 4) + cfg.rows * H * 128 * (2 + 4)
    flops = n_valid * 4 * H * 128
    gbps = nbytes / (us / 1e6) / 1e9
    tflops = flops / (us / 1e6) / 1e12
    bound = "hbm" if nbytes / (PEAK["hbm"] * 1e9) >= flops / (PEAK["mfma_bf16"] * 1e12) else "mfma"
    return {"us": us, "heads": H, "valid_slots": n_valid, "bytes": nbytes, "flops": flops,
            "GBps": gbps, "frac_hbm": gbps / PEAK["hbm"], "TFLOPs": tflops,
            "frac_bf16": tflops / PEAK["mfma_bf16"], "bound": bound,
            "note": "xk_sparse_attention_mxfp4 over the step's top-k (64 heads, sink, scale 1/sqrt(128))"}


def copy_calibration(nbytes=1 << 30, reps=4):
    """A plain device copy of known size, to scale rocprofv3 FETCH_SIZE/WRITE_SIZE."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": nbytes, "reps": reps}), flush=True)


def device_peaks(torch):
    """The GPU's CU count and peak clocks (HIP device attributes) and the
    rates reached on it, next to the spec peaks the fractions use: dense MFMA
    issue on the two prefill tile shapes (fp8 32x32x64, bf16 16x16x32; 4
    waves per SIMD, 4 independent accumulator chains each), a non-temporal
    2 GiB read stream, and torch's 1 GiB fill and copy (bytes moved / time)."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "sparse_attention_indexer_logits_amd", "libxk_peaks.so"))
    cus, clk, mclk = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    if lib.xkp_device_info(0, ctypes.byref(cus), ctypes.byref(clk), ctypes.byref(mclk)) != 0:
        raise RuntimeError("hipDeviceGetAttribute failed")
    props = torch.cuda.get_device_properties(0)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_ms(launch, reps=3):
        launch()   # warm-up
        ms = []
        for _ in range(reps):
            e0.record()
            launch()
            e1.record()
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        return min(ms)

    lib.xkp_mfma_loop.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    lib.xkp_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    blocks = 4 * cus.value          # 4 waves per workgroup: 4 waves per SIMD
    ops = torch.arange(64, dtype=torch.int32, device="cuda") * 0x01010101 % 0x3F3F3F3F
    sink = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    out = {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""), "compute_units": cus.value,
           "peak_clock_MHz": clk.value / 1e3, "memory_clock_MHz": mclk.value / 1e3, "measured": {}}
    meas = out["measured"]
    for kind, name, iters, flop in ((0, "mfma_fp8_32x32x64_TFLOPs", 2048, 2 * 32 * 32 * 64),
                                    (1, "mfma_bf16_16x16x32_TFLOPs", 8192, 2 * 16 * 16 * 32)):
        def launch(kind=kind, iters=iters):
            if lib.xkp_mfma_loop(kind, ops.data_ptr(), sink.data_ptr(), blocks, iters, stream) != 0:
                raise RuntimeError("MFMA probe launch failed")
        ms = best_ms(launch)
        meas[name] = blocks * 4 * 4 * iters * flop / (ms / 1e3) / 1e12
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(7)
    rblocks = 8 * cus.value
    rsink = torch.empty(rblocks * 256, dtype=torch.int32, device="cuda")

    def read():
        if lib.xkp_read_stream(src.data_ptr(), nbytes // 16, rsink.data_ptr(), rblocks, stream) != 0:
            raise RuntimeError("read probe launch failed")
    meas["hbm_read_GBps"] = nbytes / (best_ms(read) / 1e3) / 1e9
    # the same stream at decode-sized transfers (one launch of that many
    # bytes, timed back to back): the rate a launch of the decode stages'
    # size can reach at all
    for mib in (16, 64, 256):
        nb = mib << 20

        def read_n(nb=nb):
            if lib.xkp_read_stream(src.data_ptr(), nb // 16, rsink.data_ptr(), rblocks, stream) != 0:
                raise RuntimeError("read probe launch failed")
        meas[f"hbm_read_{mib}MiB_GBps"] = nb / (best_ms(read_n, reps=5) / 1e3) / 1e9
    del src, rsink
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    meas["hbm_fill_GBps"] = buf.numel() / (best_ms(lambda: buf.fill_(3)) / 1e3) / 1e9
    dst = torch.empty_like(buf)
    meas["hbm_copy_GBps"] = 2 * buf.numel() / (best_ms(lambda: dst.copy_(buf)) / 1e3) / 1e9
    del buf, dst
    meas["frac_of_spec"] = {
        "mfma_fp8": meas["mfma_fp8_32x32x64_TFLOPs"] / PEAK["mfma_fp8"],
        "mfma_bf16": meas["mfma_bf16_16x16x32_TFLOPs"] / PEAK["mfma_bf16"],
        "hbm_read": meas["hbm_read_GBps"] / PEAK["hbm"]}
    torch.cuda.synchronize()
    return out


def dispatch_us(torch, launches, flush=None):
    """Duration of each launch, timed alone with an event pair on the launch
    stream: p10/p50/p90 and mean in microseconds. With `flush` (a device
    buffer) the buffer is overwritten before each launch, so the launch
    starts with caches holding none of its inputs."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    vals = []
    for i, f in enumerate(launches):
        if flush is not None:
            flush.fill_(i & 0xFF)
        e0.record()
        f()
        e1.record()
        e1.synchronize()
        vals.append(e0.elapsed_time(e1) * 1e3)
    v = np.asarray(vals)
    return {"p10": float(np.percentile(v, 10)), "p50": float(np.percentile(v, 50)),
            "p90": float(np.percentile(v, 90)), "mean": float(v.mean()), "n": int(v.size)}


def setup(config, n_sets=0):
    """Inputs of a config on the device and its IndexerSteps (one per input
    copy, all writing the same outputs), after one checked eager step."""
    import torch
    import workloads
    from sparse_attention_indexer_logits_amd.pipeline import IndexerStep

    x = workloads.inputs(config)
    cfg = x["cfg"]
    d = workloads.to_device(x)
    in_bytes = sum(t.numel() * t.element_size() for key, t in d.items()
                   if key in ("q", "k", "w", "kc") and t is not None)
    n_sets = n_sets or int(min(16, max(1, -(-512 * 2 ** 20 // in_bytes))))

    def make_step(q, k, w, kc, outputs=None):
        return IndexerStep(q, k, w, d["limit"], cfg.topk, d["kv_fp4"], d["kv_scale"],
                           d["block_table"], d["row_seq"], d["q_scale"], d["k_scale"],
                           outputs=outputs, k_cache=kc, k_cache_scale=d.get("kc_scale"), K=cfg.K)

    base = make_step(d["q"], d["k"], d["w"], d.get("kc"))
    steps = [base]
    for _ in range(n_sets - 1):   # more input copies, writing the same output buffers
        steps.append(make_step(d["q"].clone(), None if d["k"] is None else d["k"].clone(),
                               d["w"].clone(), None if d.get("kc") is None else d["kc"].clone(),
                               outputs=base.outputs()))
    # one checked pass: top-k indices must be valid positions before the gather reads them
    base.run_logits()
    base.run_topk()
    torch.cuda.synchronize()
    sel = base.idx.cpu().numpy()
    lens = x["seq_len"][x["row_seq"]]
    if not (np.all(sel >= -1) and np.all(sel < lens[:, None])):
        raise RuntimeError("top-k produced out-of-range indices; not running the gather")
    base.run_gather()
    torch.cuda.synchronize()
    return x, d, steps, algorithmic_work(x, sel)


def stage_entry(name, us, work, cfg):
    """A kernel's average duration against its roof."""
    sec = us / 1e6
    if name == "logits" and cfg.T >= 8:
        peak = PEAK["mfma_fp8" if cfg.dtype == "fp8" else "mfma_bf16"]
        ach = work["logits_flops"] / sec / 1e12
        return {"bound": "mfma", "us": us, "achieved": ach, "peak": peak, "unit": "TFLOP/s",
                "frac": ach / peak, "frac_of_bf16_peak": ach / PEAK["mfma_bf16"],
                "flops": work["logits_flops"]}
    nbytes = work[f"{name}_bytes"]
    ach = nbytes / sec / 1e9
    return {"bound": "hbm", "us": us, "achieved": ach, "peak": PEAK["hbm"], "unit": "GB/s",
            "frac": ach / PEAK["hbm"], "bytes": nbytes}


def measure(args, config, full):
    """The step of one config: graph-replayed wall time per step, each
    kernel's average and per-dispatch durations; with `full`, also the
    fused step, the consumer and the CPU oracle baseline."""
    import torch

    x, d, steps, work = setup(config, args.sets)
    cfg = x["cfg"]
    n_sets = len(steps)
    base = steps[0]
    eager_out = [t.clone() for t in base.outputs()]

    for i in range(args.warmup):
        steps[i % n_sets]()
    torch.cuda.synchronize()
    # eager launches, for reference: host launch cost included
    n_eager = min(args.steps, 50)
    t0 = time.perf_counter()
    for i in range(n_eager):
        steps[i % n_sets]()
    torch.cuda.synchronize()
    ms_step_eager = (time.perf_counter() - t0) * 1e3 / n_eager

    # one HIP graph per input copy holds a whole step (three kernels), and one
    # graph holds a round of n_sets steps (one per input copy)
    graphs, round_graph = step_graphs(torch, steps, lambda s: s())
    for rep in range(2):   # replays must reproduce the eager outputs bit for bit
        for g in (graphs[0], round_graph):
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(base.outputs(), eager_out)):
                raise RuntimeError("graph replay differs from the eager step")
            steps[0]()          # eager work between replays
            torch.cuda.synchronize()
    ms_step = time_steps(torch, graphs, round_graph, args.steps, args.warmup)

    # average durations: a graph of back-to-back launches of one kernel,
    # rotating the input copies, timed with events on the launch stream
    n_in_graph = 20
    stages = {}
    flush = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device="cuda")
    for name in ("logits", "topk", "gather"):
        us = _graph_us(torch, [getattr(steps[i % n_sets], "run_" + name) for i in range(n_in_graph)],
                       max(1, args.steps // n_in_graph))
        st = stage_entry(name, us, work, cfg)
        # each dispatch alone: warm (inputs as the step leaves them) and cold
        # (512 MiB written first, so no cache holds the inputs)
        n_disp = max(10, min(50, args.steps))
        st["dispatch_warm_us"] = dispatch_us(torch, [getattr(steps[i % n_sets], "run_" + name)
                                                     for i in range(n_disp)])
        st["dispatch_cold_us"] = dispatch_us(torch, [getattr(steps[i % n_sets], "run_" + name)
                                                     for i in range(n_disp)], flush)
        stages[name] = st
    del flush
    if not all(torch.equal(a, b) for a, b in zip(base.outputs(), eager_out)):
        raise RuntimeError("timed launches changed the step's outputs")

    tg_bytes = work["topk_bytes"] + work["gather_bytes"]
    tg_gbps = tg_bytes / ((stages["topk"]["us"] + stages["gather"]["us"]) / 1e6) / 1e9
    out = {"ms_per_step": ms_step, "ms_per_step_eager": ms_step_eager, "stages": stages,
           "topk_gather_GBps": tg_gbps, "topk_gather_frac_hbm": tg_gbps / PEAK["hbm"],
           "logits_kernel_TFLOPs": work["logits_flops"] / (stages["logits"]["us"] / 1e6) / 1e12,
           "value_TFLOPs": work["logits_flops"] / (ms_step / 1e3) / 1e12,
           "input_copies_rotated": n_sets, "work": work}
    if full:
        ms = {k: v["us"] / 1e3 for k, v in stages.items()}
        if cfg.T >= 8 and cfg.kcache is None:
            fused = fused_timing(args, cfg, steps, n_sets, eager_out, ms)
            fused["value"] = work["logits_flops"] / (fused["ms_per_step"] / 1e3) / 1e12
            out["fused"] = fused
        out["consumer"] = consumer_timing(args, x, d, steps, n_sets)
    del graphs, round_graph, steps
    return x, out


def kernel_only(args):
    """One stage (or the step's three) launched --steps times back to back
    (eagerly), after the checked step: a short program for counter runs."""
    import torch
    x, d, steps, work = setup(args.config, 1)
    s = steps[0]
    if args.kernel == "logits_topk":
        s.enable_fused()
    if args.kernel == "consumer":
        consumer_timing(args, x, d, steps, 1)
        torch.cuda.synchronize()
    else:
        names = ("logits", "topk", "gather") if args.kernel == "step" else (args.kernel,)
        for _ in range(args.steps):
            for name in names:
                getattr(s, "run_" + name)()
        torch.cuda.synchronize()
    print(json.dumps({"kernel": args.kernel, "config": args.config, "launches": args.steps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=DEFAULT_CONFIG)
    ap.add_argument("--extra-configs", default=None,
                    help="comma-separated configs whose stage tables join the line (default: the "
                         f"decode and Flash prefill workloads with the default --config, none otherwise)")
    ap.add_argument("--sets", type=int, default=0, help="input copies rotated across steps (0=auto)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (PMC byte-counter calibration)")
    ap.add_argument("--producers", action="store_true",
                    help="time the input producers (fp8 row quantizer for q and k, mxfp4 cache "
                         "writer for k) on the config's shapes instead of the step")
    ap.add_argument("--cpu-table", action="store_true",
                    help="only time the CPU oracle per stage on all host cores and on one thread "
                         "(tiny, Flash decode and Flash prefill workloads)")
    ap.add_argument("--kernel", choices=("logits", "topk", "gather", "step", "logits_topk", "consumer"),
                    help="only launch this stage (step: the three stages in order) --steps times, "
                         "for profiler counter runs")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the indexer path here "
              "is built and timed on a single MI355X.", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.cpu_table:
        cpu_table(args)
        return
    if args.producers:
        producers(args)
        return
    if args.kernel:
        kernel_only(args)
        return

    import torch

    try:   # auxiliary: a failure here is reported in the line, not fatal to it
        device = device_peaks(torch)
    except (OSError, RuntimeError) as e:
        device = {"error": f"{type(e).__name__}: {e}"}
    x, res = measure(args, args.config, full=True)
    cfg = x["cfg"]
    stages = res["stages"]
    dom = max(stages, key=lambda s: stages[s]["us"])
    roof = {k: stages[dom][k] for k in ("bound", "achieved", "peak", "unit", "frac")}
    if "frac_of_bf16_peak" in stages[dom]:
        roof["frac_of_bf16_peak"] = stages[dom]["frac_of_bf16_peak"]
    roof["kernel"] = dom
    roof["traffic"] = measured_traffic(args.config, dom)
    roof["traffic_unit"] = "bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)"
    line = {
        "metric": METRIC, "value": res["value_TFLOPs"], "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"],
        "ms_per_step_eager": res["ms_per_step_eager"], "launch": "hip_graph",
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic: seeded numpy PCG64 inputs with the DeepSeek-V4 indexer shapes",
        "config": {"workload": cfg.name, "B": cfg.B, "T": cfg.T, "K": cfg.K, "H": 64, "D": 128,
                   "topk": cfg.topk, "qk_dtype": cfg.dtype, "limit": "causal"
                   if cfg.causal_offset is not None else "per-sequence length",
                   "causal_offset": cfg.causal_offset,
                   "cache": "mxfp4 E2M1+E8M0, block 64",
                   "keys": "dense" if cfg.kcache is None else f"paged {cfg.kcache} cache, block 64",
                   "input_copies_rotated": res["input_copies_rotated"]},
        "topk_gather_GBps": res["topk_gather_GBps"], "topk_gather_frac_hbm": res["topk_gather_frac_hbm"],
        "logits_kernel_TFLOPs": res["logits_kernel_TFLOPs"],
        "stages": stages, "roofline": roof, "work": res["work"], "device": device,
    }
    for k in ("fused", "consumer"):
        if k in res:
            line[k] = res[k]
    extra = args.extra_configs
    if extra is None:
        extra = EXTRA_CONFIGS if args.config == DEFAULT_CONFIG else ""
    others = {}
    for name in [c for c in extra.split(",") if c and c != args.config]:
        torch.cuda.empty_cache()
        xo, ro = measure(args, name, full=False)
        others[name] = {"ms_per_step": ro["ms_per_step"], "value_TFLOPs": ro["value_TFLOPs"],
                        "topk_gather_GBps": ro["topk_gather_GBps"],
                        "topk_gather_frac_hbm": ro["topk_gather_frac_hbm"],
                        "input_copies_rotated": ro["input_copies_rotated"],
                        "stages": ro["stages"], "work": ro["work"]}
        for st, v in others[name]["stages"].items():
            v["traffic"] = measured_traffic(name, st)
        print(f"[bench] {name}: " + ", ".join(f"{st} {v['us']:.1f} us ({100 * v['frac']:.1f}%)"
                                              for st, v in ro["stages"].items()), file=sys.stderr, flush=True)
    if others:
        line["other_configs"] = others
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(x, res["work"], args.cpu_budget)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
