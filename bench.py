#!/usr/bin/env python3
"""CSA2 decode benchmark on one MI355X.

A step is one pass of the whole hot path over one batch: compress the new
latent row of every sequence into the cache, score every visible entry with
the indexer, select the top-k, and attend over the kept rows plus the window.
The default workload is decode_32k (16 sequences x 32768 context, bf16,
ratio 1, Full layer).  Inputs are seeded synthetic tensors already resident
in HBM when timing starts.  Several identical copies of the cache are rotated
step by step so that no step finds the previous step's data in the 256 MB
Infinity Cache.

The timed steps replay HIP graphs captured from the library's calls (one
graph per cache copy; --eager launches them directly).  The same steps are
then run again with the library's kernel trace on, which brackets every
kernel with HIP events on its launch stream; the roofline is that of the
dominant kernel, the full-domain indexer scan: algorithmic HBM bytes per
launch over its mean duration for decode (one query per sequence; the decode
scan also writes the step's new entries, so their compress bytes count with
it), MFMA flops per launch for prefill (many queries share each sequence's
K).

Prints one JSON line: whole-step tokens/s, the per-kernel device times, the
scan roofline, and the float64 CPU oracle timed on a bounded sample of the
same workload on the host cores (all BLAS threads, then one).  Each extra
workload (--extra; by default fp4_1m, 2 x 1M context with FP4 KV, and
group_256k, 4 x 256K through a Full, two Reindex and a Reuse layer) is timed
the same way in the same run and reported as an object of that line.  Decode
rooflines carry two denominators: the published 8 TB/s HBM peak and the
rate the library's streaming-read probe measures for a working set of the
scan's size on this GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD public figure
METRIC = "CSA2 decode tokens/s and achieved HBM GB/s (% peak) at 32K–1M context"


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, AMD public figure


def entry_bytes(width: int, kv: str, group: int) -> float:
    if kv == "fp4":
        return width / 2 + width / group
    return width * (2 if kv == "bf16" else 4)


def visible_counts(wl):
    """Visible cache entries of each query position (the same for every sequence)."""
    import numpy as np

    t = wl.q_positions()[0].astype(np.int64)
    return np.minimum(wl.capacity, (t + 1) // wl.ratio)


def scan_work(wl) -> dict:
    """Algorithmic work of one full-domain indexer scan launch: every sequence's
    visible indexer K read once, the queries and head weights read once; the
    MFMA flops of the score contraction (one multiply-add per head, channel
    and (query, visible entry) pair)."""
    act = 2 if wl.act == "bf16" else 4
    n_vis = visible_counts(wl)
    idx_b = entry_bytes(wl.d_idx, wl.kv, wl.idx_group)
    k_bytes = wl.batch * int(n_vis.max()) * idx_b
    q_bytes = wl.batch * wl.n_q * wl.n_idx_heads * (wl.d_idx * act + 4)
    flops = 2 * wl.n_idx_heads * wl.d_idx * wl.batch * int(n_vis.sum())
    return {"bytes": float(k_bytes + q_bytes), "flops": float(flops)}


def algorithmic_bytes(wl) -> dict:
    """Bytes the method must move per step, by stage (no scratch, no re-reads):
    each sequence's indexer K is read once; a sequence's kept main-KV rows,
    pool rows and window rows are counted once each (at most its n_q queries'
    worth, at most the whole cache), its queries' own tensors once per query.
    With one query per sequence (decode) every query's rows are its own."""
    act = 2 if wl.act == "bf16" else 4
    main_b = entry_bytes(wl.d, wl.kv, wl.main_group)
    idx_b = entry_bytes(wl.d_idx, wl.kv, wl.idx_group)
    nq = wl.batch * wl.n_q
    n_new = wl.new // wl.ratio
    compress = wl.batch * (wl.new * wl.d * act + n_new * (main_b + idx_b)) + wl.d * wl.d_idx * act
    index = scan_work(wl)["bytes"] + nq * wl.topk * 4
    for p in wl.layers[1:]:
        if p.mode == "reindex":  # pool-domain rescoring: the pools' entries, the queries' indexer tensors
            pool_rows = min(wl.n_q * min(wl.cand_blocks * 8, wl.capacity), wl.capacity)
            index += wl.batch * pool_rows * idx_b + nq * (wl.n_idx_heads * (wl.d_idx * act + 4) + wl.topk * 4)
    swa_b = 1 if wl.swa == "fp8" else act  # window element: E4M3 byte or activation
    kept_rows = min(wl.n_q * wl.topk, wl.capacity)
    window_rows = wl.n_q + wl.window - 1
    attn_one = (wl.batch * (kept_rows * main_b + window_rows * wl.d * swa_b)
                + nq * (wl.topk * 4 + 2 * wl.n_heads * wl.d * act + wl.n_heads * 4))
    attn = attn_one * len(wl.layers)
    return {"compress": compress, "index": index, "attn": attn, "total": compress + index + attn}


# sources that define the scan kernels; a counter summary holds their digest
SCAN_SOURCES = ("kv_cache_compression_csa2_amd/csrc/index_scan.hip",
                "kv_cache_compression_csa2_amd/csrc/compress_entry.hpp",
                "kv_cache_compression_csa2_amd/csrc/device_common.hpp")


def code_digest(texts) -> str:
    """Digest of source texts with their // comments and blank lines left out
    (a comment edit leaves the compiled kernels, and so a counter record, as
    they were)."""
    h = hashlib.sha256()
    for text in texts:
        for line in text.splitlines():
            code = line.split("//", 1)[0].rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def sources_digest(paths) -> str:
    texts = []
    for p in paths:
        with open(os.path.join(ROOT, p)) as f:
            texts.append(f.read())
    return code_digest(texts)


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's
    counts) from the committed counter summary for this kernel and workload;
    None if there is none, or if the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic: "):
                rec = json.loads(line[len("traffic: "):])
                if rec.get("sources_sha256") != sources_digest(SCAN_SOURCES):
                    return None
                return rec.get("bytes_per_launch")
    return None


def run_gpu(wl, steps: int, warmup: int, copies: int, use_graph: bool):
    import torch

    import synth
    from kv_cache_compression_csa2_amd import binding as B
    from kv_cache_compression_csa2_amd import runner

    inp = synth.Inputs(wl)
    step = runner.DeviceStep(wl, inp, device="cuda")
    caches = [step.cache]
    for _ in range(copies - 1):
        c = runner.DeviceCache(wl, wl.capacity, "cuda")
        c.main.copy_(step.cache.main)
        c.idx_store.copy_(step.cache.idx_store)
        if c.main_scale is not None:
            c.main_scale.copy_(step.cache.main_scale)
            c.idx_scale.copy_(step.cache.idx_scale)
        c.n_entries.copy_(step.cache.n_entries)
        caches.append(c)
    structs = [c.struct() for c in caches]
    ws = step.workspace()
    cargs = step.compress_args() if wl.new else None
    layers = step.layer_structs()

    def one(i):
        # one decode step on cache copy i: compress the new rows, then the layer group
        B.csa2_layer_group(step.dims, structs[i % copies], layers, step.q_pos, wl.n_q, cargs, ws)

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    graphs = []
    if use_graph:
        for c in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                one(c)
            graphs.append(g)
        for c in range(copies):
            graphs[c].replay()
        torch.cuda.synchronize()

    # timed region: exactly `steps` steps, nothing else enqueued
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if graphs:
            graphs[i % copies].replay()
        else:
            one(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps

    # the same steps again, launched directly with the library's kernel trace on:
    # HIP events around every kernel, on the launch stream
    B.csa2_trace_enable(64 * steps)
    for i in range(steps):
        one(i)
    torch.cuda.synchronize()
    recs, dropped = B.csa2_trace_read(64 * steps)
    B.csa2_trace_enable(0)
    if dropped or len(recs) % steps:
        raise RuntimeError(f"kernel trace incomplete: {len(recs)} records, {dropped} dropped")
    per_step = len(recs) // steps
    launches = []  # (kernel, mean ms) for each launch position of a step
    for j in range(per_step):
        names = {recs[i * per_step + j][0] for i in range(steps)}
        if len(names) != 1:
            raise RuntimeError("steps launched different kernel sequences")
        launches.append((recs[j][0], sum(recs[i * per_step + j][1] for i in range(steps)) / steps))
    return ms, launches


def run_oproj(n_tok: int, steps: int, warmup: int, copies: int) -> dict:
    """The grouped output projection alone at the production shape (64 heads
    x 512 into 8 groups of rank 1024) for n_tok attention-output rows;
    `copies` weight sets are rotated so the Infinity Cache cannot hold them."""
    import torch

    import synth
    from kv_cache_compression_csa2_amd import binding as B

    width, groups, rank = 64 * 512, 8, 1024
    x, w = synth.oproj_inputs(n_tok, width, groups, rank, "bf16")
    xd = torch.from_numpy(x).to("cuda").to(torch.bfloat16)
    ws = [torch.from_numpy(w).to("cuda").to(torch.bfloat16) for _ in range(copies)]
    y = torch.empty((n_tok, groups * rank), dtype=torch.bfloat16, device="cuda")
    del x, w

    def one(i):
        B.csa2_grouped_out_proj(B.BF16, n_tok, width, groups, rank, xd, ws[i % copies], y)

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    B.csa2_trace_enable(steps)
    for i in range(steps):
        one(i)
    torch.cuda.synchronize()
    recs, dropped = B.csa2_trace_read(steps)
    B.csa2_trace_enable(0)
    if dropped or len(recs) != steps:
        raise RuntimeError(f"kernel trace incomplete: {len(recs)} records, {dropped} dropped")
    kname = recs[0][0]
    kms = sum(r[1] for r in recs) / steps
    wbytes = groups * rank * (width // groups) * 2
    nbytes = wbytes + n_tok * width * 2 + n_tok * groups * rank * 2
    flops = 2 * n_tok * width * rank
    if n_tok <= 64:
        achieved = nbytes / (kms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "per_launch": nbytes, "avg_ms": round(kms, 5),
                "traffic": None}
    else:
        mceil = mfma_ceiling()
        achieved = flops / (kms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": kname, "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "per_launch": flops,
                "avg_ms": round(kms, 5), "measured_peak": mceil["tflops"],
                "frac_of_measured": round(achieved / mceil["tflops"], 4), "traffic": None}
    return {"metric": "grouped_out_proj_tokens_per_s", "value": round(n_tok / (kms * 1e-3), 1), "unit": "tokens/s",
            "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_launch_wall": round(ms, 5),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": f"grouped_out_proj_{n_tok}", "tokens": n_tok, "width": width, "groups": groups,
                       "rank": rank, "weight_copies": copies},
            "roofline": roof, "cpu_baseline": None}


def read_ceiling(nbytes: float, copies: int = 4, reps: int = 20) -> dict:
    """Measured streaming-read rate for a working set of `nbytes`: the
    library's read probe over `copies` rotated buffers of that size (so the
    Infinity Cache cannot hold the one being read), mean device time from the
    kernel trace."""
    import torch

    from kv_cache_compression_csa2_amd import binding as B

    n = int(nbytes) // 16 * 16
    bufs = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    for i in range(copies):
        B.csa2_read_probe(bufs[i], n, sink)
    torch.cuda.synchronize()
    B.csa2_trace_enable(reps)
    for i in range(reps):
        B.csa2_read_probe(bufs[i % copies], n, sink)
    torch.cuda.synchronize()
    recs, dropped = B.csa2_trace_read(reps)
    B.csa2_trace_enable(0)
    if dropped or len(recs) != reps:
        raise RuntimeError(f"read probe trace incomplete: {len(recs)} records, {dropped} dropped")
    ms = sum(r[1] for r in recs) / reps
    return {"bytes": n, "ms": round(ms, 5), "gbps": round(n / (ms * 1e-3) / 1e9, 1), "copies": copies}


def mfma_ceiling(iters: int = 4096, workgroups: int = 512, reps: int = 20) -> dict:
    """Measured bf16 matrix-core rate: the library's matrix-core probe
    (independent 32x32x16 bf16 product chains on register operands, two
    workgroups per compute unit, no memory traffic), mean device time of
    `reps` back-to-back launches from the kernel trace, after one warm-up."""
    import torch

    from kv_cache_compression_csa2_amd import binding as B

    sink = torch.zeros(4, dtype=torch.float32, device="cuda")
    B.csa2_mfma_probe(iters, workgroups, sink)
    torch.cuda.synchronize()
    B.csa2_trace_enable(reps)
    for _ in range(reps):
        B.csa2_mfma_probe(iters, workgroups, sink)
    torch.cuda.synchronize()
    recs, dropped = B.csa2_trace_read(reps)
    B.csa2_trace_enable(0)
    if dropped or len(recs) != reps:
        raise RuntimeError(f"matrix-core probe trace incomplete: {len(recs)} records, {dropped} dropped")
    ms = sum(r[1] for r in recs) / reps
    flops = workgroups * B.MFMA_PROBE_FLOP_PER_WG_ITER * iters
    return {"flops": flops, "ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "workgroups": workgroups, "iters": iters}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(wl, seconds: float, single_thread_seconds: float = 0.0) -> dict:
    """The float64 oracle timed on the host cores on a sample of the workload's sequences."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import synth
    from oracle import csa2 as oc
    from oracle import driver

    inp = synth.Inputs(wl)
    seqs = [0, 1][: wl.batch]
    dims = driver.dims_of(wl)
    caches = [driver.build_cache(inp, b, wl.context) for b in seqs]  # untimed: cache contents incl. the new entry
    specs = driver.layer_specs(inp, seqs)
    new_lat = [inp.latent(b, wl.prior, wl.context).astype(np.float64) for b in seqs]
    logits, w_ik = inp.pair_logits(), inp.w_ik()
    q_pos = wl.q_positions()[seqs]
    n_entries = [c.n_entries for c in caches]

    def timed(limit):
        done = 0
        t0 = time.perf_counter()
        while True:
            for i in range(len(seqs)):
                if wl.new:
                    oc.make_entries(new_lat[i], wl.prior, logits, w_ik, wl.ratio, wl.d_rope, driver.rope_cfg(wl),
                                    wl.kv, wl.main_group, wl.idx_group)
            oc.run_group(dims, caches, n_entries, q_pos, specs)
            done += len(seqs) * wl.n_q
            if time.perf_counter() - t0 >= limit:
                break
        return done, time.perf_counter() - t0

    done, el = timed(seconds)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    out = {"value": done / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{wl.name}: sequences {seqs} of {wl.batch}, one decode step each, repeated "
                     f"{done // max(1, len(seqs) * wl.n_q)} times in {el:.1f} s (cache build untimed)",
           "cpu_model": cpu_model(), "affinity_cores": len(os.sched_getaffinity(0))}
    if single_thread_seconds > 0:
        from threadpoolctl import threadpool_limits

        with threadpool_limits(limits=1):
            d1, e1 = timed(single_thread_seconds)
        out["single_thread_value"] = d1 / e1
        out["single_thread_sample"] = f"the same step, BLAS limited to 1 thread, repeated {d1 // max(1, len(seqs) * wl.n_q)} times in {e1:.1f} s"
    return out


def measure(wl, args) -> dict:
    """Time one workload's step (graph replays), its kernels (library trace),
    the scan's roofline and its measured ceiling: the streaming-read rate at
    the scan's bytes (one query per sequence) or the matrix-core rate (many)."""
    ms, launches = run_gpu(wl, args.steps, args.warmup, args.copies, not args.eager)
    print(f"[bench] gpu done: {ms:.4f} ms/step; kernels (ms): "
          + ", ".join(f"{k} {v:.4f}" for k, v in launches), file=sys.stderr, flush=True)
    nbytes = algorithmic_bytes(wl)
    tokens = wl.batch * wl.n_q
    work = scan_work(wl)
    scan_ms = next(v for k, v in launches if k.startswith("scan_"))
    scan_name = next(k for k, v in launches if k.startswith("scan_"))
    if scan_name.startswith("scan_fused_"):  # the decode scan also writes the step's entries
        work = {"bytes": work["bytes"] + nbytes["compress"], "flops": work["flops"]}
    ceiling = None
    if wl.n_q == 1:
        ceiling = read_ceiling(work["bytes"], copies=args.copies)
        print(f"[bench] read ceiling at {ceiling['bytes'] / 1e6:.1f} MB: {ceiling['gbps']:.0f} GB/s",
              file=sys.stderr, flush=True)
        achieved = work["bytes"] / (scan_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": scan_name, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4), "per_launch": work["bytes"],
                "avg_ms": round(scan_ms, 5), "measured_peak": ceiling["gbps"],
                "frac_of_measured": round(achieved / ceiling["gbps"], 4)}
    else:
        mceil = mfma_ceiling()
        print(f"[bench] matrix-core ceiling: {mceil['tflops']:.0f} TFLOP/s", file=sys.stderr, flush=True)
        achieved = work["flops"] / (scan_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": scan_name, "achieved": round(achieved, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4), "per_launch": work["flops"],
                "avg_ms": round(scan_ms, 5), "measured_peak": mceil["tflops"],
                "frac_of_measured": round(achieved / mceil["tflops"], 4)}
    roof["traffic"] = recorded_traffic(wl.name, scan_name)
    step_gbps = nbytes["total"] / (ms * 1e-3) / 1e9
    return {
        "value": round(tokens / (ms * 1e-3), 1), "ms_per_step": round(ms, 5),
        "dtype": wl.act if wl.kv != "fp4" else "bf16+fp4kv",
        "config": {"workload": wl.name, "batch": wl.batch, "context": wl.context, "ratio": wl.ratio,
                   "kv": wl.kv, "heads": f"{wl.n_heads}x{wl.d}", "indexer": f"{wl.n_idx_heads}x{wl.d_idx}",
                   "topk": wl.topk, "window": wl.window, "window_rows": "fp8" if wl.swa == "fp8" else wl.act,
                   "queries_per_seq": wl.n_q,
                   "layers": [p.mode for p in wl.layers], "cache_copies": args.copies,
                   "launch": "eager" if args.eager else "hip_graph"},
        "step_hbm_gbps": round(step_gbps, 1),
        "step_hbm_frac": round(step_gbps / HBM_PEAK_GBPS, 4),
        "step_hbm_frac_of_measured": round(step_gbps / ceiling["gbps"], 4) if ceiling else None,
        "step_bytes": nbytes["total"],
        "kernels_ms": [[k, round(v, 5)] for k, v in launches],
        "roofline": roof,
    }


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_32k")
    ap.add_argument("--copies", type=int, default=4, help="rotated cache copies (defeats the Infinity Cache)")
    ap.add_argument("--eager", action="store_true", help="launch the timed steps directly instead of replaying HIP graphs")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-single-seconds", type=float, default=6.0,
                    help="also time the oracle with BLAS limited to one thread (0 skips it)")
    ap.add_argument("--extra", default="fp4_1m,group_256k",
                    help="comma-separated workloads timed after the main one and reported as objects of the "
                         "same line ('none' for none)")
    ap.add_argument("--oproj-tokens", type=int, default=0,
                    help="time only the grouped output projection, for this many attention-output rows")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB 5 times (calibrates HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        return 2

    if args.oproj_tokens:
        out = run_oproj(args.oproj_tokens, args.steps, args.warmup, max(args.copies, 6))
        print(json.dumps(out), flush=True)
        return 0

    import synth

    wl = synth.get(args.workload)
    print(f"[bench] {wl.name}: {wl.description}", file=sys.stderr, flush=True)
    res = measure(wl, args)
    if args.copy_mib:
        import torch

        n = args.copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] copy calibration: 5 copies of {args.copy_mib} MiB", file=sys.stderr, flush=True)

    extras = {}
    for name in [x for x in args.extra.split(",") if x and x != "none" and x != wl.name]:
        import torch

        torch.cuda.empty_cache()
        ewl = synth.get(name)
        print(f"[bench] {ewl.name}: {ewl.description}", file=sys.stderr, flush=True)
        r = measure(ewl, args)
        extras[name] = {"value": r["value"], "unit": "tokens/s", "ms_per_step": r["ms_per_step"],
                        "dtype": r["dtype"], "config": r["config"], "step_hbm_gbps": r["step_hbm_gbps"],
                        "step_hbm_frac": r["step_hbm_frac"], "step_hbm_frac_of_measured": r["step_hbm_frac_of_measured"],
                        "step_bytes": r["step_bytes"], "kernels_ms": r["kernels_ms"], "roofline": r["roofline"]}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds, args.cpu_single_seconds)
        print(f"[bench] cpu baseline done: {cpu['value']:.2f} tokens/s", file=sys.stderr, flush=True)
    out = {
        "metric": METRIC, "value": res["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": res["dtype"], "data": "synthetic",
        "config": res["config"],
        "step_hbm_gbps": res["step_hbm_gbps"], "step_hbm_frac": res["step_hbm_frac"],
        "step_hbm_frac_of_measured": res["step_hbm_frac_of_measured"], "step_bytes": res["step_bytes"],
        "kernels_ms": res["kernels_ms"], "roofline": res["roofline"], "cpu_baseline": cpu,
    }
    out.update(extras)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
