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

Prints one JSON line: whole-step decode tokens/s, the roofline of the
dominant kernel (the indexer scan+select call, timed with HIP events on the
launch stream), and the float64 CPU oracle timed on a bounded sample of the
same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD public figure
METRIC = "CSA2 decode tokens/s and achieved HBM GB/s (% peak) at 32K–1M context"


def entry_bytes(width: int, kv: str, group: int) -> float:
    if kv == "fp4":
        return width / 2 + width / group
    return width * (2 if kv == "bf16" else 4)


def algorithmic_bytes(wl) -> dict:
    """Bytes the method must move per step, by stage (no scratch, no re-reads)."""
    act = 2 if wl.act == "bf16" else 4
    main_b = entry_bytes(wl.d, wl.kv, wl.main_group)
    idx_b = entry_bytes(wl.d_idx, wl.kv, wl.idx_group)
    nq = wl.batch * wl.n_q
    n_new = wl.new // wl.ratio
    compress = wl.batch * (wl.new * wl.d * act + n_new * (main_b + idx_b)) + wl.d * wl.d_idx * act
    t_last = wl.context - 1
    n_vis = min(wl.capacity, (t_last + 1) // wl.ratio)
    index = wl.batch * wl.n_q * n_vis * idx_b + nq * (wl.n_idx_heads * wl.d_idx * act + wl.n_idx_heads * 4 + wl.topk * 4)
    attn = nq * (wl.topk * (main_b + 4) + wl.window * wl.d * act + 2 * wl.n_heads * wl.d * act + wl.n_heads * 4)
    return {"compress": compress, "index": index, "attn": attn, "total": compress + index + attn}


def run_gpu(wl, steps: int, warmup: int, copies: int):
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
        c.idx.copy_(step.cache.idx)
        if c.main_scale is not None:
            c.main_scale.copy_(step.cache.main_scale)
            c.idx_scale.copy_(step.cache.idx_scale)
        c.n_entries.copy_(step.cache.n_entries)
        caches.append(c)
    structs = [c.struct() for c in caches]
    single_full = len(wl.layers) == 1 and wl.layers[0].mode == "full"
    L = step.layers[0]
    ws = step.workspace()
    ws_idx = ws
    cargs = step.compress_args()

    def one(i, ev=None):
        cs = structs[i % len(structs)]
        if not single_full:
            if ev:
                ev[0].record()
            B.csa2_layer_group(step.dims, cs, step.layer_structs(), step.q_pos, wl.n_q, cargs, ws)
            if ev:
                ev[3].record()
            return
        if ev:
            ev[0].record()
        if wl.new:
            B.csa2_compress(step.dims, cs, step.latent_new, step.first_pos, wl.new, step.pair_logits, step.w_ik)
        if ev:
            ev[1].record()
        B.csa2_index_topk(step.dims, cs, L["q_idx"], L["head_w"], step.q_pos, wl.n_q, None, L["topk"],
                          L["pool"], None, ws_idx)
        if ev:
            ev[2].record()
        B.csa2_sparse_attn(step.dims, cs, L["q"], step.q_pos, wl.n_q, L["topk"], L["swa"], L["swa_first"],
                           L["swa"].shape[1], L["out"], L["lse"], ws)
        if ev:
            ev[3].record()

    for i in range(warmup):
        one(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        one(warmup + i, evs[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stages = {}
    if single_full:
        stages = {
            "compress": sum(e[0].elapsed_time(e[1]) for e in evs) / steps,
            "index_topk": sum(e[1].elapsed_time(e[2]) for e in evs) / steps,
            "sparse_attn": sum(e[2].elapsed_time(e[3]) for e in evs) / steps,
        }
    stages["step_events"] = sum(e[0].elapsed_time(e[3]) for e in evs) / steps
    return (t1 - t0) * 1e3 / steps, stages


def cpu_baseline(wl, seconds: float) -> dict:
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
    done = 0
    t0 = time.perf_counter()
    while True:
        for i in range(len(seqs)):
            if wl.new:
                oc.make_entries(new_lat[i], wl.prior, logits, w_ik, wl.ratio, wl.d_rope, wl.rope_theta, wl.kv,
                                wl.main_group, wl.idx_group)
        oc.run_group(dims, caches, n_entries, q_pos, specs)
        done += len(seqs) * wl.n_q
        if time.perf_counter() - t0 >= seconds:
            break
    el = time.perf_counter() - t0
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": done / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{wl.name}: sequences {seqs} of {wl.batch}, one decode step each, repeated "
                      f"{done // max(1, len(seqs) * wl.n_q)} times in {el:.1f} s (cache build untimed)"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode_32k")
    ap.add_argument("--copies", type=int, default=4, help="rotated cache copies (defeats the Infinity Cache)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        return 2

    import synth

    wl = synth.get(args.workload)
    print(f"[bench] {wl.name}: {wl.description}", file=sys.stderr, flush=True)
    ms, stages = run_gpu(wl, args.steps, args.warmup, args.copies)
    print(f"[bench] gpu done: {ms:.4f} ms/step, stages {stages}", file=sys.stderr, flush=True)
    nbytes = algorithmic_bytes(wl)
    tokens = wl.batch * wl.n_q
    roof = None
    if "index_topk" in stages:
        achieved = nbytes["index"] / (stages["index_topk"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": "csa2_index_topk (indexer scan + select)", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "bytes_per_launch": nbytes["index"], "avg_ms": round(stages["index_topk"], 5), "traffic": None}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds)
        print(f"[bench] cpu baseline done: {cpu['value']:.2f} tokens/s", file=sys.stderr, flush=True)
    out = {
        "metric": METRIC, "value": round(tokens / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": wl.act if wl.kv != "fp4" else "bf16+fp4kv",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "context": wl.context, "ratio": wl.ratio,
                   "kv": wl.kv, "heads": f"{wl.n_heads}x{wl.d}", "indexer": f"{wl.n_idx_heads}x{wl.d_idx}",
                   "topk": wl.topk, "window": wl.window, "layers": [p.mode for p in wl.layers],
                   "cache_copies": args.copies},
        "step_hbm_gbps": round(nbytes["total"] / (ms * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(nbytes["total"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "step_bytes": nbytes["total"],
        "stages_ms": {k: round(v, 5) for k, v in stages.items()},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
