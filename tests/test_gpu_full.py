"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The GPU runs the whole step for every sequence (cache built by csa2_compress,
then csa2_layer_group).  The oracle checks sampled sequences and queries: it
builds the full indexer K of a sampled sequence (every score is checked) and
makes main-KV rows only for the entries it reads.  Cache bytes are compared on
sampled rows, including the step's new entries.
"""
import time

import numpy as np
import pytest

import synth
from oracle import driver
from tests import harness

pytestmark = pytest.mark.gpu

# workload -> (sampled sequences, sampled queries or None for all)
FULL = {
    "decode_32k": ([0, 15], None),
    "group_256k": ([3], None),
    "fp4_1m": ([1], None),
    "prefill_128k": ([0], [0, 1, 2, 255, 256, 511, 777, 1024, 1500, 2047, 2048, 2049, 3000, 3583, 4094, 4095]),
    "encoder_block_128k": ([0], [0, 1, 1023, 2047, 2048, 3071, 4094, 4095]),
    "fp4_1m_pages": ([0], None),
    "decoder_prefill_64k": ([0], [0, 2049, 4095]),
    "fp4_1m_yarn": ([1], None),
    "replay_64k": ([0], [0, 1, 64, 126, 127]),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_sampled(name):
    import torch

    from kv_cache_compression_csa2_amd import runner

    wl = synth.get(name)
    inp = synth.Inputs(wl)
    seqs, queries = FULL[name]
    t0 = time.time()
    print(f"[full] {name}: building GPU caches for {wl.batch} x {wl.capacity} entries", flush=True)
    step = runner.DeviceStep(wl, inp)
    step.run()
    torch.cuda.synchronize()
    print(f"[full] {name}: GPU step done in {time.time() - t0:.1f}s; oracle caches for {seqs}", flush=True)
    caches = [driver.LazyMainCache(inp, b, wl.context) for b in seqs]
    print(f"[full] {name}: oracle caches built at {time.time() - t0:.1f}s", flush=True)
    rng = np.random.default_rng(0)
    for c, b in zip(caches, seqs):
        new = np.arange(wl.n_prior_entries, wl.capacity)
        ids = np.unique(np.concatenate([rng.integers(0, wl.capacity, 512), new[:64], new[-64:]]))
        harness.compare_cache_rows(step, c, b, ids)
    summary = harness.check_step(step, inp, seqs, caches, queries)
    print(f"[full] {name}: parity {summary} at {time.time() - t0:.1f}s", flush=True)
