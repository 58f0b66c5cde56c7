"""Checkpoint and resume through the caches' documented byte layout: the
main KV, its scales, the indexer K tiles, their scales and the entry counts
are plain caller-owned buffers, so saving them to files, loading them into a
fresh set of buffers and running the next step gives bit-identical results
(top-k, pools, outputs, LSE, and the caches after the step).  The pages keep
a persistent prefix cache and rebuild the window by bounded replay (zartbot
walkthrough 2.2.2; 36Kr "FP4 and Bounded Replay"); this checks the part the
library owns: nothing but the buffers carries state between steps."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu

PLANES = ("main", "main_scale", "idx_store", "idx_scale", "n_entries")


def _outputs(st):
    return [{k: (None if L[k] is None else L[k].clone()) for k in ("topk", "pool", "out", "lse")} for L in st.layers]


@pytest.mark.parametrize("name", ["fp4_small", "hsi_small"])
def test_caches_saved_to_files_resume_bit_identical(name, tmp_path):
    import torch

    from kv_cache_compression_csa2_amd import runner

    wl = synth.get(name)
    inp = synth.Inputs(wl)
    st = runner.DeviceStep(wl, inp)  # caches built from the prior positions
    saved = {}
    for p in PLANES:
        t = getattr(st.cache, p)
        if t is not None:
            path = tmp_path / f"{p}.npy"
            np.save(path, t.cpu().view(torch.uint8).numpy() if t.dtype != torch.int32 else t.cpu().numpy())
            saved[p] = (path, t.dtype, tuple(t.shape))
    st.run()
    torch.cuda.synchronize()
    want = _outputs(st)
    after = {p: getattr(st.cache, p).clone() for p in saved}

    fresh = runner.DeviceStep(wl, inp, build_prior=False)  # empty caches
    for p, (path, dtype, shape) in saved.items():
        a = np.load(path)  # no pickles
        t = torch.from_numpy(a).to("cuda")
        t = t if dtype == torch.int32 else t.view(dtype)
        getattr(fresh.cache, p).copy_(t.reshape(shape))
    fresh.run()
    torch.cuda.synchronize()
    for li, (w, L) in enumerate(zip(want, fresh.layers)):
        for k in ("topk", "pool", "out", "lse"):
            if w[k] is not None:
                assert torch.equal(w[k], L[k]), f"{name} layer {li}: {k} differs after resume"
    for p in saved:
        assert torch.equal(after[p], getattr(fresh.cache, p)), f"{name}: cache plane {p} differs after resume"
    print(f"[checkpoint] {name}: {len(saved)} planes, {sum(np.load(v[0]).nbytes for v in saved.values())} bytes", flush=True)
