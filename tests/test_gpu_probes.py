"""The measurement probes behind bench.py's measured ceilings, run through the
C ABI: the streaming read and the matrix-core loop launch, are recorded by
the kernel trace under their own names, and report plausible rates (above a
tenth of, and not above, the published figures: 8 TB/s and 2.5 PFLOP/s)."""
import pytest

pytestmark = pytest.mark.gpu


def test_probes_run_and_are_traced():
    import torch

    from kv_cache_compression_csa2_amd import binding as B

    n = 64 << 20
    buf = torch.ones(n, dtype=torch.uint8, device="cuda")
    isink = torch.zeros(4, dtype=torch.int32, device="cuda")
    fsink = torch.zeros(4, dtype=torch.float32, device="cuda")
    B.csa2_read_probe(buf, n, isink)
    B.csa2_mfma_probe(64, 512, fsink)
    torch.cuda.synchronize()
    B.csa2_trace_enable(2)
    B.csa2_read_probe(buf, n, isink)
    B.csa2_mfma_probe(1024, 512, fsink)
    torch.cuda.synchronize()
    recs, dropped = B.csa2_trace_read(2)
    B.csa2_trace_enable(0)
    assert dropped == 0 and [r[0] for r in recs] == ["read_probe_kernel", "mfma_probe_kernel"]
    gbps = n / (recs[0][1] * 1e-3) / 1e9
    tflops = 512 * B.MFMA_PROBE_FLOP_PER_WG_ITER * 1024 / (recs[1][1] * 1e-3) / 1e12
    print(f"read probe {gbps:.0f} GB/s, matrix-core probe {tflops:.0f} TFLOP/s", flush=True)
    assert 800 < gbps <= 8000 and 250 < tflops <= 2500
    # neither sink matched its constant: nothing was written
    assert int(isink.abs().sum()) == 0 and float(fsink.abs().sum()) == 0.0
