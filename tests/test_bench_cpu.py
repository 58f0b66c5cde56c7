"""The benchmark's work accounting on the CPU: algorithmic bytes and flops of
the measured workloads, worked out by hand from their shapes.

decode_32k: 16 sequences x 32768 visible entries x 256 B of bf16 indexer K
(134,217,728 B) + 16 x 32 x (128 x 2 + 4) B of indexer queries and head
weights, the compress step (one 1024 B latent row in, a 1024 B main row and
a 256 B indexer row out per sequence, W_ik 512 x 128 x 2 B once), 512 int32
ids per query, and attention reading 512 kept rows (1024 B) + 128 window
rows (1024 B) and the 64 x 512 bf16 query, writing the output and 64 float32
log-sum-exps.
"""
import bench
import synth


def test_decode_32k_bytes():
    wl = synth.get("decode_32k")
    scan = 16 * 32768 * 256 + 16 * 32 * (128 * 2 + 4)
    compress = 16 * (1024 + 1024 + 256) + 512 * 128 * 2
    index = scan + 16 * 512 * 4
    attn = 16 * (512 * 1024 + 128 * 1024) + 16 * (512 * 4 + 2 * 64 * 512 * 2 + 64 * 4)
    got = bench.algorithmic_bytes(wl)
    assert bench.scan_work(wl)["bytes"] == scan
    assert (got["compress"], got["index"], got["attn"]) == (compress, index, attn)
    assert got["total"] == 147_171_328


def test_fp4_1m_bytes_and_scan_flops():
    wl = synth.get("fp4_1m")
    # FP4 indexer K: 64 code bytes + 4 scale bytes per entry; main KV 256 + 16
    scan = 2 * 1048576 * 68 + 2 * 32 * (128 * 2 + 4)
    assert bench.scan_work(wl)["bytes"] == scan
    assert bench.scan_work(wl)["flops"] == 2 * 32 * 128 * 2 * 1048576
    assert bench.algorithmic_bytes(wl)["total"] == 143_568_296


def test_prefill_scan_flops_count_visible_pairs_only():
    wl = synth.get("prefill_128k")
    # query at 131072 + q sees 65536 + (q + 1) // 2 entries (ratio 2)
    pairs = sum(65536 + (q + 1) // 2 for q in range(4096))
    assert pairs == 272_629_760
    assert bench.scan_work(wl)["flops"] == 2 * 32 * 128 * pairs


def test_multi_query_rows_count_once():
    wl = synth.get("prefill_128k")
    # 4096 queries x 512 kept rows exceed the cache: each cached row once
    one_layer = bench.algorithmic_bytes(wl)["attn"]
    rows = 67584 * 1024 + (4096 + 127) * 1024
    per_query = 4096 * (512 * 4 + 2 * 64 * 512 * 2 + 64 * 4)
    assert one_layer == rows + per_query


def test_code_digest_ignores_comments_only():
    """A counter record stays valid across comment edits of the scan sources and
    is invalidated by any code edit."""
    import bench

    a = "int f(int x) {  // doubled\n  return 2 * x;\n}\n"
    b = "// a new header comment\nint f(int x) {  // twice x\n\n  return 2 * x;\n}\n"
    c = "int f(int x) {\n  return 3 * x;\n}\n"
    assert bench.code_digest([a]) == bench.code_digest([b])
    assert bench.code_digest([a]) != bench.code_digest([c])


def test_counter_records_match_the_scan_sources_and_the_accounting():
    """Each committed HBM counter summary under profiles/ was taken on the scan
    code as it stands (its digest of the scan sources is the current one, so
    the bench line reports its traffic), and the algorithmic bytes it divides
    by are the ones bench.py counts for that kernel and workload today.  A
    change to the scan sources needs its counters taken again."""
    import glob
    import json
    import os

    paths = sorted(glob.glob(os.path.join(bench.ROOT, "profiles", "*_hbm_counters.txt")))
    assert paths
    for path in paths:
        rec = None
        with open(path) as f:
            for line in f:
                if line.startswith("traffic: "):
                    rec = json.loads(line[len("traffic: "):])
        assert rec is not None, path
        kernel, workload = rec["kernel"], rec["workload"]
        assert os.path.basename(path) == f"{kernel}_{workload}_hbm_counters.txt"
        assert rec["sources_sha256"] == bench.sources_digest(bench.SCAN_SOURCES), \
            f"{path}: taken on other scan sources"
        assert bench.recorded_traffic(workload, kernel) == rec["bytes_per_launch"]
        # (each of the three is rounded to a byte on its own)
        assert abs(rec["bytes_per_launch"] - rec["fetch_bytes_per_launch"] - rec["write_bytes_per_launch"]) <= 1
        wl = synth.get(workload)
        alg = bench.scan_work(wl)["bytes"]
        if kernel.startswith("scan_fused_"):
            alg += bench.algorithmic_bytes(wl)["compress"]
        assert rec["algorithmic_bytes_per_launch"] == alg, path


def test_bench_refuses_more_than_one_gpu():
    """The library has no multi-GPU path: bench.py says so and exits with 2
    before it touches a GPU."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=bench.ROOT, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_cpu_baseline_object():
    """The cpu_baseline object of the bench line: the oracle's own step on a
    bounded sample, with the fields the line carries."""
    wl = synth.get("decode_dense")  # 2 x 401 entries: a step takes milliseconds
    out = bench.cpu_baseline(wl, 0.3, 0.2)
    assert out["kind"] == "oracle" and out["unit"] == "tokens/s"
    assert out["value"] > 0 and out["single_thread_value"] > 0
    assert isinstance(out["cores"], int) and out["cores"] >= 1
    assert out["affinity_cores"] >= 1 and out["cpu_model"]
    assert out["sample"].startswith("decode_dense: sequences [0, 1] of 2")
