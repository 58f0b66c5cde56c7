"""The C ABI on a CPU-only host: the library loads, exports what csa2.h declares,
and rejects every malformed call before touching the GPU (fake device
pointers are never dereferenced on the host)."""
import ctypes
import os
import re

import pytest

from kv_cache_compression_csa2_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x100000  # 16-byte aligned, never dereferenced by the host-side checks


def declared_functions():
    text = open(os.path.join(ROOT, "include", "csa2.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa2_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) == set(B.EXPORTED)
    lib = B.library()
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert B.csa2_abi_version() == 7
    assert B.status_str(0) == "CSA2_OK"
    assert B.status_str(-4) == "CSA2_ERR_MODE_ORDER"
    assert B.status_str(-99) == "CSA2_ERR_UNKNOWN"


def dims(**kw):
    base = dict(d=512, d_rope=64, n_heads=64, n_idx_heads=32, d_idx=128, topk=512, window=128, block_size=8,
                cand_blocks=2048, act_dtype=B.BF16, rope_theta=10000.0)
    base.update(kw)
    return B.Dims(**base)


def cache(**kw):
    base = dict(kv_dtype=B.BF16, ratio=1, main_group=32, idx_group=32, batch=2, reserved0=0, capacity=4096,
                main=FAKE, main_scale=None, idx_k=FAKE, idx_scale=None, n_entries=FAKE)
    base.update(kw)
    return B.KVCache(**base)


def call_index(d=None, c=None, ws=FAKE, ws_bytes=1 << 40, pool_in=None, pool_out=None, idx_q=FAKE):
    lib = B.library()
    d = d or dims()
    c = c or cache()
    return lib.csa2_index_topk(ctypes.byref(d), ctypes.byref(c), idx_q, FAKE, FAKE, 1, pool_in, FAKE, pool_out, None,
                               ws, ws_bytes, None)


@pytest.mark.parametrize(
    "d,c,status",
    [
        (dict(d=100), {}, -2),
        (dict(d_rope=3), {}, -1),
        (dict(block_size=16), {}, -2),
        (dict(topk=4096), {}, -2),
        (dict(cand_blocks=0), {}, -2),
        (dict(act_dtype=7), {}, -2),
        (dict(rope_theta=0.0), {}, -1),
        (dict(swa_dtype=B.FP4), {}, -2),
        (dict(rope_factor=0.5), {}, -1),
        (dict(rope_factor=16.0, rope_orig_len=0), {}, -1),
        ({}, dict(ratio=3), -2),
        ({}, dict(kv_dtype=9), -2),
        ({}, dict(capacity=(1 << 20) + 1), -2),
        ({}, dict(reserved0=1), -1),
        ({}, dict(main=None), -1),
        ({}, dict(main=FAKE + 4), -1),
        ({}, dict(idx_k=None), -1),
        ({}, dict(kv_dtype=B.FP4, main_scale=FAKE, idx_scale=FAKE, main_group=8), -2),
        ({}, dict(kv_dtype=B.FP4, main_scale=None, idx_scale=FAKE), -1),
    ],
)
def test_index_rejects_bad_dims_and_cache(d, c, status):
    assert call_index(dims(**d), cache(**c)) == status
    assert B.last_error()


def test_index_rejects_bad_arguments():
    assert call_index(pool_in=FAKE, pool_out=FAKE) == -1
    assert call_index(idx_q=None) == -1
    assert call_index(idx_q=FAKE + 2) == -1
    assert call_index(ws=None) == -3
    assert call_index(ws=FAKE + 16) == -3
    assert call_index(ws_bytes=1024) == -3


def test_null_dims_and_cache():
    lib = B.library()
    assert lib.csa2_index_topk(None, ctypes.byref(cache()), FAKE, FAKE, FAKE, 1, None, FAKE, None, None, FAKE, 1 << 40,
                               None) == -1
    assert lib.csa2_sparse_attn(ctypes.byref(dims()), None, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 128, FAKE, None, FAKE,
                                1 << 40, None) == -1


def test_compress_rejects_bad_arguments():
    lib = B.library()
    d, c = dims(), cache()
    assert lib.csa2_compress(ctypes.byref(d), ctypes.byref(c), FAKE, FAKE, 4, FAKE, FAKE, None) == -1  # logits at ratio 1
    c2 = cache(ratio=2)
    assert lib.csa2_compress(ctypes.byref(d), ctypes.byref(c2), FAKE, FAKE, 4, None, FAKE, None) == -1  # no logits
    assert lib.csa2_compress(ctypes.byref(d), ctypes.byref(c2), FAKE, FAKE, 3, FAKE, FAKE, None) == -1  # odd rows
    assert lib.csa2_compress(ctypes.byref(d), ctypes.byref(c), None, FAKE, 4, None, FAKE, None) == -1
    assert lib.csa2_compress(ctypes.byref(d), ctypes.byref(cache(idx_k=None)), FAKE, FAKE, 4, None, FAKE, None) == -1


def test_attention_rejects_bad_arguments_and_allows_no_indexer_k():
    lib = B.library()
    d = dims()
    c = cache(idx_k=None)
    assert lib.csa2_sparse_attn(ctypes.byref(d), ctypes.byref(c), FAKE, FAKE, 0, FAKE, FAKE, FAKE, 128, FAKE, None,
                                FAKE, 1 << 40, None) == -1
    assert lib.csa2_sparse_attn(ctypes.byref(d), ctypes.byref(c), FAKE, FAKE, 1, FAKE, None, FAKE, 128, FAKE, None,
                                FAKE, 1 << 40, None) == -1
    assert lib.csa2_sparse_attn(ctypes.byref(d), ctypes.byref(c), FAKE, FAKE, 1, FAKE, FAKE, FAKE, -1, FAKE, None,
                                FAKE, 1 << 40, None) == -1


def layer(mode, source=-1, make_pool=0, pool=None, topk=FAKE):
    return B.Layer(mode=mode, source=source, make_pool=make_pool, n_swa=128, q=FAKE, idx_q=FAKE, head_w=FAKE,
                   swa_kv=FAKE, swa_first_pos=FAKE, out=FAKE, lse=None, topk=topk, pool=pool)


@pytest.mark.parametrize(
    "layers,status",
    [
        ([layer(B.REUSE, 0)], -4),  # Reuse without an earlier layer
        ([layer(B.FULL), layer(B.REUSE, 1)], -4),  # source is not earlier
        ([layer(B.FULL), layer(B.REUSE, 0, topk=None), layer(B.REUSE, 1)], -4),  # Reuse of a Reuse
        ([layer(B.FULL), layer(B.REINDEX, 0)], -4),  # Reindex source without a pool
        ([layer(B.FULL, 0)], -4),  # Full with a source
        ([layer(B.FULL, make_pool=1, pool=None)], -1),  # pool requested without buffer
        ([layer(7)], -2),
    ],
)
def test_layer_group_mode_order(layers, status):
    lib = B.library()
    arr = (B.Layer * len(layers))(*layers)
    assert lib.csa2_layer_group(ctypes.byref(dims()), ctypes.byref(cache()), len(layers), arr, FAKE, 1, None, FAKE,
                                1 << 40, None) == status


@pytest.mark.parametrize("heads,d", [(8, 64), (64, 512), (32, 512), (1, 32)])
def test_workspace_size_any_head_count(heads, d):
    """Sizing never divides by a head-group count (8 heads, 64-d is the tiny workload)."""
    n = B.csa2_workspace_size(dims(n_heads=heads, d=d, d_rope=16), cache(), B.EP_SPARSE_ATTN, 16)
    assert n >= 0
    assert B.csa2_workspace_size(dims(n_heads=heads, d=d, d_rope=16), cache(), B.EP_LAYER_GROUP, 16) > 0


def test_workspace_size():
    d, c = dims(), cache()
    n = B.csa2_workspace_size(d, c, B.EP_INDEX_TOPK, 1)
    rows = c.batch
    assert n >= rows * 4096 * 4 + rows * 512 * 4 + rows * 64 * 4
    assert B.csa2_workspace_size(d, c, B.EP_COMPRESS, 1) == 0
    assert B.csa2_workspace_size(d, c, B.EP_LAYER_GROUP, 1) >= n
    with pytest.raises(B.Csa2Error):
        B.csa2_workspace_size(dims(d=3), c, B.EP_INDEX_TOPK, 1)
    for n_q in (0, 65536):  # outside the calls' 1..65535
        with pytest.raises(B.Csa2Error):
            B.csa2_workspace_size(d, c, B.EP_INDEX_TOPK, n_q)
    assert B.csa2_workspace_size(d, c, B.EP_INDEX_TOPK, 65535) > 0


def test_trace_api_without_launches():
    from kv_cache_compression_csa2_amd import binding as B

    assert B.csa2_kernel_name(3) == "scan_mfma_bf16_kernel"
    assert B.csa2_kernel_name(5) == "select_kernel"
    assert B.csa2_kernel_name(99) == "unknown"
    lib = B.library()
    assert lib.csa2_trace_enable(-1) == -1  # CSA2_ERR_INVALID_ARG
    recs, dropped = B.csa2_trace_read(16)
    assert recs == [] and dropped == 0
    st = lib.csa2_trace_enable(4)  # no device here: a HIP error; with one: enabled
    assert st in (0, -5)
    assert lib.csa2_trace_enable(0) == 0


@pytest.mark.parametrize("args, status", [
    ((B.FP4, 4, 512, 8, 64), -2),   # cache-only dtype
    ((B.BF16, 4, 500, 8, 64), -1),  # width not a multiple of the groups
    ((B.BF16, -1, 512, 8, 64), -1),
    ((B.BF16, 4, 512, 0, 64), -1),
    ((B.BF16, 4, 512, 8, 0), -1),
])
def test_grouped_out_proj_rejects_bad_arguments(args, status):
    lib = B.library()
    assert lib.csa2_grouped_out_proj(*args, FAKE, FAKE, FAKE, None) == status
    assert B.last_error()


def test_grouped_out_proj_checks_pointers_and_allows_no_tokens():
    lib = B.library()
    assert lib.csa2_grouped_out_proj(B.BF16, 4, 512, 8, 64, None, FAKE, FAKE, None) == -1
    assert lib.csa2_grouped_out_proj(B.BF16, 4, 512, 8, 64, FAKE + 2, FAKE, FAKE, None) == -1
    # no tokens: nothing to do, no pointer needed, no GPU call
    assert lib.csa2_grouped_out_proj(B.BF16, 0, 512, 8, 64, None, None, None, None) == 0
    assert B.last_error() == ""


def test_read_probe_rejects_bad_arguments():
    lib = B.library()
    assert lib.csa2_read_probe(FAKE, 0, FAKE, None) == -1
    assert lib.csa2_read_probe(FAKE, 24, FAKE, None) == -1
    assert lib.csa2_read_probe(None, 1 << 20, FAKE, None) == -1
    assert lib.csa2_read_probe(FAKE + 8, 1 << 20, FAKE, None) == -1
    assert lib.csa2_read_probe(FAKE, 1 << 20, None, None) == -1
    assert B.csa2_kernel_name(16) == "read_probe_kernel"


def test_mfma_probe_rejects_bad_arguments():
    lib = B.library()
    assert lib.csa2_mfma_probe(0, 512, FAKE, None) == -1
    assert lib.csa2_mfma_probe((1 << 24) + 1, 512, FAKE, None) == -1
    assert lib.csa2_mfma_probe(16, 0, FAKE, None) == -1
    assert lib.csa2_mfma_probe(16, 65537, FAKE, None) == -1
    assert lib.csa2_mfma_probe(16, 512, None, None) == -1
    assert B.csa2_kernel_name(17) == "mfma_probe_kernel"
    assert B.csa2_kernel_name(18) == "scan_fused_bf16_kernel"
    assert B.csa2_kernel_name(19) == "scan_fused_fp4_kernel"
    assert B.MFMA_PROBE_FLOP_PER_WG_ITER == 4 * 8 * 32 * 32 * 16 * 2


def test_noalloc_group_checks_arguments_and_its_scratch_limit_before_any_hip_call():
    """csa2_layer_group_noalloc runs the same checks as csa2_layer_group and
    refuses a shape whose scratch exceeds CSA2_NOALLOC_SCRATCH_BYTES (64 MiB)
    with CSA2_ERR_WORKSPACE, before it touches the GPU."""
    lib = B.library()
    arr = (B.Layer * 1)(layer(B.REUSE, 0))
    assert lib.csa2_layer_group_noalloc(ctypes.byref(dims()), ctypes.byref(cache()), 1, arr, FAKE, 1, None, None) == -4
    arr = (B.Layer * 1)(layer(B.FULL))
    big = cache(batch=64, capacity=1 << 20)  # 64 sequences x 1M entries: ~300 MB of scores
    need = B.csa2_workspace_size(dims(), big, B.EP_LAYER_GROUP, 1)
    assert need > 64 << 20
    assert lib.csa2_layer_group_noalloc(ctypes.byref(dims()), ctypes.byref(big), 1, arr, FAKE, 1, None, None) == -3
    assert "64 MiB" in B.last_error() or str(64 << 20) in B.last_error()
    # the decode shapes it is for fit
    for b, cap in ((16, 32768), (2, 1 << 20), (4, 1 << 18)):
        assert B.csa2_workspace_size(dims(), cache(batch=b, capacity=cap), B.EP_LAYER_GROUP, 1) <= 64 << 20
