"""ctypes binding of libcsa2.so: the csa2.h entry points under the same names.

Argument marshalling only: torch tensors become device pointers, the current
torch stream becomes the HIP stream, and a negative status raises
``Csa2Error``.  Every step of the path runs in the library's kernels; if the
library is missing the import fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_int, c_int32, c_int64, c_size_t, c_void_p

# torch ships its own HIP runtime (soname libamdhip64.so.7).  Loading torch
# first makes libcsa2.so bind to that same runtime instead of pulling a second
# copy from /opt/rocm: one process must run one HIP runtime, or device
# pointers and streams from torch would belong to a runtime our kernels do
# not run in.
import torch  # noqa: F401  (must precede the CDLL below)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa2.so")

F32, BF16, FP4, FP8 = 0, 1, 2, 3
FULL, REINDEX, REUSE = 0, 1, 2
EP_COMPRESS, EP_INDEX_TOPK, EP_SPARSE_ATTN, EP_LAYER_GROUP = 0, 1, 2, 3


class Csa2Error(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{status_str(status)} ({status}): {msg}")
        self.status = status


class Dims(ctypes.Structure):
    _fields_ = [
        ("d", c_int32), ("d_rope", c_int32), ("n_heads", c_int32), ("n_idx_heads", c_int32), ("d_idx", c_int32),
        ("topk", c_int32), ("window", c_int32), ("block_size", c_int32), ("cand_blocks", c_int32),
        ("act_dtype", c_int32), ("rope_theta", c_double), ("swa_dtype", c_int32), ("rope_orig_len", c_int32),
        ("rope_factor", c_double),
    ]


class KVCache(ctypes.Structure):
    _fields_ = [
        ("kv_dtype", c_int32), ("ratio", c_int32), ("main_group", c_int32), ("idx_group", c_int32),
        ("batch", c_int32), ("reserved0", c_int32), ("capacity", c_int64),
        ("main", c_void_p), ("main_scale", c_void_p), ("idx_k", c_void_p), ("idx_scale", c_void_p),
        ("n_entries", c_void_p),
    ]


class Layer(ctypes.Structure):
    _fields_ = [
        ("mode", c_int32), ("source", c_int32), ("make_pool", c_int32), ("n_swa", c_int32),
        ("q", c_void_p), ("idx_q", c_void_p), ("head_w", c_void_p), ("swa_kv", c_void_p),
        ("swa_first_pos", c_void_p), ("out", c_void_p), ("lse", c_void_p), ("topk", c_void_p), ("pool", c_void_p),
    ]


class TraceRecord(ctypes.Structure):
    _fields_ = [("kernel", c_int32), ("ms", ctypes.c_float)]


class PlanLayer(ctypes.Structure):
    _fields_ = [("group", c_int32), ("mode", c_int32), ("source", c_int32), ("make_pool", c_int32)]


class CompressArgs(ctypes.Structure):
    _fields_ = [
        ("latent", c_void_p), ("first_pos", c_void_p), ("n_pos", c_int32), ("reserved0", c_int32),
        ("pair_logits", c_void_p), ("w_ik", c_void_p),
    ]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m kv_cache_compression_csa2_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

_lib.csa2_abi_version.restype = c_int32
_lib.csa2_status_str.restype = ctypes.c_char_p
_lib.csa2_status_str.argtypes = [c_int]
_lib.csa2_last_error.restype = ctypes.c_char_p
_lib.csa2_workspace_size.restype = c_size_t
_lib.csa2_workspace_size.argtypes = [POINTER(Dims), POINTER(KVCache), c_int32, c_int32]
_lib.csa2_compress.restype = c_int
_lib.csa2_compress.argtypes = [POINTER(Dims), POINTER(KVCache), c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p]
_lib.csa2_index_topk.restype = c_int
_lib.csa2_index_topk.argtypes = [POINTER(Dims), POINTER(KVCache), c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                 c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
_lib.csa2_sparse_attn.restype = c_int
_lib.csa2_sparse_attn.argtypes = [POINTER(Dims), POINTER(KVCache), c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                  c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
_lib.csa2_layer_group.restype = c_int
_lib.csa2_layer_group.argtypes = [POINTER(Dims), POINTER(KVCache), c_int32, POINTER(Layer), c_void_p, c_int32,
                                  POINTER(CompressArgs), c_void_p, c_size_t, c_void_p]
_lib.csa2_layer_plan.restype = c_int
_lib.csa2_layer_plan.argtypes = [c_int32, POINTER(c_int32), c_int32, POINTER(c_int32), c_int32, POINTER(c_int32),
                                 c_int32, POINTER(PlanLayer)]
_lib.csa2_layer_group_noalloc.restype = c_int
_lib.csa2_layer_group_noalloc.argtypes = [POINTER(Dims), POINTER(KVCache), c_int32, POINTER(Layer), c_void_p, c_int32,
                                          POINTER(CompressArgs), c_void_p]
_lib.csa2_grouped_out_proj.restype = c_int
_lib.csa2_grouped_out_proj.argtypes = [c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p,
                                       c_void_p]
_lib.csa2_trace_enable.restype = c_int
_lib.csa2_trace_enable.argtypes = [c_int32]
_lib.csa2_trace_read.restype = c_int
_lib.csa2_trace_read.argtypes = [POINTER(TraceRecord), c_int32, POINTER(c_int32)]
_lib.csa2_read_probe.restype = c_int
_lib.csa2_read_probe.argtypes = [c_void_p, c_int64, c_void_p, c_void_p]
_lib.csa2_mfma_probe.restype = c_int
_lib.csa2_mfma_probe.argtypes = [c_int64, c_int32, c_void_p, c_void_p]
_lib.csa2_kernel_name.restype = ctypes.c_char_p
_lib.csa2_kernel_name.argtypes = [c_int32]

EXPORTED = ("csa2_compress", "csa2_index_topk", "csa2_sparse_attn", "csa2_layer_group", "csa2_workspace_size",
            "csa2_status_str", "csa2_last_error", "csa2_abi_version", "csa2_trace_enable", "csa2_trace_read",
            "csa2_kernel_name", "csa2_grouped_out_proj", "csa2_read_probe", "csa2_mfma_probe",
            "csa2_layer_group_noalloc", "csa2_layer_plan")


def library() -> ctypes.CDLL:
    return _lib


def status_str(status: int) -> str:
    return _lib.csa2_status_str(status).decode()


def last_error() -> str:
    return _lib.csa2_last_error().decode()


def _check(status: int) -> None:
    if status != 0:
        raise Csa2Error(status, last_error())


def ptr(t) -> c_void_p:
    """Device pointer of a contiguous torch tensor (None -> NULL)."""
    if t is None:
        return c_void_p(None)
    if isinstance(t, int):
        return c_void_p(t)
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch

        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def csa2_abi_version() -> int:
    return _lib.csa2_abi_version()


def csa2_workspace_size(dims: Dims, cache: KVCache, entry_point: int, n_q: int) -> int:
    n = _lib.csa2_workspace_size(ctypes.byref(dims), ctypes.byref(cache), entry_point, n_q)
    if n == 0 and last_error():
        raise Csa2Error(-1, last_error())
    return n


def csa2_compress(dims, cache, latent, first_pos, n_pos, pair_logits, w_ik, stream=None) -> None:
    _check(_lib.csa2_compress(ctypes.byref(dims), ctypes.byref(cache), ptr(latent), ptr(first_pos), n_pos,
                              ptr(pair_logits), ptr(w_ik), _stream(stream)))


def csa2_index_topk(dims, cache, idx_q, head_w, q_pos, n_q, pool_in, topk_out, pool_out, topk_scores, ws,
                    stream=None) -> None:
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.csa2_index_topk(ctypes.byref(dims), ctypes.byref(cache), ptr(idx_q), ptr(head_w), ptr(q_pos), n_q,
                                ptr(pool_in), ptr(topk_out), ptr(pool_out), ptr(topk_scores), ptr(ws), ws_bytes,
                                _stream(stream)))


def csa2_sparse_attn(dims, cache, q, q_pos, n_q, topk, swa_kv, swa_first_pos, n_swa, out, lse, ws,
                     stream=None) -> None:
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.csa2_sparse_attn(ctypes.byref(dims), ctypes.byref(cache), ptr(q), ptr(q_pos), n_q, ptr(topk),
                                 ptr(swa_kv), ptr(swa_first_pos), n_swa, ptr(out), ptr(lse), ptr(ws), ws_bytes,
                                 _stream(stream)))


def csa2_layer_group(dims, cache, layers, q_pos, n_q, compress, ws, stream=None) -> None:
    """``layers``: a sequence of Layer structs; ``compress``: CompressArgs or None."""
    arr = (Layer * len(layers))(*layers)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(_lib.csa2_layer_group(ctypes.byref(dims), ctypes.byref(cache), len(layers), arr, ptr(q_pos), n_q,
                                 None if compress is None else ctypes.byref(compress), ptr(ws), ws_bytes,
                                 _stream(stream)))


def csa2_layer_plan(ratios, kv_src, idx_src, cand_src) -> list[tuple[int, int, int, int]]:
    """(group, mode, source, make_pool) per layer, from host lists (see csa2.h)."""
    n = len(ratios)
    arr = lambda xs: (c_int32 * max(1, len(xs)))(*xs)
    out = (PlanLayer * n)()
    _check(_lib.csa2_layer_plan(n, arr(ratios), len(kv_src), arr(kv_src), len(idx_src), arr(idx_src), cand_src, out))
    return [(p.group, p.mode, p.source, p.make_pool) for p in out]


def csa2_layer_group_noalloc(dims, cache, layers, q_pos, n_q, compress, stream=None) -> None:
    """csa2_layer_group with the library's own scratch (no workspace argument)."""
    arr = (Layer * len(layers))(*layers)
    _check(_lib.csa2_layer_group_noalloc(ctypes.byref(dims), ctypes.byref(cache), len(layers), arr, ptr(q_pos), n_q,
                                         None if compress is None else ctypes.byref(compress), _stream(stream)))


def csa2_grouped_out_proj(act_dtype, n_tok, width, n_groups, rank, x, w, y, stream=None) -> None:
    """y[t][g*rank + r] = sum_c x[t][g*K + c] * w[g][r][c], K = width / n_groups."""
    _check(_lib.csa2_grouped_out_proj(act_dtype, n_tok, width, n_groups, rank, ptr(x), ptr(w), ptr(y),
                                      _stream(stream)))


def csa2_trace_enable(max_kernels: int) -> None:
    """Record device times of up to ``max_kernels`` launches (0 turns tracing off)."""
    _check(_lib.csa2_trace_enable(max_kernels))


def csa2_trace_read(max_records: int = 65536) -> tuple[list[tuple[str, float]], int]:
    """(kernel name, ms) per recorded launch in launch order, and the dropped count."""
    buf = (TraceRecord * max_records)()
    dropped = c_int32(0)
    n = _lib.csa2_trace_read(buf, max_records, ctypes.byref(dropped))
    if n < 0:
        raise Csa2Error(n, "trace read failed")
    return [(csa2_kernel_name(buf[i].kernel), float(buf[i].ms)) for i in range(n)], int(dropped.value)


MFMA_PROBE_FLOP_PER_WG_ITER = 4 * 8 * 32768  # CSA2_MFMA_PROBE_FLOP_PER_WG_ITER


def csa2_mfma_probe(iters: int, workgroups: int, sink, stream=None) -> None:
    _check(_lib.csa2_mfma_probe(iters, workgroups, ptr(sink), _stream(stream)))


def csa2_read_probe(buf, nbytes: int, sink, stream=None) -> None:
    """Stream ``nbytes`` of device tensor ``buf`` once (a measurement utility; see csa2.h)."""
    _check(_lib.csa2_read_probe(ptr(buf), nbytes, ptr(sink), _stream(stream)))


def csa2_kernel_name(kernel: int) -> str:
    return _lib.csa2_kernel_name(kernel).decode()
