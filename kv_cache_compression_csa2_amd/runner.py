"""Device buffers for one CSA2 workload and a step through the C ABI.

Plumbing only: torch allocates device memory and supplies the stream; every
computation happens in libcsa2's kernels.  ``wl`` is a workload description
(batch, ratio, widths, top-k, window, dtypes, prior/new positions, queries,
layer plan) and ``inp`` its seeded inputs (float32 arrays whose values are
exact in the activation dtype).
"""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B

_DT = {"f32": B.F32, "bf16": B.BF16, "fp4": B.FP4}
_MODE = {"full": B.FULL, "reindex": B.REINDEX, "reuse": B.REUSE}


def act_tensor(x: np.ndarray, act: str, device) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    return t.to(torch.bfloat16) if act == "bf16" else t


def make_dims(wl) -> B.Dims:
    return B.Dims(d=wl.d, d_rope=wl.d_rope, n_heads=wl.n_heads, n_idx_heads=wl.n_idx_heads, d_idx=wl.d_idx,
                  topk=wl.topk, window=wl.window, block_size=wl.block_size, cand_blocks=wl.cand_blocks,
                  act_dtype=_DT[wl.act], rope_theta=wl.rope_theta, swa_dtype=B.FP8 if wl.swa == "fp8" else 0,
                  rope_orig_len=wl.rope_orig_len, rope_factor=wl.rope_factor)


def idx_padded_rows(capacity: int) -> int:
    """Indexer K rows per sequence in the library's tile storage (32-row tiles)."""
    return (capacity + 31) // 32 * 32


class DeviceCache:
    """Main KV + indexer K of ``batch`` sequences with ``capacity`` entry slots.

    The indexer K lives in the library's tile storage (``idx_store``: per
    sequence, 32-row tiles whose 16-byte chunks are transposed); ``idx``
    returns it as row-major rows ([batch][padded rows][...]) for inspection.
    """

    def __init__(self, wl, capacity: int, device="cuda"):
        self.wl = wl
        self.capacity = capacity
        b, d, di = wl.batch, wl.d, wl.d_idx
        kv = wl.kv
        rows = idx_padded_rows(capacity)
        if kv == "fp4":
            self.main = torch.zeros((b, capacity, d // 2), dtype=torch.uint8, device=device)
            self.main_scale = torch.zeros((b, capacity, d // wl.main_group), dtype=torch.uint8, device=device)
            self.idx_dtype, self.idx_row_bytes = torch.uint8, di // 2
            self.idx_scale = torch.zeros((b, capacity, di // wl.idx_group), dtype=torch.uint8, device=device)
        else:
            dt = torch.bfloat16 if kv == "bf16" else torch.float32
            self.main = torch.zeros((b, capacity, d), dtype=dt, device=device)
            self.idx_dtype, self.idx_row_bytes = dt, di * (2 if kv == "bf16" else 4)
            self.main_scale = self.idx_scale = None
        self.idx_store = torch.zeros((b, rows * self.idx_row_bytes), dtype=torch.uint8, device=device)
        self.n_entries = torch.zeros(b, dtype=torch.int32, device=device)

    @property
    def idx(self) -> torch.Tensor:
        """The indexer K as row-major rows (a copy), [batch][padded rows][d_idx or d_idx/2]."""
        b, rb = self.wl.batch, self.idx_row_bytes
        t = self.idx_store.view(b, -1, rb // 16, 32, 16).permute(0, 1, 3, 2, 4).reshape(b, -1, rb)
        return t.contiguous().view(self.idx_dtype)

    def struct(self, with_idx: bool = True) -> B.KVCache:
        wl = self.wl
        return B.KVCache(
            kv_dtype=_DT[wl.kv], ratio=wl.ratio, main_group=wl.main_group, idx_group=wl.idx_group, batch=wl.batch,
            reserved0=0, capacity=self.capacity, main=B.ptr(self.main), main_scale=B.ptr(self.main_scale),
            idx_k=B.ptr(self.idx_store) if with_idx else None, idx_scale=B.ptr(self.idx_scale) if with_idx else None,
            n_entries=B.ptr(self.n_entries),
        )


class DeviceStep:
    """All device tensors of one step of ``wl`` and the calls that run it."""

    def __init__(self, wl, inp, device="cuda", build_prior=True, prior_chunk=1 << 15):
        self.wl, self.inp, self.device = wl, inp, device
        self.dims = make_dims(wl)
        self.cache = DeviceCache(wl, wl.capacity, device)
        logits = inp.pair_logits()
        self.pair_logits = None if logits is None else torch.from_numpy(logits).to(device)
        self.w_ik = act_tensor(inp.w_ik(), wl.act, device)
        if build_prior and wl.prior:
            self.build_prior(prior_chunk)
        self.cache.n_entries.fill_(wl.capacity)
        # step inputs
        self.first_pos = torch.full((wl.batch,), wl.prior, dtype=torch.int32, device=device)
        if wl.new:
            lat = np.stack([inp.latent(b, wl.prior, wl.context) for b in range(wl.batch)])
            self.latent_new = act_tensor(lat, wl.act, device)
        self.q_pos = torch.from_numpy(wl.q_positions()).to(device)
        self.layers = []
        for li, plan in enumerate(wl.layers):
            swa, swa_first = inp.swa(li)
            L = dict(
                plan=plan, q=act_tensor(inp.q(li), wl.act, device),
                swa=(torch.from_numpy(swa).to(device) if wl.swa == "fp8" else act_tensor(swa, wl.act, device)),
                swa_first=torch.from_numpy(swa_first).to(device),
                out=torch.empty((wl.batch, wl.n_q, wl.n_heads, wl.d), device=device,
                                dtype=torch.bfloat16 if wl.act == "bf16" else torch.float32),
                lse=torch.empty((wl.batch, wl.n_q, wl.n_heads), dtype=torch.float32, device=device),
                topk=torch.full((wl.batch, wl.n_q, wl.topk), -7, dtype=torch.int32, device=device),
                pool=torch.full((wl.batch, wl.n_q, wl.cand_blocks), -7, dtype=torch.int32, device=device)
                if plan.make_pool else None,
            )
            if plan.mode != "reuse":
                L["q_idx"] = act_tensor(inp.q_idx(li), wl.act, device)
                L["head_w"] = torch.from_numpy(inp.head_w(li)).to(device)
            self.layers.append(L)
        cs = self.cache.struct()
        self.ws = torch.empty(B.csa2_workspace_size(self.dims, cs, B.EP_LAYER_GROUP, wl.n_q) + 256,
                              dtype=torch.uint8, device=device)

    def workspace(self) -> torch.Tensor:
        """The workspace, 256-byte aligned."""
        off = (-self.ws.data_ptr()) % 256
        return self.ws[off:]

    def build_prior(self, chunk: int) -> None:
        """Compress every prior latent row into the cache (chunked; not part of a step)."""
        wl = self.wl
        chunk -= chunk % wl.ratio
        cs = self.cache.struct()
        for p0 in range(0, wl.prior, chunk):
            p1 = min(wl.prior, p0 + chunk)
            lat = np.stack([self.inp.latent(b, p0, p1) for b in range(wl.batch)])
            lat_t = act_tensor(lat, wl.act, self.device)
            fp = torch.full((wl.batch,), p0, dtype=torch.int32, device=self.device)
            B.csa2_compress(self.dims, cs, lat_t, fp, p1 - p0, self.pair_logits, self.w_ik)
        torch.cuda.synchronize()

    def layer_structs(self) -> list:
        out = []
        for L in self.layers:
            plan = L["plan"]
            out.append(B.Layer(
                mode=_MODE[plan.mode], source=plan.source, make_pool=int(plan.make_pool),
                n_swa=L["swa"].shape[1], q=B.ptr(L["q"]), idx_q=B.ptr(L.get("q_idx")), head_w=B.ptr(L.get("head_w")),
                swa_kv=B.ptr(L["swa"]), swa_first_pos=B.ptr(L["swa_first"]), out=B.ptr(L["out"]), lse=B.ptr(L["lse"]),
                topk=B.ptr(L["topk"]), pool=B.ptr(L["pool"]),
            ))
        return out

    def compress_args(self):
        if not self.wl.new:
            return None
        return B.CompressArgs(latent=B.ptr(self.latent_new), first_pos=B.ptr(self.first_pos), n_pos=self.wl.new,
                              reserved0=0, pair_logits=B.ptr(self.pair_logits), w_ik=B.ptr(self.w_ik))

    def run(self, stream=None) -> None:
        """One step: compress the new rows, then every layer of the group."""
        B.csa2_layer_group(self.dims, self.cache.struct(), self.layer_structs(), self.q_pos, self.wl.n_q,
                           self.compress_args(), self.workspace(), stream)
