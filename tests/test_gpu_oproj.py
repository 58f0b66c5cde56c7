"""GPU parity of csa2_grouped_out_proj (zartbot walkthrough, section 1.2:
o_lora_rank 1024 in o_groups 8) against the float64 oracle on seeded inputs.

Tolerance, from the arithmetic: products of bf16 (or float32) inputs are
summed in float32, in an order the matrix cores choose, so a sum of K terms
is within K 2^-24 S of the exact one, S = sum |x_c w_c| (the oracle on |x|,
|w|); a bf16 output (8 significant bits) then rounds to nearest, within
2^-8 of its value.
"""
import numpy as np
import pytest

import synth
from oracle import csa2 as oc

pytestmark = pytest.mark.gpu

# (n_tok, width, groups, rank, act, rows the oracle checks: None = all)
CASES = [
    (16, 32768, 8, 1024, "bf16", None),  # decode: 16 sequences x 64 heads x 512
    (4096, 32768, 8, 1024, "bf16", [0, 1, 31, 32, 33, 2047, 2048, 4064, 4095]),  # a 4096-query chunk
    (37, 512, 4, 96, "bf16", None),  # ragged token tile, one output tile per wave
    (1000, 1024, 8, 128, "bf16", None),  # two output tiles per wave, ragged tokens
    (130, 1024, 2, 64, "bf16", None),  # K 512: 8 chunks, one per wave
    (5, 96, 3, 20, "f32", None),  # plain kernel, float32
    (3, 96, 3, 32, "bf16", None),  # K 32: plain kernel in bf16
    (7, 512, 1, 64, "bf16", None),  # one group
    (1, 4096, 8, 32, "bf16", None),  # one token
    (9, 10240, 2, 64, "bf16", None),  # K 5120: waves past 4 chunks loop again, with masked tails
    (17, 4096, 4, 64, "bf16", None),  # just past the 16-token kernel
    (1000, 1024, 8, 512, "bf16", None),  # 128 x 128 LDS tiles, ragged last token tile
    (500, 1536, 8, 1024, "bf16", None),  # LDS tiles with an odd number of 64-channel slices
]


def _run(n_tok, width, groups, rank, act):
    import torch

    from kv_cache_compression_csa2_amd import binding as B

    x, w = synth.oproj_inputs(n_tok, width, groups, rank, act)
    tdt = torch.bfloat16 if act == "bf16" else torch.float32
    xd = torch.from_numpy(x).to("cuda").to(tdt)
    wd = torch.from_numpy(w).to("cuda").to(tdt)
    y = torch.full((n_tok, groups * rank), float("nan"), dtype=tdt, device="cuda")
    B.csa2_grouped_out_proj(B.BF16 if act == "bf16" else B.F32, n_tok, width, groups, rank, xd, wd, y)
    torch.cuda.synchronize()
    return x, w, y.float().cpu().numpy()


@pytest.mark.parametrize("n_tok, width, groups, rank, act, rows", CASES)
def test_grouped_out_proj_parity(n_tok, width, groups, rank, act, rows):
    print(f"[oproj] tokens {n_tok}, width {width}, groups {groups}, rank {rank}, {act}", flush=True)
    x, w, y = _run(n_tok, width, groups, rank, act)
    assert not np.isnan(y).any(), "outputs left unwritten"
    sel = np.arange(n_tok) if rows is None else np.asarray(rows)
    ref = oc.grouped_out_proj(x[sel], w)
    mag = oc.grouped_out_proj(np.abs(x[sel]), np.abs(w))
    k = width // groups
    tol = k * 2.0 ** -24 * mag * (1 + 2.0 ** -8)
    if act == "bf16":
        tol += 2.0 ** -8 * np.abs(ref)
    err = np.abs(y[sel] - ref)
    worst = np.unravel_index(np.argmax(err - tol), err.shape)
    assert np.all(err <= tol), f"max excess at {worst}: got {y[sel][worst]}, want {ref[worst]}, tol {tol[worst]}"


def test_grouped_out_proj_no_tokens_writes_nothing():
    import torch

    from kv_cache_compression_csa2_amd import binding as B

    y = torch.full((4, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((4, 512), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((8, 8, 64), dtype=torch.bfloat16, device="cuda")
    B.csa2_grouped_out_proj(B.BF16, 0, 512, 8, 8, x, w, y)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)
