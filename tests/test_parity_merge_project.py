"""GPU parity of the LSE merge followed by the W_UV value projection,
through the C ABI, against the oracle.

Tolerance, from the arithmetic: the kernel rounds the merged latent to bf16
(unit roundoff u = 2^-9) before the projection, accumulates the products in
fp32 and rounds the output to bf16, so |g - r| <= u * sum_k |latent_k w_dk|
+ u * |r| plus fp32 terms far below; the check allows twice that.  The LSE
follows R15 (1e-3 absolute).
"""
import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from parity_util import LSE_ATOL
from sparse_attention_decode_dsa_amd import dsa
from sparse_attention_decode_dsa_amd import workload as W

pytestmark = pytest.mark.gpu
U = 2.0 ** -9


def _u16(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def check_projected(g_out, g_lse, latent, w_bits, r_lse):
    """g_out [R,H,Dv] from the GPU; latent [R,H,512] the oracle's merged
    latent; returns the largest error in units of the bound."""
    w = O.bf16_decode(w_bits)
    ref = O.project_v(latent, w_bits)
    mag = np.einsum("rhk,hdk->rhd", np.abs(latent), np.abs(w))
    bound = 2 * U * (mag + np.abs(ref)) + 1e-30
    err = np.abs(g_out - ref)
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert worst <= 1.0, f"projected output off by {worst:.2f} of the bound"
    fin = np.isfinite(r_lse)
    assert np.array_equal(fin, np.isfinite(g_lse))
    if fin.any():
        assert np.max(np.abs(g_lse[fin] - r_lse[fin])) <= LSE_ATOL
    return worst


@pytest.mark.parametrize("rows,heads,splits", [(37, 32, 4), (16, 16, 1), (5, 32, 32), (64, 32, 64)])
def test_synthetic_partials(rows, heads, splits):
    po, pl = W.make_partials(rows, heads, splits, seed=rows + splits)
    w = W.make_w_uv(heads, seed=heads)
    out, lse = dsa.lse_merge_project(po.cuda(), pl.cuda(), w.cuda())
    torch.cuda.synchronize()
    latent, r_lse = O.lse_merge(po.double().numpy(), pl.double().numpy())
    worst = check_projected(out.float().cpu().double().numpy(), lse.cpu().double().numpy(), latent, _u16(w), r_lse)
    print(f"  worst {worst:.3f} of the bound", flush=True)
    if rows >= 3:    # the all-empty row projects to zero
        assert torch.all(out[2] == 0) and torch.all(torch.isneginf(lse[2]))


def test_after_the_tiny_decode_step():
    """The step's own partials (4 attention splits) merged and projected on the
    GPU.  The step is checked against the oracle as in the step's parity; the
    merge and projection against the oracle's merge of the same bf16 partials
    and LSEs, projected (the partials' own rounding is the attention's, which
    the step's check covers)."""
    from test_parity_gpu import compare_step, run_step
    inp = W.to(W.make("c0"), "cuda")
    step = run_step(inp, 4, 4)
    compare_step(inp, step, range(inp.n_rows), max_swap_rows=1)
    w = W.make_w_uv(inp.mla_heads, seed=7)
    out, lse = dsa.lse_merge_project(step.part_o, step.part_lse, w.cuda())
    torch.cuda.synchronize()
    latent, r_lse = O.lse_merge(step.part_o.double().cpu().numpy(), step.part_lse.double().cpu().numpy())
    check_projected(out.float().cpu().double().numpy(), lse.cpu().double().numpy(), latent, _u16(w), r_lse)