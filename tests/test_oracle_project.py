"""Pins for the oracle's value projection (W_UV) fused after the LSE merge.

Tied to: scalar loops on tiny inputs, a closed form (weights that pick
entries of the latent), and the page's own order of operations (projecting
each split before the merge gives the same result).  A projection over the
wrong axis of the weights fails the brute-force pin.
"""
import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O


def _bf16_bits(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _brute(x, w):
    r, h, k = x.shape
    dv = w.shape[1]
    out = np.zeros((r, h, dv))
    for a in range(r):
        for b in range(h):
            for d in range(dv):
                acc = 0.0
                for j in range(k):
                    acc += x[a, b, j] * w[b, d, j]
                out[a, b, d] = acc
    return out


def test_projection_matches_scalar_loops():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 2, 512))
    wb = _bf16_bits(rng.standard_normal((2, 5, 512)) / 20)
    got = O.project_v(x, wb)
    np.testing.assert_allclose(got, _brute(x, O.bf16_decode(wb)), rtol=1e-12, atol=1e-12)


def test_selection_weights_pick_latent_entries():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 3, 512))
    w = np.zeros((3, 128, 512), dtype=np.float32)
    pick = rng.integers(0, 512, (3, 128))
    for h in range(3):
        w[h, np.arange(128), pick[h]] = 1.0
    got = O.project_v(x, _bf16_bits(w))
    for h in range(3):
        np.testing.assert_array_equal(got[:, h], x[:, h, pick[h]])


def test_projecting_each_split_before_the_merge_gives_the_same_result():
    rng = np.random.default_rng(3)
    r, h, s = 4, 3, 5
    po = rng.standard_normal((r, h, s, 512))
    pl = rng.standard_normal((r, h, s)) * 3
    pl[0, 1, :] = -np.inf        # an empty row
    pl[2, 0, 1] = -np.inf        # an empty split
    wb = _bf16_bits(rng.standard_normal((h, 128, 512)) / 20)
    out, lse = O.lse_merge_project(po, pl, wb)
    # the page's order: project every split, then merge
    proj = np.einsum("rhsk,hdk->rhsd", po, O.bf16_decode(wb))
    out2, lse2 = O.lse_merge(proj, pl)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(lse, lse2)
    assert np.all(out[0, 1] == 0) and np.isneginf(lse[0, 1])


def test_wrong_weight_axis_fails_the_brute_force_pin():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((2, 2, 512))
    wb = _bf16_bits(rng.standard_normal((2, 512, 512)) / 20)   # square, so both axes type-check
    w = O.bf16_decode(wb)
    wrong = np.einsum("rhk,hkd->rhd", x, w)                   # contracts the output axis instead
    assert not np.allclose(wrong, _brute(x, w), rtol=1e-6)
    np.testing.assert_allclose(O.project_v(x, wb), _brute(x, w), rtol=1e-12, atol=1e-12)
