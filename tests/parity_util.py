"""Comparison rules shared by the GPU parity tests.

Tolerances (stated where the pages or the arithmetic fix them):
* fp8 codes, top-k counts and index sets: bit-exact, except that the two
  sets may differ only by slots whose oracle score lies within 1e-3 relative
  of the oracle's k-th score (the tie band; absolute floor 1e-6 * max|s|
  for a k-th score near zero); ties at bitwise-equal scores keep the lower
  slot on both sides.
* attention output (bf16): per (row, head) max|g - r| / max|r| <= 2e-2.
* lse: |g - r| <= 1e-3 absolute.
* scores (diagnostic): |g - r| <= 1e-4 * max_t |r_t| per row; the GPU sums
  fp8 products in fp32 in MFMA order, the oracle in fp64.
"""
import numpy as np

OUT_RTOL = 2e-2
LSE_ATOL = 1e-3
SCORE_RTOL = 1e-4
BAND_REL = 1e-3


def bf16_to_f64(t):
    return t.float().cpu().double().numpy()


def check_topk_row(g_idx, g_cnt, o_idx, o_cnt, o_scores, v, k):
    """Returns the number of tie-band swaps (0 when the sets are equal)."""
    g_idx = np.asarray(g_idx)
    o_idx = np.asarray(o_idx)
    assert g_cnt == o_cnt == min(k, v), (g_cnt, o_cnt, v, k)
    sel = g_idx[:g_cnt]
    assert np.all(g_idx[g_cnt:] == -1)
    assert np.all(np.diff(sel) > 0), "selected slots must be strictly ascending"
    assert g_cnt == 0 or (sel[0] >= 0 and sel[-1] < v)
    gs, os_ = set(sel.tolist()), set(o_idx[:o_cnt].tolist())
    diff = gs ^ os_
    if not diff:
        return 0
    s = np.asarray(o_scores[:v], dtype=np.float64)
    tau = np.min(s[o_idx[:o_cnt]])   # the oracle's k-th largest score
    floor = 1e-6 * np.max(np.abs(s))
    band = np.abs(s - tau) <= BAND_REL * max(abs(tau), floor)
    bad = [t for t in diff if not band[t]]
    assert not bad, f"slots {bad[:8]} differ outside the tie band (tau={tau})"
    return len(diff) // 2


def check_out(g_out, g_lse, r_out, r_lse):
    """g_out [..., 512] float, r_out same shape float64."""
    err = np.max(np.abs(g_out - r_out), axis=-1)
    ref = np.max(np.abs(r_out), axis=-1)
    rel = np.where(ref > 0, err / np.maximum(ref, 1e-30), err)
    assert np.all(rel <= OUT_RTOL), f"max normwise rel err {rel.max():.3e}"
    fin = np.isfinite(r_lse)
    assert np.array_equal(fin, np.isfinite(g_lse))
    if fin.any():
        d = np.abs(g_lse[fin] - r_lse[fin])
        assert np.all(d <= LSE_ATOL), f"max lse err {d.max():.3e}"
    return float(rel.max()) if rel.size else 0.0


def check_scores(g, r, vis):
    for i, v in enumerate(vis):
        gi, ri = g[i, :v], r[i, :v]
        if v:
            tol = SCORE_RTOL * np.max(np.abs(ri))
            assert np.all(np.abs(gi - ri) <= tol), f"row {i} score err {np.max(np.abs(gi - ri)):.3e} > {tol:.3e}"
        assert np.all(np.isneginf(g[i, v:])), f"row {i}: scores past row_vis must be -inf"
