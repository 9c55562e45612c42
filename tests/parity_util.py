"""Comparison rules shared by the GPU parity tests.

Tolerances (stated where the pages or the arithmetic fix them):
* fp8 codes, top-k counts and index sets: bit-exact, except that the two
  sets may differ only by slots whose oracle score lies within 1e-3 relative
  of the oracle's k-th score (the tie band; absolute floor 1e-6 * max|s|
  for a k-th score near zero); ties at bitwise-equal scores keep the lower
  slot on both sides.
* attention output (bf16): per (row, head) max|g - r| / max|r| <= 2e-2.
* lse: |g - r| <= 1e-3 absolute.
* scores (diagnostic): per slot |g - r| <= gamma_n * A_t, the textbook
  forward-error bound of a sum of n terms computed in fp32 (gamma_n =
  n u / (1 - n u), u = 2^-24).  The GPU forms each score as a sum of
  n = Di + Hi + 2 rounded operations (the Di-term head dot in fp32, the key
  scale, the head weight, the Hi-term head sum; the fp8 products and the
  power-of-two query scale are exact), and A_t = sum_h |w_h| sum_d |q_hd k_td|
  is the sum of the magnitudes it rounds; the matrix cores' own accumulation
  is taken to round no worse than one fp32 unit per addition.  The head
  weights carry both signs, so |s_t| can sit far below A_t (a row that sees
  two slots can have max|s| = A/250) and a bound relative to max|s| would
  not follow from the arithmetic.  A dropped head, a wrong sign or a wrong key moves a score by a
  term of order A_t / Hi, orders of magnitude above the bound.
"""
import numpy as np

from oracle import dsa_oracle as O

OUT_RTOL = 2e-2
LSE_ATOL = 1e-3
U32 = 2.0 ** -24
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


def score_magnitudes(sub_np, q_code, q_scale):
    """A_t = sum_h |w_h| sum_d |q_hd| |k_td| for every visible slot of every
    row (float64 [R, max vis], 0 past a row's span), from the oracle's
    decoded operands."""
    kc = sub_np["k_code"]
    di = kc.shape[-1]
    kf = np.abs(O.fp8_e4m3fn_decode(kc.reshape(-1, di)))
    ks = np.abs(np.asarray(sub_np["k_scale"], dtype=np.float64).reshape(-1))
    vis = np.asarray(sub_np["row_vis"])
    mags = np.zeros((len(vis), max(int(vis.max()) if len(vis) else 0, 1)))
    for r, v in enumerate(vis):
        if not v:
            continue
        phys = O.physical_rows(sub_np["page_table"][sub_np["row_req"][r]], int(v),
                               sub_np["page_size"], kc.shape[0])
        qa = np.abs(O.fp8_e4m3fn_decode(q_code[r])) * np.abs(q_scale[r])[:, None]
        wa = np.abs(np.asarray(sub_np["head_w"][r], dtype=np.float64))
        mags[r, :v] = wa @ (qa @ (kf[phys] * ks[phys][:, None]).T)
    return mags


def check_scores(g, r, vis, mags, n_terms):
    """Returns the largest |g - r| / (u A_t) seen, the error in fp32 units."""
    nu = n_terms * U32
    gamma = nu / (1.0 - nu)
    worst = 0.0
    for i, v in enumerate(vis):
        gi, ri = g[i, :v], r[i, :v]
        if v:
            err = np.abs(gi - ri)
            tol = gamma * mags[i, :v]
            bad = np.nonzero(err > tol)[0]
            assert bad.size == 0, (f"row {i} slot {bad[0]} score err {err[bad[0]]:.3e}"
                                   f" > {tol[bad[0]]:.3e}")
            pos = mags[i, :v] > 0
            if pos.any():
                worst = max(worst, float(np.max(err[pos] / (U32 * mags[i, :v][pos]))))
        assert np.all(np.isneginf(g[i, v:])), f"row {i}: scores past row_vis must be -inf"
    return worst
