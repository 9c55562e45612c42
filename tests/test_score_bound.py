"""The indexer-score tolerance of the GPU parity tests, checked on the CPU.

The bound (tests/parity_util.py) must admit an honest fp32 evaluation of the
scores in another summation order, and must reject the mistakes it exists to
catch: a dropped head, a head weight of the wrong sign, a neighbouring key.
The mistakes are planted in copies of the oracle's scores, on the CPU.
"""
import numpy as np
import pytest

from oracle import dsa_oracle as O
from parity_util import check_scores, score_magnitudes
from sparse_attention_decode_dsa_amd import workload as W

# Short rows whose few scores cancel (mixed-sign head weights), beside long ones.
CFG = W.Config("bound", batch=5, kv_lens=(3, 4, 64, 300, 3000), rows_per_req=3, causal="mtp",
               page_size=1024, mla_heads=16, group_rows=3, index_splits=1, attn_splits=2)


@pytest.fixture(scope="module")
def case():
    n = W.as_numpy(W.make(CFG))
    qc, qs = O.quantize_q(n["q_idx"])
    vis = np.asarray(n["row_vis"])
    width = int(vis.max())
    ref = O.index_scores(qc, qs, n["head_w"], n["k_code"], n["k_scale"], n["page_table"],
                         n["kv_lens"], n["row_req"], n["row_vis"], n["page_size"], width)
    mags = score_magnitudes(n, qc, qs)
    return n, qc, qs, vis, ref, mags


def f32_scores(n, qc, qs, vis, width, head_w=None, shift=0):
    """Scores summed in float32, heads last-to-first, dims in reverse."""
    di = qc.shape[-1]
    kf = O.fp8_e4m3fn_decode(n["k_code"].reshape(-1, di)).astype(np.float32)
    ks = np.asarray(n["k_scale"], dtype=np.float32).reshape(-1)
    w_all = np.asarray(n["head_w"] if head_w is None else head_w, dtype=np.float32)
    out = np.full((len(vis), width), -np.inf)
    for r, v in enumerate(vis):
        if not v:
            continue
        phys = O.physical_rows(n["page_table"][n["row_req"][r]], int(v), n["page_size"],
                               n["k_code"].shape[0])
        phys = np.roll(phys, shift)
        q = O.fp8_e4m3fn_decode(qc[r]).astype(np.float32) * np.asarray(qs[r], np.float32)[:, None]
        acc = np.zeros(v, dtype=np.float32)
        for h in range(q.shape[0] - 1, -1, -1):
            dot = np.zeros(v, dtype=np.float32)
            for d in range(di - 1, -1, -1):
                dot = dot + kf[phys, d] * q[h, d]
            dot = dot * ks[phys]
            acc = acc + w_all[r, h] * np.maximum(dot, np.float32(0))
        out[r, :v] = acc
    return out


def n_terms(qc):
    return qc.shape[2] + qc.shape[1] + 2


def test_fp32_evaluation_within_bound(case):
    n, qc, qs, vis, ref, mags = case
    g = f32_scores(n, qc, qs, vis, ref.shape[1])
    check_scores(g, ref, vis, mags, n_terms(qc))
    # the fp32 error is real (the bound is not vacuous because nothing moved)
    fin = np.isfinite(ref)
    assert np.max(np.abs(g[fin] - ref[fin])) > 0


def test_dropped_head_rejected(case):
    n, qc, qs, vis, ref, mags = case
    bad = ref.copy()
    for r, v in enumerate(vis):
        if not v:
            continue
        phys = O.physical_rows(n["page_table"][n["row_req"][r]], int(v), n["page_size"],
                               n["k_code"].shape[0])
        k = O.fp8_e4m3fn_decode(n["k_code"].reshape(-1, qc.shape[-1])[phys]) \
            * np.asarray(n["k_scale"], np.float64).reshape(-1)[phys][:, None]
        q5 = O.fp8_e4m3fn_decode(qc[r, 5]) * qs[r, 5]
        bad[r, :v] -= float(n["head_w"][r, 5]) * np.maximum(k @ q5, 0.0)
    with pytest.raises(AssertionError):
        check_scores(bad, ref, vis, mags, n_terms(qc))


def test_wrong_weight_sign_rejected(case):
    n, qc, qs, vis, ref, mags = case
    w = np.asarray(n["head_w"], dtype=np.float64).copy()
    w[:, 3] = -w[:, 3]
    bad = f32_scores(n, qc, qs, vis, ref.shape[1], head_w=w)
    with pytest.raises(AssertionError):
        check_scores(bad, ref, vis, mags, n_terms(qc))


def test_neighbouring_key_rejected(case):
    n, qc, qs, vis, ref, mags = case
    bad = f32_scores(n, qc, qs, vis, ref.shape[1], shift=1)
    with pytest.raises(AssertionError):
        check_scores(bad, ref, vis, mags, n_terms(qc))
