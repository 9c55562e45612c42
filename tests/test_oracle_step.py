"""Pins for the oracle's indexer scores, top-k, split attention and LSE merge.

Every oracle function is checked against something other than itself:
brute-force scalar loops that decode through torch's fp8 cast, hand-worked
values (tests/golden/index_scores_by_hand.txt), torch's float64
scaled_dot_product_attention as an independent dense-attention routine, a
full Python sort for the top-k, closed forms (a single selected token, equal
keys) and exact invariants (positive homogeneity, page permutation, split
invariance of the merge).  The mutation tests at the end plant plausible
mistakes in a copy of the oracle and check that a pin catches each one.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(
        torch.float8_e4m3fn).to(torch.float64).numpy()


def _rand_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x30   # never a NaN code
    return c


def _tiny_index_problem(rng, hi=4, di=8, p=4, n_pages=9, kv=(13, 7), rows=3):
    k_code = _rand_codes(rng, (n_pages, p, di))
    k_scale = rng.uniform(0.1, 2.0, size=(n_pages, p))
    perm = rng.permutation(n_pages)
    max_pages = max(-(-v // p) for v in kv)
    pt = np.full((len(kv), max_pages), -1, dtype=np.int64)
    off = 0
    for b, v in enumerate(kv):
        n = -(-v // p)
        pt[b, :n] = perm[off:off + n]
        off += n
    row_req = rng.integers(0, len(kv), size=rows)
    row_vis = np.array([rng.integers(0, kv[r] + 1) for r in row_req])
    row_vis[0] = kv[row_req[0]]
    q_code = _rand_codes(rng, (rows, hi, di))
    q_scale = rng.uniform(0.1, 2.0, size=(rows, hi))
    w = rng.normal(0, 1, size=(rows, hi))
    return dict(q_code=q_code, q_scale=q_scale, head_w=w, k_code=k_code, k_scale=k_scale,
                page_table=pt, kv_lens=np.array(kv), row_req=row_req, row_vis=row_vis,
                page_size=p)


def _scores(d, score_len=None):
    score_len = score_len or int(max(d["kv_lens"]))
    return O.index_scores(d["q_code"], d["q_scale"], d["head_w"], d["k_code"], d["k_scale"],
                          d["page_table"], d["kv_lens"], d["row_req"], d["row_vis"],
                          d["page_size"], score_len)


# ----------------------------------------------------------------- scores

def _brute_scores(d, score_len):
    """Scalar loops: walk each request's pages in order, decode through torch."""
    p = d["page_size"]
    out = [[-math.inf] * score_len for _ in range(len(d["row_req"]))]
    qv = _torch_dec(d["q_code"])
    kvv = _torch_dec(d["k_code"])
    for r, (b, v) in enumerate(zip(d["row_req"], d["row_vis"])):
        t = 0
        for page in d["page_table"][b]:
            for off in range(p):
                if t >= v:
                    break
                acc = 0.0
                for h in range(qv.shape[1]):
                    dot = 0.0
                    for i in range(qv.shape[2]):
                        dot += (qv[r, h, i] * d["q_scale"][r, h]) * (kvv[page, off, i] * d["k_scale"][page, off])
                    acc += d["head_w"][r, h] * (dot if dot > 0 else 0.0)
                out[r][t] = acc
                t += 1
    return np.array(out)


def test_scores_match_brute_force_loops():
    rng = np.random.default_rng(10)
    d = _tiny_index_problem(rng)
    got = _scores(d, 13)
    ref = _brute_scores(d, 13)
    assert np.array_equal(np.isinf(got), np.isinf(ref))
    fin = np.isfinite(ref)
    np.testing.assert_allclose(got[fin], ref[fin], rtol=1e-12, atol=1e-12)


def test_scores_hand_worked_golden():
    """Two heads, 2-wide keys, three tokens on two pages of size 2; values
    worked out by hand in tests/golden/index_scores_by_hand.txt."""
    vals = {}
    with open(os.path.join(GOLDEN, "index_scores_by_hand.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                k, v = line.split("=")
                vals[k.strip()] = [float(x) for x in v.split()]
    one, two, half, neg1 = 0x38, 0x40, 0x30, 0xB8   # 1.0, 2.0, 0.5, -1.0
    q_code = np.array([[[one, two], [neg1, one]]], dtype=np.uint8)      # q0=(1,2) q1=(-1,1)
    q_scale = np.array([[1.0, 2.0]])                                    # q1 -> (-2, 2)
    w = np.array([[0.5, -1.0]])
    k_code = np.zeros((3, 2, 2), dtype=np.uint8)
    k_code[2, 0] = [one, one]      # slot 0 -> physical page 2
    k_code[2, 1] = [two, neg1]     # slot 1
    k_code[0, 0] = [half, two]     # slot 2 -> physical page 0
    k_scale = np.ones((3, 2))
    k_scale[0, 0] = 4.0
    pt = np.array([[2, 0]])
    got = O.index_scores(q_code, q_scale, w, k_code, k_scale, pt, np.array([3]),
                         np.array([0]), np.array([3]), 2, 4)
    np.testing.assert_array_equal(got[0, :3], vals["scores"])
    assert got[0, 3] == -np.inf


def test_scores_single_head_is_plain_dot_with_relu():
    rng = np.random.default_rng(11)
    d = _tiny_index_problem(rng, hi=1)
    d["head_w"] = np.ones_like(d["head_w"])
    got = _scores(d)
    p = d["page_size"]
    for r, (b, v) in enumerate(zip(d["row_req"], d["row_vis"])):
        t = np.arange(v)
        phys = d["page_table"][b][t // p] * p + t % p
        keys = _torch_dec(d["k_code"].reshape(-1, d["k_code"].shape[-1])[phys]) * d["k_scale"].reshape(-1)[phys][:, None]
        q = _torch_dec(d["q_code"][r, 0]) * d["q_scale"][r, 0]
        np.testing.assert_allclose(got[r, :v], np.maximum(keys @ q, 0), rtol=1e-13, atol=1e-13)


def test_scores_positive_homogeneity_and_weight_linearity():
    rng = np.random.default_rng(12)
    d = _tiny_index_problem(rng)
    base = _scores(d)
    d2 = dict(d, k_scale=d["k_scale"] * 3.0)
    np.testing.assert_allclose(_scores(d2), base * 3.0, rtol=1e-13)
    d3 = dict(d, head_w=-d["head_w"])
    fin = np.isfinite(base)
    np.testing.assert_allclose(_scores(d3)[fin], -base[fin], rtol=1e-13)
    # top-k is unchanged under a positive rescale of the keys
    for r, v in enumerate(d["row_vis"]):
        a, _ = O.topk_global(base[r], v, 5)
        b, _ = O.topk_global(_scores(d2)[r], v, 5)
        np.testing.assert_array_equal(a, b)


def test_page_permutation_leaves_scores_bitwise_identical():
    rng = np.random.default_rng(13)
    d = _tiny_index_problem(rng)
    base = _scores(d)
    perm = rng.permutation(d["k_code"].shape[0])   # new physical page of old page i is perm[i]
    inv = np.argsort(perm)
    d2 = dict(d, k_code=d["k_code"][inv], k_scale=d["k_scale"][inv],
              page_table=np.where(d["page_table"] >= 0, perm[np.maximum(d["page_table"], 0)], -1))
    assert np.array_equal(_scores(d2), base)


def test_scores_reject_bad_pages():
    rng = np.random.default_rng(14)
    d = _tiny_index_problem(rng)
    d["page_table"] = d["page_table"].copy()
    d["page_table"][0, 0] = d["k_code"].shape[0]
    d["row_req"] = np.zeros_like(d["row_req"])
    d["row_vis"] = np.full_like(d["row_vis"], d["kv_lens"][0])
    with pytest.raises(ValueError):
        _scores(d)


# ----------------------------------------------------------------- top-k

@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_full_python_sort_with_ties(seed):
    rng = np.random.default_rng(100 + seed)
    v = int(rng.integers(1, 500))
    k = int(rng.integers(1, 600))
    s = rng.choice([-1.5, 0.0, 0.25, 0.25, 3.0, 7.0], size=v) + (rng.random(v) < 0.3) * rng.normal(size=v)
    s = np.concatenate([s, np.full(7, -np.inf)])
    got, cnt = O.topk_global(s, v, k)
    order = sorted(range(v), key=lambda t: (-s[t], t))[: min(k, v)]
    assert cnt == min(k, v)
    np.testing.assert_array_equal(got[:cnt], sorted(order))
    assert np.all(got[cnt:] == -1)


@pytest.mark.parametrize("seed", range(8))
def test_split_then_merge_equals_global(seed):
    rng = np.random.default_rng(200 + seed)
    v = int(rng.integers(0, 3000))
    k = int(rng.integers(1, 800))
    n_splits = int(rng.integers(1, 24))
    s = np.round(rng.normal(size=v), 1)       # many exact ties
    a, ca = O.topk_global(s, v, k)
    b, cb = O.topk_split_merge(s, v, k, n_splits)
    assert ca == cb
    np.testing.assert_array_equal(a, b)


def test_topk_short_row_keeps_everything_and_empty_row():
    s = np.array([3.0, -1.0, 2.0])
    got, cnt = O.topk_global(s, 3, 8)
    assert cnt == 3 and list(got) == [0, 1, 2, -1, -1, -1, -1, -1]
    got, cnt = O.topk_split_merge(np.zeros(0), 0, 4, 3)
    assert cnt == 0 and list(got) == [-1] * 4


def test_split_ranges_partition():
    for n in (0, 1, 7, 600, 2375, 131072):
        for s in (1, 3, 16, 32):
            r = O.split_ranges(n, s)
            assert len(r) == s and r[0][0] == 0 and r[-1][1] == n
            assert all(a[1] == b[0] for a, b in zip(r, r[1:]))


# ----------------------------------------------------------------- attention

def _mla_problem(rng, h=3, n_tok=40, p=8, n_pages=7):
    kv_code = _rand_codes(rng, (n_pages, p, O.D_QK))
    kv_scale = rng.uniform(0.002, 0.01, size=(n_pages, p))
    q = torch.randn(1, h, O.D_QK, dtype=torch.float64, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30))))
    q_bits = q.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    pt = np.array([rng.permutation(n_pages)[: -(-n_tok // p)]])
    return q_bits, kv_code, kv_scale, pt


def test_dense_attention_matches_torch_sdpa():
    """A row shorter than k selects everything, so sparse = dense attention."""
    rng = np.random.default_rng(20)
    q_bits, kv_code, kv_scale, pt = _mla_problem(rng)
    n = 40
    idx = np.arange(n)[None]
    sm = 0.05
    po, pl = O.sparse_mla(q_bits, kv_code, kv_scale, pt, np.array([0]), idx, np.array([n]), sm, 1, 8)
    x = _torch_dec(kv_code.reshape(-1, O.D_QK)[pt[0][np.arange(n) // 8] * 8 + np.arange(n) % 8])
    x = torch.from_numpy(x * kv_scale.reshape(-1)[pt[0][np.arange(n) // 8] * 8 + np.arange(n) % 8][:, None])
    q = torch.from_numpy(O.bf16_decode(q_bits))[0]
    # SDPA over [heads, 1, D] queries against shared keys/values.
    qh = q[:, None, :]                               # [H, 1, 576]
    kh = x[None].expand(q.shape[0], n, O.D_QK)       # [H, n, 576]
    vh = x[None, :, :O.D_LATENT].expand(q.shape[0], n, O.D_LATENT).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(qh, kh.contiguous(), vh, scale=sm)[:, 0]
    np.testing.assert_allclose(po[0, :, 0], ref.numpy(), rtol=1e-11, atol=1e-13)
    lse_ref = torch.logsumexp(sm * (q @ x.T), dim=1).numpy()
    np.testing.assert_allclose(pl[0, :, 0], lse_ref, rtol=1e-13, atol=1e-13)


def test_single_token_and_equal_keys_closed_forms():
    rng = np.random.default_rng(21)
    x = rng.normal(size=(1, O.D_QK))
    q = rng.normal(size=(2, O.D_QK))
    o, lse = O.attend_split(q, x, 0.1)
    np.testing.assert_allclose(o, np.repeat(x[:, :O.D_LATENT], 2, 0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.1 * (q @ x[0]), rtol=1e-14)
    # identical keys: uniform weights -> mean of the values, lse = l + ln n
    xs = np.repeat(x, 5, 0)
    xs[:, :O.D_LATENT] += rng.normal(size=(5, O.D_LATENT)) * 0  # keys identical incl. values
    o, lse = O.attend_split(q, xs, 0.1)
    np.testing.assert_allclose(o, np.repeat(x[:, :O.D_LATENT], 2, 0), rtol=1e-14)
    np.testing.assert_allclose(lse, 0.1 * (q @ x[0]) + math.log(5), rtol=1e-14)
    # keys identical on the rope part only, latent differs: then keys differ, so
    # check the mean-of-values case with q orthogonal to everything (q = 0)
    xv = rng.normal(size=(6, O.D_QK))
    o, lse = O.attend_split(np.zeros((1, O.D_QK)), xv, 1.0)
    np.testing.assert_allclose(o[0], xv[:, :O.D_LATENT].mean(0), rtol=1e-13)
    np.testing.assert_allclose(lse, [math.log(6)], rtol=1e-14)


@pytest.mark.parametrize("n_splits", [1, 2, 3, 7, 64])
def test_split_attention_merges_to_unsplit(n_splits):
    rng = np.random.default_rng(22 + n_splits)
    q_bits, kv_code, kv_scale, pt = _mla_problem(rng, n_tok=40)
    sel = np.sort(rng.choice(40, size=23, replace=False))
    idx = np.full((1, 32), -1)
    idx[0, :23] = sel
    po1, pl1 = O.sparse_mla(q_bits, kv_code, kv_scale, pt, np.array([0]), idx, np.array([23]), 0.07, 1, 8)
    pos, pls = O.sparse_mla(q_bits, kv_code, kv_scale, pt, np.array([0]), idx, np.array([23]), 0.07, n_splits, 8)
    out, lse = O.lse_merge(pos, pls)
    np.testing.assert_allclose(out, po1[:, :, 0], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(lse, pl1[:, :, 0], rtol=1e-13)
    if n_splits > 23:
        assert np.all(np.isneginf(pls[0, :, 23:])) and np.all(pos[0, :, 23:] == 0)


def test_lse_merge_identities():
    rng = np.random.default_rng(23)
    o = rng.normal(size=(2, 3, 1, 8))
    l = rng.normal(size=(2, 3, 1))
    out, lse = O.lse_merge(o, l)
    np.testing.assert_array_equal(out, o[..., 0, :])
    np.testing.assert_array_equal(lse, l[..., 0])
    o2 = np.concatenate([o, np.zeros_like(o)], axis=2)
    l2 = np.concatenate([l, np.full_like(l, -np.inf)], axis=2)
    out2, lse2 = O.lse_merge(o2, l2)
    np.testing.assert_allclose(out2, out, rtol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=1e-15)
    out3, lse3 = O.lse_merge(np.zeros((1, 4, 8)), np.full((1, 4), -np.inf))
    assert np.all(out3 == 0) and np.all(np.isneginf(lse3))
    # weights: two splits with lse a, b merge with weights e^a/(e^a+e^b)
    oa, ob = rng.normal(size=8), rng.normal(size=8)
    out4, lse4 = O.lse_merge(np.stack([oa, ob])[None], np.array([[0.3, -1.2]]))
    wa = math.exp(0.3) / (math.exp(0.3) + math.exp(-1.2))
    np.testing.assert_allclose(out4[0], wa * oa + (1 - wa) * ob, rtol=1e-14)
    np.testing.assert_allclose(lse4[0], math.log(math.exp(0.3) + math.exp(-1.2)), rtol=1e-15)


# ----------------------------------------------------------------- whole step

def _tiny_step_inputs(seed=30, h=2, kv=(37, 90), top_k=16, p=8):
    rng = np.random.default_rng(seed)
    n_pages = sum(-(-v // p) for v in kv) + 2
    perm = rng.permutation(n_pages)
    pt = np.full((len(kv), max(-(-v // p) for v in kv)), -1)
    off = 0
    for b, v in enumerate(kv):
        n = -(-v // p)
        pt[b, :n] = perm[off:off + n]
        off += n
    qi = torch.randn(len(kv), 64, 128, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    qm = torch.randn(len(kv), h, O.D_QK, generator=torch.Generator().manual_seed(seed + 1)).to(torch.bfloat16)
    return {
        "q_idx": qi.view(torch.int16).numpy().view(np.uint16),
        "head_w": rng.normal(0, 0.125, size=(len(kv), 64)),
        "q_mla": qm.view(torch.int16).numpy().view(np.uint16),
        "k_code": _rand_codes(rng, (n_pages, p, 128)), "k_scale": rng.uniform(0.001, 0.01, (n_pages, p)),
        "kv_code": _rand_codes(rng, (n_pages, p, O.D_QK)), "kv_scale": rng.uniform(0.001, 0.01, (n_pages, p)),
        "page_table": pt, "kv_lens": np.array(kv), "row_req": np.arange(len(kv)),
        "row_vis": np.array(kv), "page_size": p, "top_k": top_k, "sm_scale": 1 / 24,
    }


def test_decode_step_split_counts_do_not_change_results():
    inp = _tiny_step_inputs()
    a = O.decode_step(inp, 1, 1)
    b = O.decode_step(inp, 5, 3)
    np.testing.assert_array_equal(a["topk_idx"], b["topk_idx"])
    np.testing.assert_allclose(a["out"], b["out"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(a["lse"], b["lse"], rtol=1e-13)
    # rows restricted to a subset give the same rows
    c = O.decode_step(inp, 1, 1, rows=[1])
    np.testing.assert_array_equal(c["topk_idx"][0], a["topk_idx"][1])
    np.testing.assert_allclose(c["out"][0], a["out"][1], rtol=1e-14)


# ----------------------------------------------------------------- mutation checks

def _mutant_index_scores(kind):
    def f(q_code, q_scale, head_w, k_code, k_scale, page_table, kv_lens, row_req, row_vis, page_size, score_len):
        if kind == "no_relu":
            orig = np.maximum
            try:
                O.np.maximum = lambda a, b: a
                return O.index_scores(q_code, q_scale, head_w, k_code, k_scale, page_table, kv_lens,
                                      row_req, row_vis, page_size, score_len)
            finally:
                O.np.maximum = orig
        if kind == "no_kscale":
            return O.index_scores(q_code, q_scale, head_w, k_code, np.ones_like(k_scale), page_table,
                                  kv_lens, row_req, row_vis, page_size, score_len)
        if kind == "wrong_page":
            return O.index_scores(q_code, q_scale, head_w, k_code, k_scale, np.where(page_table >= 0, (page_table + 1) % k_code.shape[0], -1),
                                  kv_lens, row_req, row_vis, page_size, score_len)
        raise ValueError(kind)
    return f


@pytest.mark.parametrize("kind", ["no_relu", "no_kscale", "wrong_page"])
def test_brute_force_pin_catches_planted_score_mistakes(kind):
    rng = np.random.default_rng(40)
    d = _tiny_index_problem(rng)
    bad = _mutant_index_scores(kind)(d["q_code"], d["q_scale"], d["head_w"], d["k_code"], d["k_scale"],
                                     d["page_table"], d["kv_lens"], d["row_req"], d["row_vis"],
                                     d["page_size"], 13)
    ref = _brute_scores(d, 13)
    fin = np.isfinite(ref)
    assert not np.allclose(bad[fin], ref[fin], rtol=1e-12, atol=1e-12)


def test_sdpa_pin_catches_transposed_or_unscaled_attention():
    rng = np.random.default_rng(41)
    x = rng.normal(size=(9, O.D_QK))
    q = rng.normal(size=(2, O.D_QK))
    qt, xt = torch.from_numpy(q), torch.from_numpy(x)
    ref = torch.nn.functional.scaled_dot_product_attention(
        qt[:, None], xt[None].expand(2, 9, O.D_QK).contiguous(),
        xt[None, :, :O.D_LATENT].expand(2, 9, O.D_LATENT).contiguous(), scale=0.2)[:, 0].numpy()
    good, _ = O.attend_split(q, x, 0.2)
    np.testing.assert_allclose(good, ref, rtol=1e-12, atol=1e-14)
    unscaled, _ = O.attend_split(q, x, 1.0)
    assert not np.allclose(unscaled, ref, rtol=1e-6)
    # values taken from the rope tail instead of the latent head
    logits = 0.2 * q @ x.T
    p = np.exp(logits - logits.max(1, keepdims=True))
    wrong = (p / p.sum(1, keepdims=True)) @ x[:, O.D_QK - O.D_LATENT:]
    assert not np.allclose(wrong, ref, rtol=1e-6)
