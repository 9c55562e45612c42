"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Inputs are seeded and synthetic (sparse_attention_decode_dsa_amd.workload);
the oracle never sees anything the GPU computed.  Rules and tolerances are in
tests/parity_util.py.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from parity_util import (bf16_to_f64, check_out, check_scores, check_topk_row,
                         score_magnitudes)
from sparse_attention_decode_dsa_amd import dsa
from sparse_attention_decode_dsa_amd import workload as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run_step(inp, index_splits=None, attn_splits=None, group_rows=None, score_stride=None):
    step = dsa.DecodeStep(inp, index_splits, attn_splits, group_rows, score_stride)
    step.run()
    torch.cuda.synchronize()
    dsa.check_status(step.status)
    return step


def compare_step(inp, step, rows, max_swap_rows=None):
    """Oracle on `rows` of `inp` vs the GPU step; returns rows with tie swaps."""
    rows = list(rows)
    sub = W.subset(inp, rows)
    ref = O.decode_step(W.as_numpy(sub), step.index_splits, step.attn_splits)
    # The indexer quantizes its queries in the kernel with the helpers that
    # quantize_q runs on its own: the codes of this workload's queries.
    q_code, q_scale = dsa.quantize_q(inp.q_idx[rows].contiguous())
    np.testing.assert_array_equal(q_code.cpu().numpy(), ref["q_code"])
    np.testing.assert_array_equal(q_scale.cpu().double().numpy(), ref["q_scale"])
    vis = sub.row_vis.numpy()
    g_scores = step.scores[rows].cpu().double().numpy()
    r_scores = np.full_like(g_scores, -np.inf)
    r_scores[:, :ref["scores"].shape[1]] = ref["scores"]
    sub_np = W.as_numpy(sub)
    mags = score_magnitudes(sub_np, ref["q_code"], ref["q_scale"])
    hi, di = ref["q_code"].shape[1:]
    ulps = check_scores(g_scores, r_scores, vis, mags, di + hi + 2)
    say(f"  scores: max err {ulps:.2f} u*A (bound {di + hi + 2} u*A)")
    g_idx = step.topk_idx[rows].cpu().numpy()
    g_cnt = step.topk_count[rows].cpu().numpy()
    g_out = bf16_to_f64(step.out[rows])
    g_lse = step.out_lse[rows].cpu().double().numpy()
    swapped = []
    for i in range(len(rows)):
        if check_topk_row(g_idx[i], g_cnt[i], ref["topk_idx"][i], ref["topk_count"][i],
                          ref["scores"][i], vis[i], inp.top_k):
            swapped.append(i)
    # What each row's output is compared with: the oracle's own step, except
    # for rows whose selection differs from the oracle's inside the tie band.
    # Those attend other tokens, so the oracle attends the GPU's selection
    # (validated just above) for them; no row goes unchecked.
    ref["out_cmp"] = ref["out"].copy()
    ref["lse_cmp"] = ref["lse"].copy()
    if swapped:
        r_out, r_lse = oracle_on_selection(sub_np, swapped, g_idx, g_cnt, step.attn_splits)
        ref["out_cmp"][swapped] = r_out
        ref["lse_cmp"][swapped] = r_lse
    for i in range(len(rows)):
        check_out(g_out[i], g_lse[i], ref["out_cmp"][i], ref["lse_cmp"][i])
    swapped = [rows[i] for i in swapped]
    if max_swap_rows is not None:
        assert len(swapped) <= max_swap_rows, swapped
    return ref, sub, swapped


def oracle_on_selection(sub_np, which, g_idx, g_cnt, n_splits):
    """The oracle's attention and merge for rows `which` of the subset, over
    the given (GPU) selected lists instead of its own."""
    which = list(which)
    po, pl = O.sparse_mla(sub_np["q_mla"][which], sub_np["kv_code"], sub_np["kv_scale"],
                          sub_np["page_table"], np.asarray(sub_np["row_req"])[which],
                          np.asarray(g_idx)[which], np.asarray(g_cnt)[which], float(sub_np["sm_scale"]),
                          n_splits, int(sub_np["page_size"]))
    return O.lse_merge(po, pl)


def mla_on_oracle_selection(sub, ref, n_splits):
    """The GPU attention kernels fed the oracle's own top-k, vs the oracle."""
    g = W.to(sub, "cuda")
    idx = torch.from_numpy(ref["topk_idx"].astype(np.int32)).cuda()
    cnt = torch.from_numpy(ref["topk_count"].astype(np.int32)).cuda()
    st = dsa.new_status()
    if n_splits == 1:
        out, lse, _ = dsa.sparse_mla_decode(g.q_mla, g.kv_cache, g.page_table, g.row_req,
                                            g.row_vis, idx, cnt, 1, g.sm_scale, status=st)
    else:
        po, pl, _ = dsa.sparse_mla_decode(g.q_mla, g.kv_cache, g.page_table, g.row_req,
                                          g.row_vis, idx, cnt, n_splits, g.sm_scale, status=st)
        out, lse = dsa.lse_merge(po, pl)
    torch.cuda.synchronize()
    dsa.check_status(st)
    return check_out(bf16_to_f64(out), lse.cpu().double().numpy(), ref["out"], ref["lse"])


# ------------------------------------------------------------------ quantize

def test_quantize_q_bit_exact():
    g = torch.Generator().manual_seed(5)
    q = torch.randn(37, 64, 128, generator=g) * torch.exp(torch.randn(37, 64, 1, generator=g) * 4)
    q[0, 0] = 0.0                      # all-zero head
    q[0, 1] = 0.0
    q[0, 1, 3] = 448.0                 # amax exactly 448
    q[0, 2] = -0.0                     # negative zeros
    q[1, 5] *= 1e-30                   # tiny head
    q[2, 7] *= 1e30                    # huge head
    qb = q.to(torch.bfloat16)
    codes, scale = dsa.quantize_q(qb.cuda())
    torch.cuda.synchronize()
    rc, rs = O.quantize_q(qb.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(scale.cpu().double().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


# ------------------------------------------------------------------ top-k alone

def _synthetic_scores(rng, r, stride, vis, tie_frac=0.3):
    s = rng.normal(size=(r, stride)).astype(np.float32)
    ties = rng.random((r, stride)) < tie_frac
    s[ties] = rng.choice(np.array([-0.5, 0.0, 0.75, 1.5, 2.25], dtype=np.float32), size=ties.sum())
    for i, v in enumerate(vis):
        s[i, v:] = -np.inf
    return s


@pytest.mark.parametrize("k,n_splits", [(2048, 1), (2048, 4), (2048, 16), (7, 3), (1, 1), (100, 64)])
def test_topk_bit_exact_on_synthetic_scores(k, n_splits):
    rng = np.random.default_rng(1000 + k + n_splits)
    stride = 32768 if n_splits == 1 else 40000
    vis = [0, 1, k - 1 if k > 1 else 1, k, k + 1, 5000, stride // 2 + 3, stride]
    vis = [min(v, stride) for v in vis]
    s = _synthetic_scores(rng, len(vis), stride, vis)
    say(f"topk k={k} splits={n_splits} vis={vis}")
    idx, cnt, st = dsa.topk(torch.from_numpy(s).cuda(), torch.tensor(vis, dtype=torch.int32).cuda(),
                            k, n_splits)
    torch.cuda.synchronize()
    dsa.check_status(st)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for i, v in enumerate(vis):
        ri, rc = O.topk_split_merge(s[i].astype(np.float64), v, k, n_splits)
        gi, gc = O.topk_global(s[i].astype(np.float64), v, k)
        np.testing.assert_array_equal(ri, gi)   # the oracle's own split/merge invariant
        assert cnt[i] == rc, (i, v)
        np.testing.assert_array_equal(idx[i], ri)


@pytest.mark.parametrize("k,n_splits,stride", [(2048, 4, 65536), (6112, 4, 65536), (6113, 4, 65536),
                                               (2048, 8, 65536), (512, 5, 69632)])
def test_topk_more_splits_than_cus(k, n_splits, stride):
    """80 rows, so more split workgroups than the chip's 256 CUs: the launch
    takes the compact filter layout (two workgroups a CU; lists of up to 16
    keys a thread staged in two rounds) for k up to its limit, 6112, and the
    full layout above it.  Spans cover empty rows, k +- 1, split edges and
    the whole stride.  Bit-exact against the oracle's global top-k."""
    rng = np.random.default_rng(7 + k + n_splits)
    rows = 80
    spans = [0, 1, k - 1, k, k + 1, 5000, stride // 2 + 3, stride, stride - 1, 16383, 16384, 16385]
    vis = [min(max(v, 0), stride) for v in (spans * (rows // len(spans) + 1))[:rows]]
    s = _synthetic_scores(rng, rows, stride, vis)
    say(f"topk k={k} splits={n_splits} rows={rows} stride={stride}")
    idx, cnt, st = dsa.topk(torch.from_numpy(s).cuda(), torch.tensor(vis, dtype=torch.int32).cuda(),
                            k, n_splits)
    torch.cuda.synchronize()
    dsa.check_status(st)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for i, v in enumerate(vis):
        gi, gc = O.topk_global(s[i].astype(np.float64), v, k)
        assert cnt[i] == gc, (i, v)
        np.testing.assert_array_equal(idx[i], gi)


@pytest.mark.parametrize("n_splits", [1, 3])
def test_topk_with_infinities_matches_oracle(n_splits):
    """Rows with -inf inside the visible span (tokens on invalid pages, keys
    with bad scales), fewer finite scores than k, and +inf scores: the
    selection still follows (score desc, slot asc)."""
    rng = np.random.default_rng(31 + n_splits)
    r, stride, k = 6, 12000, 2048
    s = rng.normal(size=(r, stride)).astype(np.float32)
    vis = [12000, 12000, 9000, 12000, 5000, 3000]
    s[0, rng.random(stride) < 0.95] = -np.inf      # ~600 finite scores < k
    s[1, rng.random(stride) < 0.5] = -np.inf       # ~6000 finite scores > k
    s[2, :4000] = -np.inf
    s[3, [5, 77, 11000]] = np.inf                  # +inf at the top
    s[4, rng.random(stride) < 0.7] = -np.inf
    s[4, [10, 20]] = np.inf
    s[5] = -np.inf                                 # nothing finite at all
    for i, v in enumerate(vis):
        s[i, v:] = -np.inf
    idx, cnt, st = dsa.topk(torch.from_numpy(s).cuda(), torch.tensor(vis, dtype=torch.int32).cuda(), k,
                            n_splits)
    torch.cuda.synchronize()
    dsa.check_status(st)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for i, v in enumerate(vis):
        ri, rc = O.topk_global(s[i].astype(np.float64), v, k)
        assert cnt[i] == rc, (i, v)
        np.testing.assert_array_equal(idx[i], ri)


@pytest.mark.parametrize("n_splits", [2, 4])
def test_topk_cut_that_misses_falls_back_to_the_whole_row(n_splits):
    """Scores planted at the row sample's positions (floor(i * v / 512))
    make every split's cut too high, so fewer than k keys pass it; the merge
    then selects from the whole row, with the same result as the oracle."""
    rng = np.random.default_rng(60 + n_splits)
    r, stride, k = 3, 32768, 2048
    vis = [32768, 20000, 9000]
    s = rng.normal(size=(r, stride)).astype(np.float32)
    for i, v in enumerate(vis):
        pos = (np.arange(512, dtype=np.int64) * v) // 512
        s[i, pos] = 50.0 + rng.random(512).astype(np.float32)
        s[i, v:] = -np.inf
    idx, cnt, st = dsa.topk(torch.from_numpy(s).cuda(), torch.tensor(vis, dtype=torch.int32).cuda(), k, n_splits)
    torch.cuda.synchronize()
    dsa.check_status(st)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for i, v in enumerate(vis):
        ri, rc = O.topk_global(s[i].astype(np.float64), v, k)
        assert cnt[i] == rc
        np.testing.assert_array_equal(idx[i], ri)


@pytest.mark.parametrize("n_splits", [4, 16])
def test_topk_split_merge_over_score_shapes(n_splits):
    """Rows whose kept keys the merge's histogram must resolve: a kept range
    across zero (negative cut, positive k-th score), scores a few ulps apart,
    subnormal scores, scores spread over 60 decades, a range too wide for
    fp32 (cut near -2.5e38, top near +2.5e38), and a row whose k-th score is
    shared by a block of equal keys.  Bit-exact against the oracle."""
    rng = np.random.default_rng(90 + n_splits)
    r, stride, k = 6, 40000, 2048
    vis = [5000, 40000, 30000, 40000, 24000, 40000]
    s = rng.normal(size=(r, stride)).astype(np.float32)
    s[1] = np.float32(1.0) + np.float32(1e-7) * s[1]
    s[2] = s[2] * np.float32(1e-40)
    s[3] = np.sign(s[3]) * np.float32(10.0) ** rng.uniform(-30, 30, stride).astype(np.float32)
    s[4] = np.where(rng.random(stride) < 0.05, np.float32(2.5e38), np.float32(-2.5e38)) + s[4] * np.float32(1e37)
    s[5, rng.random(stride) < 0.2] = np.float32(2.0)   # the top ~2.3% ties at 2.0
    for i, v in enumerate(vis):
        s[i, v:] = -np.inf
    assert np.isfinite(s[:, :min(vis)]).all()
    say(f"topk shapes splits={n_splits}")
    idx, cnt, st = dsa.topk(torch.from_numpy(s).cuda(), torch.tensor(vis, dtype=torch.int32).cuda(), k, n_splits)
    torch.cuda.synchronize()
    dsa.check_status(st)
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for i, v in enumerate(vis):
        ri, rc = O.topk_global(s[i].astype(np.float64), v, k)
        assert cnt[i] == rc, i
        np.testing.assert_array_equal(idx[i], ri, err_msg=f"row {i}")


def test_topk_all_equal_scores_keep_lowest_slots():
    s = np.zeros((2, 9000), dtype=np.float32)
    vis = [9000, 4097]
    for n_splits in (1, 3):
        idx, cnt, st = dsa.topk(torch.from_numpy(s).cuda(), torch.tensor(vis, dtype=torch.int32).cuda(),
                                2048, n_splits)
        torch.cuda.synchronize()
        dsa.check_status(st)
        assert cnt.cpu().tolist() == [2048, 2048]
        np.testing.assert_array_equal(idx.cpu().numpy(), np.tile(np.arange(2048), (2, 1)))


# ------------------------------------------------------------------ LSE merge alone

@pytest.mark.parametrize("r,h,s", [(5, 32, 7), (20, 32, 3), (40, 32, 9), (33, 32, 2), (3, 16, 64),
                                   (64, 32, 4), (6, 32, 1)])
def test_lse_merge_synthetic(r, h, s):
    """Pair counts under 512, under 1024 and above, with the one-split and
    the batched kernels (a pair's columns go to 4, 2 or 1 wavefronts)."""
    rng = np.random.default_rng(7 + r + s)
    po = rng.normal(size=(r, h, s, 512)).astype(np.float32)
    pl = (rng.normal(size=(r, h, s)) * 5).astype(np.float32)
    e = min(2, s - 1)
    pl[0, :, e] = -np.inf                 # an empty split
    pl[1, 3, :] = -np.inf                 # an empty row
    po[0, :, e] = 0.0
    po[1, 3, :] = 0.0
    po_b = torch.from_numpy(po).to(torch.bfloat16)     # the partials' format; the oracle merges the same values
    out, lse = dsa.lse_merge(po_b.cuda(), torch.from_numpy(pl).cuda())
    torch.cuda.synchronize()
    ro, rl = O.lse_merge(po_b.double().numpy(), pl.astype(np.float64))
    check_out(bf16_to_f64(out), lse.cpu().double().numpy(), ro, rl)
    assert np.all(out[1, 3].float().cpu().numpy() == 0) and np.isneginf(lse[1, 3].item())


# ------------------------------------------------------------------ whole step, C0

@pytest.mark.parametrize("splits", [(4, 4), (1, 1), (2, 3)])
def test_c0_step_matches_oracle(splits):
    inp = W.to(W.make("c0"), "cuda")
    say(f"c0 step splits={splits}")
    step = run_step(inp, *splits)
    ref, sub, swapped = compare_step(inp, step, range(inp.n_rows), max_swap_rows=1)
    # request 0 is shorter than top-k: every slot selected, attention is dense
    assert step.topk_count[0].item() == 1500
    np.testing.assert_array_equal(step.topk_idx[0, :1500].cpu().numpy(), np.arange(1500))


@pytest.mark.parametrize("n_splits", [1, 4, 64])
def test_c0_attention_on_oracle_selection(n_splits):
    inp = W.make("c0")
    ref = O.decode_step(W.as_numpy(inp), 4, n_splits)
    say(f"c0 mla splits={n_splits}")
    mla_on_oracle_selection(inp, ref, n_splits)


def split_tile_paths(inp, idx, cnt, n_splits, slack=11.5, lazy=8.0):
    """The attention kernel's running-max rule replayed on the host (float32
    logits in base-2 units, per head): a tile whose largest logit exceeds the
    running max by more than `slack` takes the exact path, one that exceeds
    it by more than `lazy` moves it on the fast path.  Returns (exact paths
    after a split's first tile, fast-path moves)."""
    code = W.kv_code_view(inp.kv_cache).contiguous().view(torch.float8_e4m3fn).float()
    sc = W.kv_scale_view(inp.kv_cache)
    q = inp.q_mla.float()
    p = inp.page_size
    chunk = -(-inp.top_k // n_splits)
    exact = moves = 0
    for r in range(inp.n_rows):
        b = int(inp.row_req[r])
        sel = torch.from_numpy(np.asarray(idx[r, :cnt[r]], dtype=np.int64))
        pages, offs = inp.page_table[b, sel // p].long(), sel % p
        lg = (q[r] @ (code[pages, offs] * sc[pages, offs][:, None]).T) * (inp.sm_scale / np.log(2.0))
        for sp in range(n_splits):
            lo, hi = sp * chunk, min((sp + 1) * chunk, int(cnt[r]))
            m = torch.full((lg.shape[0],), -float("inf"))
            for t0 in range(lo, hi, 64):
                tm = lg[:, t0:min(t0 + 64, hi)].max(dim=1).values
                big = bool((tm > m + slack).any())
                moved = torch.where(tm > m + lazy, tm, m)
                if big and t0 > lo:
                    exact += 1
                elif not big and bool((moved != m).any()):
                    moves += 1
                m = moved
    return exact, moves


@pytest.mark.parametrize("n_splits,heads,factor", [(1, 16, 8), (4, 16, 8), (4, 32, 8), (3, 32, 8),
                                                   (1, 16, 3), (4, 32, 3)])
def test_attention_logit_jumps_mid_split(n_splits, heads, factor):
    """Selected rows whose MLA scales are raised `factor`-fold in tiles 2
    and 5 of every split, so their positive logits rise above the running
    maximum of the tiles before them and their negative ones fall below.
    8-fold: by more than the attention kernel's exact-path threshold, a
    path the synthetic workloads otherwise take only at a split's first
    tile.  3-fold: by less, but enough to move the running max on the fast
    path.  The GPU attention on the oracle's selection against the oracle."""
    base = W.make("c0")
    inp = W.make(dataclasses.replace(base.cfg, mla_heads=heads))
    ref = O.decode_step(W.as_numpy(inp), 4, n_splits)
    idx, cnt = ref["topk_idx"], ref["topk_count"]
    kv = inp.kv_cache.clone()
    kvs = W.kv_scale_view(kv)
    p = inp.page_size
    chunk = -(-inp.top_k // n_splits)
    for r in range(inp.n_rows):
        b = int(inp.row_req[r])
        for sp in range(n_splits):
            lo, hi = sp * chunk, min((sp + 1) * chunk, int(cnt[r]))
            for tile in (2, 5):
                for j in range(lo + 64 * tile, min(lo + 64 * tile + 8, hi)):
                    t = int(idx[r, j])
                    kvs[int(inp.page_table[b, t // p]), t % p] *= factor
    jumped = dataclasses.replace(inp, kv_cache=kv)
    exact, moves = split_tile_paths(jumped, idx, cnt, n_splits)
    say(f"logit jumps x{factor}: splits={n_splits} heads={heads}: {exact} exact paths mid-split, "
        f"{moves} fast-path moves")
    assert (exact if factor == 8 else moves) >= 4
    ref2 = O.decode_step(W.as_numpy(jumped), 4, n_splits)
    np.testing.assert_array_equal(ref2["topk_idx"], idx)   # the index keys did not change
    mla_on_oracle_selection(jumped, ref2, n_splits)


# ------------------------------------------------------------------ bulk decode, sampled rows

@pytest.mark.parametrize("name", ["c1", "c1_l32k"])
def test_bulk_decode_sampled_rows(name):
    inp = W.make(name, device="cuda")
    say(f"{name}: B={inp.n_rows} pages={inp.n_pages} splits=({inp.cfg.index_splits},{inp.cfg.attn_splits})")
    step = run_step(inp)
    vis = inp.row_vis.cpu().numpy()
    rows = sorted({int(np.argmin(vis)), int(np.argmax(vis)), 0, 17, 63})
    ref, sub, swapped = compare_step(inp, step, rows, max_swap_rows=2)
    say(f"{name}: rows {rows} swapped {swapped}")
    mla_on_oracle_selection(sub, ref, inp.cfg.attn_splits)


def test_bulk_decode_step_with_physical_rows_sampled_rows():
    """The step with the top-k emitting physical rows and the attention
    gathering them directly, on sampled rows against the oracle."""
    inp = W.make("c1_l32k", device="cuda")
    step = dsa.DecodeStep(inp, phys_rows=True)
    assert step.phys_rows
    step.run()
    torch.cuda.synchronize()
    dsa.check_status(step.status)
    ref, sub, swapped = compare_step(inp, step, [0, 17, 40, 63], max_swap_rows=2)
    say(f"c1_l32k rows: swapped {swapped}")


def test_bulk_decode_step_with_index_topk_sampled_rows():
    """The step with scores and top-k from one dsa_index_topk call (the
    indexer keeps candidates, a merge selects), on sampled rows against the
    oracle."""
    inp = W.make("c1_l32k", device="cuda")
    step = dsa.DecodeStep(inp, index_topk=True)
    assert step.index_topk
    step.run()
    torch.cuda.synchronize()
    dsa.check_status(step.status)
    ref, sub, swapped = compare_step(inp, step, [0, 17, 40, 63], max_swap_rows=2)
    say(f"c1_l32k fused: swapped {swapped}")


# ------------------------------------------------------------------ edge rows, page sizes, strides

EDGE_DECODE = W.Config("edge_decode", batch=10, kv_lens=(0, 1, 63, 64, 65, 2047, 2048, 2049, 5000, 777),
                       page_size=16, mla_heads=16)


@pytest.mark.parametrize("page_size,top_k,splits,stride_pad,heads", [
    (16, 2048, (1, 1), 0, 16),      # empty, one-token and page-edge rows; k above most rows
    (1024, 2048, (3, 5), 3, 32),    # one page holds most rows; odd stride (unaligned rows)
    (64, 100, (2, 64), 1, 16),      # small k, more attention splits than entries
    (16, 1, (1, 2), 0, 32),         # k = 1
])
def test_edge_rows_match_oracle(page_size, top_k, splits, stride_pad, heads):
    cfg = dataclasses.replace(EDGE_DECODE, page_size=page_size, top_k=top_k, mla_heads=heads,
                              index_splits=splits[0], attn_splits=splits[1])
    inp = W.to(W.make(cfg), "cuda")
    stride = (int(inp.row_vis.max()) + 63) // 64 * 64 + stride_pad
    say(f"edge decode P={page_size} k={top_k} splits={splits} stride={stride} H={heads}")
    step = run_step(inp, splits[0], splits[1], None, stride)
    compare_step(inp, step, range(inp.n_rows), max_swap_rows=2)
    assert step.topk_count[0].item() == 0 and step.topk_count[1].item() == 1
    assert torch.all(step.out[0] == 0) and torch.all(torch.isneginf(step.out_lse[0]))


@pytest.mark.parametrize("cfg", [
    # Two rows per request scored as one group: a dead group (kv_len 0), short
    # and page-straddling spans on the balanced schedule.
    W.Config("edge_g2", batch=4, kv_lens=(0, 130, 2100, 70), rows_per_req=2, page_size=64,
             mla_heads=16, group_rows=2, index_splits=1, attn_splits=3),
    # MTP-style causal groups of three, spans down to one token, 1024-token pages.
    W.Config("edge_mtp", batch=5, kv_lens=(3, 4, 64, 300, 3000), rows_per_req=3, causal="mtp",
             page_size=1024, mla_heads=32, group_rows=3, index_splits=1, attn_splits=2),
    # The remaining group sizes of the balanced schedule, MTP-causal, spans
    # from one token to past a 2048-token page boundary.
    W.Config("edge_g4", batch=3, kv_lens=(4, 700, 2500), rows_per_req=4, causal="mtp",
             page_size=64, mla_heads=16, group_rows=4, index_splits=1, attn_splits=2),
    W.Config("edge_g5", batch=3, kv_lens=(5, 1000, 2100), rows_per_req=5, causal="mtp",
             page_size=256, mla_heads=16, group_rows=5, index_splits=2, attn_splits=1),
    W.Config("edge_g7", batch=2, kv_lens=(7, 3000), rows_per_req=7, causal="mtp",
             page_size=16, mla_heads=32, group_rows=7, index_splits=1, attn_splits=3),
], ids=["groups_of_2", "mtp_groups_of_3", "mtp_groups_of_4", "mtp_groups_of_5", "mtp_groups_of_7"])
def test_edge_groups_match_oracle(cfg):
    inp = W.to(W.make(cfg), "cuda")
    say(f"{cfg.name}: rows={inp.n_rows} vis={inp.row_vis.tolist()}")
    step = run_step(inp)
    compare_step(inp, step, range(inp.n_rows), max_swap_rows=2)


@pytest.mark.parametrize("group_rows,groups", [
    (2, 1030),   # more groups than one balanced launch holds: the chunked launch of row groups
    (2, 1024),   # exactly as many as it holds: the largest partition scan
    (6, 513),    # the same past the limit for groups of six
], ids=["g2_chunked", "g2_balanced_full", "g6_chunked"])
def test_many_row_groups_sampled_rows(group_rows, groups):
    cfg = W.Config(f"many_g{group_rows}", batch=groups, kv_range=(group_rows, 700), rows_per_req=group_rows,
                   causal="mtp", page_size=64, mla_heads=16, group_rows=group_rows, index_splits=1,
                   attn_splits=1)
    inp = W.to(W.make(cfg), "cuda")
    vis = inp.row_vis.cpu().numpy()
    say(f"{cfg.name}: groups={groups} rows={inp.n_rows} vis {int(vis.min())}..{int(vis.max())}")
    step = run_step(inp)
    n = inp.n_rows
    rows = sorted({0, 1, group_rows, n // 2, n // 2 + 1, n - group_rows, n - 1, int(np.argmax(vis))})
    compare_step(inp, step, rows, max_swap_rows=2)


# ------------------------------------------------------------------ long context, MTP verify, prefill

def test_long_context_planted_sampled_rows():
    """8 requests up to 131072 tokens, 16 index splits, 32 attention splits,
    4 planted slots per request (both caches' scales x8).  Sampled rows cover
    every request length (9600, 38000, 77000, 131072)."""
    inp = W.make("c2", device="cuda")
    say(f"c2: B={inp.n_rows} vis={inp.row_vis.tolist()}")
    step = run_step(inp)
    idx = step.topk_idx.cpu().numpy()
    hit = sum(len(set(inp.planted_slots[b].tolist()) & set(idx[b].tolist())) for b in range(inp.n_rows))
    say(f"c2: {hit} of {inp.planted_slots.numel()} planted slots selected")
    rows = [0, 1, 3, 5, 6]
    ref, sub, swapped = compare_step(inp, step, rows, max_swap_rows=2)
    say(f"c2: swapped {swapped}")
    # A planted slot whose oracle score lies clearly above the row's k-th
    # score (outside the tie band) is in the oracle's top-k, so the GPU must
    # have selected it.
    must = 0
    for i, r in enumerate(rows):
        s = ref["scores"][i]
        tau = np.min(s[ref["topk_idx"][i][:ref["topk_count"][i]]])
        b = int(inp.row_req[r])
        for t in inp.planted_slots[b].tolist():
            if s[t] > tau + 1e-3 * abs(tau):
                must += 1
                assert t in set(idx[r].tolist()), f"row {r}: planted slot {t} (score {s[t]:.4g} > {tau:.4g})"
    say(f"c2: {must} planted slots above the k-th score, all selected")
    assert must > 0
    mla_on_oracle_selection(sub, ref, inp.cfg.attn_splits)


def test_mtp_verify_grouped_rows():
    """32 requests x 6 causal rows scored as groups of 6 against one key
    stream; sampled requests 0 and 31 (12 rows)."""
    inp = W.make("c3", device="cuda")
    say(f"c3: R={inp.n_rows} group_rows={inp.cfg.group_rows}")
    step = run_step(inp)
    rows = list(range(0, 6)) + list(range(inp.n_rows - 6, inp.n_rows))
    ref, sub, swapped = compare_step(inp, step, rows, max_swap_rows=2)
    say(f"c3: swapped {swapped}")
    mla_on_oracle_selection(sub, ref, inp.cfg.attn_splits)


def test_long_prefix_prefill_sampled_rows():
    """4096 prefill rows after a 65536-token prefix, groups of 8 rows,
    5 index splits, one attention split; sampled rows across the range."""
    inp = W.make("c4", device="cuda")
    say(f"c4: R={inp.n_rows} vis {int(inp.row_vis.min())}..{int(inp.row_vis.max())}")
    step = run_step(inp)
    cnt = step.topk_count.cpu().numpy()
    assert np.all(cnt == np.minimum(inp.top_k, inp.row_vis.cpu().numpy()))
    rows = [0, 1, 7, 8, 2047, 4095]
    ref, sub, swapped = compare_step(inp, step, rows, max_swap_rows=1)
    say(f"c4: swapped {swapped}")
    mla_on_oracle_selection(sub, ref, inp.cfg.attn_splits)


# ------------------------------------------------------------------ properties

@pytest.mark.parametrize("name", ["c1_l32k", "c1", "c2"])
def test_whole_row_key_loads_give_the_same_scores(name):
    """The decode indexer's whole-row, non-temporal key loads (the caller's
    flag) score exactly as its half-row loads, on uniform and on ragged rows
    (the flag only promises long rows; it never changes a score), with every
    row of the workload in one launch.  A step asked for it takes it only
    when every row spans at least 3/4 of the score stride; by default never."""
    inp = W.to(W.make(name), "cuda")
    assert not dsa.DecodeStep(inp).whole_rows
    step = dsa.DecodeStep(inp, whole_rows=True)
    assert step.whole_rows == (name == "c1_l32k")
    say(f"whole-row loads {name}")
    args = (inp.q_idx, inp.head_w, inp.k_code, inp.k_scale, inp.page_table, inp.kv_lens, inp.row_req,
            inp.row_vis)
    half, st0 = dsa.index_scores(*args, score_stride=step.score_stride)
    whole, st1 = dsa.index_scores(*args, score_stride=step.score_stride, whole_rows=True)
    torch.cuda.synchronize()
    dsa.check_status(st0)
    dsa.check_status(st1)
    assert torch.equal(half.view(torch.int32), whole.view(torch.int32))


def test_page_permutation_and_run_to_run_determinism():
    inp = W.to(W.make("c0"), "cuda")
    a = run_step(inp)
    out_a = a.out.clone()
    b = run_step(inp)
    assert torch.equal(out_a, b.out) and torch.equal(a.topk_idx, b.topk_idx)
    # permute the physical pages and remap the block table
    n = inp.n_pages
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(3)).cuda()
    inv = torch.argsort(perm)
    pt = inp.page_table.long()
    new_pt = torch.where(pt >= 0, perm[pt.clamp(min=0)], pt).to(torch.int32)
    from dataclasses import replace
    p = replace(inp, k_code=inp.k_code[inv], k_scale=inp.k_scale[inv], kv_cache=inp.kv_cache[inv],
                page_table=new_pt.contiguous())
    c = run_step(p)
    assert torch.equal(out_a, c.out) and torch.equal(a.topk_idx, c.topk_idx)
    assert torch.equal(a.scores, c.scores)


def test_bad_page_id_is_reported_not_read():
    inp = W.to(W.make("c0"), "cuda")
    pt = inp.page_table.clone()
    pt[1, 10] = inp.n_pages + 5           # inside request 1's span
    from dataclasses import replace
    bad = replace(inp, page_table=pt)
    step = dsa.DecodeStep(bad)
    step.run()
    torch.cuda.synchronize()
    with pytest.raises(dsa.DsaError, match="PAGE_OOB"):
        dsa.check_status(step.status)


def test_undersized_row_inputs_are_rejected_before_launch():
    """A row-indexed input or a caller's output with fewer rows than the call
    is told is a DsaError from the binding: nothing is launched on it."""
    inp = W.to(W.make("c0"), "cuda")
    step = run_step(inp, attn_splits=2)
    r = inp.q_mla.shape[0]
    args = (inp.q_mla, inp.kv_cache, inp.page_table, inp.row_req, inp.row_vis)
    short = {"topk_idx": (step.topk_idx[:r - 1].contiguous(), step.topk_count),
             "topk_count": (step.topk_idx, step.topk_count[:r - 1].contiguous())}
    for name, (idx, cnt) in short.items():
        with pytest.raises(dsa.DsaError, match=name):
            dsa.sparse_mla_decode(*args, idx, cnt, 2, inp.sm_scale)
    with pytest.raises(dsa.DsaError, match="row_vis"):
        dsa.sparse_mla_decode(*args[:4], inp.row_vis[:r - 1].contiguous(), step.topk_idx, step.topk_count,
                              2, inp.sm_scale)
    with pytest.raises(dsa.DsaError, match="part_o"):
        dsa.sparse_mla_decode(*args, step.topk_idx, step.topk_count, 2, inp.sm_scale,
                              part_o=torch.empty((r - 1, inp.q_mla.shape[1], 2, 512), dtype=torch.bfloat16,
                                                 device="cuda"))
    with pytest.raises(dsa.DsaError, match="row_list"):
        dsa.sparse_mla_decode_shared(*args, torch.zeros(r - 1, dtype=torch.int32, device="cuda"),
                                     step.topk_idx, step.topk_count, 2, inp.sm_scale)
    with pytest.raises(dsa.DsaError, match="row_vis"):
        dsa.topk(step.scores, inp.row_vis[:r - 1].contiguous(), inp.top_k)
    with pytest.raises(dsa.DsaError, match="topk_idx"):
        dsa.topk(step.scores, inp.row_vis, inp.top_k,
                 topk_idx=torch.empty((r, inp.top_k - 1), dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg", ["c0", "c2"])
def test_graph_replays_match_eager(cfg):
    """The step captured in a HIP graph (as bench.py times it) and replayed
    several times, with eager work and synchronisations in between, gives the
    eager result bit for bit on every replay."""
    inp = W.to(W.make(cfg), "cuda")
    step = run_step(inp)
    want = (step.scores.clone(), step.topk_idx.clone(), step.topk_count.clone(), step.out.clone(),
            step.out_lse.clone())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step.run()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step.run()
    for rep in range(4):
        step.scores.fill_(0.5)          # eager work between replays
        step.out.zero_()
        step.topk_idx.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        dsa.check_status(step.status)
        got = (step.scores, step.topk_idx, step.topk_count, step.out, step.out_lse)
        for a, b in zip(got, want):
            assert torch.equal(a.view(torch.uint8) if a.dtype != torch.int32 else a,
                               b.view(torch.uint8) if b.dtype != torch.int32 else b), f"replay {rep}"


# ------------------------------------------------------------------ error paths

def test_nan_score_is_reported_and_selection_stays_valid():
    rng = np.random.default_rng(21)
    r, stride, k = 3, 4096, 100
    s = torch.from_numpy(rng.standard_normal((r, stride)).astype(np.float32))
    s[1, 17] = float("nan")
    s[1, 3000] = float("nan")
    vis = torch.tensor([4096, 3100, 50], dtype=torch.int32)
    st = dsa.new_status()
    idx, cnt, _ = dsa.topk(s.cuda(), vis.cuda(), k, 1, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & dsa.DEV_NAN
    idx, cnt = idx.cpu().numpy(), cnt.cpu().numpy()
    for i in range(r):
        c = min(k, int(vis[i]))
        assert cnt[i] == c
        sel = idx[i, :c]
        assert np.all(np.diff(sel) > 0) and sel[0] >= 0 and sel[-1] < vis[i] and np.all(idx[i, c:] == -1)
    # rows without a NaN select exactly as the oracle does
    for i in (0, 2):
        o_idx, o_cnt = O.topk_global(s[i].double().numpy(), int(vis[i]), k)
        np.testing.assert_array_equal(idx[i, :o_cnt], o_idx[:o_cnt])


def test_invalid_selected_entries_are_left_out_and_reported():
    """Entries past the row's span or negative are skipped: the row attends the
    remaining ones, which the oracle computes from the filtered list."""
    inp = W.to(W.make("c0"), "cuda")
    step = run_step(inp, 1, 4)
    idx = step.topk_idx.clone()
    cnt = step.topk_count.clone()
    vis = inp.row_vis.cpu().numpy()
    bad = idx.cpu().numpy().copy()
    bad[0, 3] = vis[0] + 5          # past the span
    bad[1, 0] = -2                  # negative
    bad[1, 100] = vis[1]            # one past the end
    st = dsa.new_status()
    po, pl, _ = dsa.sparse_mla_decode(inp.q_mla, inp.kv_cache, inp.page_table, inp.row_req, inp.row_vis,
                                      torch.from_numpy(bad).cuda(), cnt, 4, inp.sm_scale, status=st)
    out, lse = dsa.lse_merge(po, pl)
    torch.cuda.synchronize()
    assert int(st.item()) & dsa.DEV_TOPK_OOB
    sub = W.subset(inp, range(inp.n_rows))
    n = W.as_numpy(sub)
    c = cnt.cpu().numpy()
    keep = [np.array([t for t in bad[i, :c[i]] if 0 <= t < vis[i]]) for i in range(inp.n_rows)]
    k = bad.shape[1]
    f_idx = np.full((inp.n_rows, k), -1, dtype=np.int64)
    f_cnt = np.array([len(x) for x in keep])
    for i, x in enumerate(keep):
        f_idx[i, :len(x)] = x
    kv_code = n["kv_code"]
    r_po, r_pl = O.sparse_mla(n["q_mla"], kv_code, n["kv_scale"], n["page_table"], n["row_req"], f_idx, f_cnt,
                              inp.sm_scale, 1, inp.page_size)
    r_out, r_lse = O.lse_merge(r_po, r_pl)
    check_out(bf16_to_f64(out), lse.cpu().double().numpy(), r_out, r_lse)


def test_inconsistent_row_geometry_gives_an_empty_row():
    """Each call writes a row whose geometry it finds inconsistent as empty,
    reports it, and leaves the other rows as a clean call writes them."""
    from dataclasses import replace
    inp = W.to(W.make("c0"), "cuda")
    good = run_step(inp, 1, 1)
    args = (inp.q_idx, inp.head_w, inp.k_code, inp.k_scale, inp.page_table, inp.kv_lens)
    # indexer: a span past the request's kv_len
    vis = inp.row_vis.clone()
    vis[0] = inp.kv_lens[int(inp.row_req[0])] + 1
    st = dsa.new_status()
    sc, _ = dsa.index_scores(*args, inp.row_req, vis, score_stride=good.score_stride, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & dsa.DEV_ROW_RANGE
    assert torch.all(torch.isneginf(sc[0])) and torch.equal(sc[1], good.scores[1])
    # top-k: a span past the score stride
    vis = inp.row_vis.clone()
    vis[0] = good.score_stride + 1
    st = dsa.new_status()
    idx, cnt, _ = dsa.topk(good.scores, vis, inp.top_k, 1, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & dsa.DEV_ROW_RANGE
    assert int(cnt[0]) == 0 and torch.all(idx[0] == -1)
    assert torch.equal(idx[1], good.topk_idx[1]) and int(cnt[1]) == int(good.topk_count[1])
    # attention: a request out of range
    rr = inp.row_req.clone()
    rr[0] = inp.page_table.shape[0]
    st = dsa.new_status()
    out, lse, _ = dsa.sparse_mla_decode(inp.q_mla, inp.kv_cache, inp.page_table, rr, inp.row_vis,
                                        good.topk_idx, good.topk_count, 1, inp.sm_scale, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & dsa.DEV_ROW_RANGE
    assert torch.all(out[0] == 0) and torch.all(torch.isneginf(lse[0]))
    assert torch.equal(out[1], good.out[1])


def test_rows_of_different_requests_in_one_group_are_reported():
    cfg = W.Config("grp_err", batch=2, kv_lens=(300, 500), rows_per_req=2, page_size=64, mla_heads=16,
                   group_rows=2, index_splits=1, attn_splits=1)
    inp = W.to(W.make(cfg), "cuda")
    rr = inp.row_req.clone()
    rr[1] = 1 - rr[1]          # the first group now mixes the two requests
    from dataclasses import replace
    st = dsa.new_status()
    sc, _ = dsa.index_scores(inp.q_idx, inp.head_w, inp.k_code, inp.k_scale, inp.page_table, inp.kv_lens,
                             rr, inp.row_vis, group_rows=2, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & dsa.DEV_GROUP
    assert torch.all(torch.isneginf(sc[1]))     # the offending row is empty


def test_bad_scales_are_reported_and_left_out():
    """Scales that are not positive finite numbers.  In the index-key cache
    (negative, zero, NaN): the indexer sets DSA_DEV_SCALE, scores those tokens
    -inf and writes every other score as a clean call does.  In the MLA cache
    (negative, NaN, +inf) at selected slots: the attention sets the bit and
    leaves those tokens out; the row attends the others, which the oracle
    computes from the filtered list."""
    from dataclasses import replace
    inp = W.to(W.make("c0"), "cuda")
    good = run_step(inp, 1, 4)
    pt = inp.page_table.cpu()
    p = inp.page_size

    def at(b, t):
        return int(pt[b, t // p]), t % p

    ks = inp.k_scale.clone()
    planted = {(1, 100): -0.5, (1, 4000): float("nan"), (1, 2000): 0.0, (0, 7): -1e-30}
    for (b, t), val in planted.items():
        ks[at(b, t)] = val
    st = dsa.new_status()
    sc, _ = dsa.index_scores(inp.q_idx, inp.head_w, inp.k_code, ks, inp.page_table, inp.kv_lens,
                             inp.row_req, inp.row_vis, score_stride=good.score_stride, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == dsa.DEV_SCALE
    want = good.scores.clone()
    for (b, t) in planted:
        want[b, t] = -float("inf")
    assert torch.equal(sc, want)

    # MLA rows: bad scales at selected slots of both rows.
    idx = good.topk_idx.cpu().numpy()
    cnt = good.topk_count.cpu().numpy()
    kv = inp.kv_cache.clone()
    kvs = W.kv_scale_view(kv)
    bad_slots = {0: [int(idx[0, 3]), int(idx[0, 1499])], 1: [int(idx[1, 0]), int(idx[1, 1000])]}
    vals = [-2.0, float("nan"), float("inf"), -0.0]
    for j, (b, t) in enumerate((b, t) for b, ts in bad_slots.items() for t in ts):
        kvs[at(b, t)] = vals[j]
    st = dsa.new_status()
    po, pl, _ = dsa.sparse_mla_decode(inp.q_mla, kv, inp.page_table, inp.row_req, inp.row_vis,
                                      good.topk_idx, good.topk_count, 4, inp.sm_scale, status=st)
    out, lse = dsa.lse_merge(po, pl)
    torch.cuda.synchronize()
    assert int(st.item()) == dsa.DEV_SCALE
    n = W.as_numpy(W.subset(inp, range(inp.n_rows)))
    k = idx.shape[1]
    f_idx = np.full((inp.n_rows, k), -1, dtype=np.int64)
    f_cnt = np.zeros(inp.n_rows, dtype=np.int64)
    for i in range(inp.n_rows):
        keep = [t for t in idx[i, :cnt[i]] if t not in bad_slots[i]]
        f_idx[i, :len(keep)] = keep
        f_cnt[i] = len(keep)
    r_po, r_pl = O.sparse_mla(n["q_mla"], n["kv_code"], n["kv_scale"], n["page_table"], n["row_req"], f_idx,
                              f_cnt, inp.sm_scale, 1, inp.page_size)
    r_out, r_lse = O.lse_merge(r_po, r_pl)
    check_out(bf16_to_f64(out), lse.cpu().double().numpy(), r_out, r_lse)


# ------------------------------------------------------------------ MTP IndexShare

def compare_index_share(inp, step, chains):
    """Oracle IndexShare step on whole chains `chains` vs the GPU step: the
    chains' first rows' scores and selections, then every row's output.  A
    chain whose selection differs inside the tie band is compared with the
    oracle's attention over the GPU's selection."""
    c = step.index_share
    rows = [ch * c + i for ch in chains for i in range(c)]
    sub = W.subset(inp, rows)
    sub_np = W.as_numpy(sub)
    ref = O.decode_step_index_share(sub_np, c, step.index_splits, step.attn_splits)
    lead_vis = sub.row_vis.numpy()[::c]
    g_scores = step.scores[chains].cpu().double().numpy()
    r_scores = np.full_like(g_scores, -np.inf)
    r_scores[:, :ref["scores"].shape[1]] = ref["scores"]
    lead_np = dict(sub_np, row_req=sub_np["row_req"][::c], row_vis=sub_np["row_vis"][::c],
                   head_w=sub_np["head_w"][::c])
    mags = score_magnitudes(lead_np, ref["q_code"], ref["q_scale"])
    ulps = check_scores(g_scores, r_scores, lead_vis, mags, 128 + 64 + 2)
    say(f"  lead scores: max err {ulps:.2f} u*A")
    g_idx = step.topk_idx[chains].cpu().numpy()
    g_cnt = step.topk_count[chains].cpu().numpy()
    out_cmp, lse_cmp = ref["out"].copy(), ref["lse"].copy()
    swapped = []
    for j in range(len(chains)):
        if check_topk_row(g_idx[j], g_cnt[j], ref["topk_idx"][j], ref["topk_count"][j], ref["scores"][j],
                          lead_vis[j], inp.top_k):
            swapped.append(chains[j])
            ch_rows = list(range(j * c, (j + 1) * c))
            o, l = oracle_on_selection(sub_np, ch_rows, np.repeat(g_idx, c, 0), np.repeat(g_cnt, c, 0),
                                       step.attn_splits)
            out_cmp[ch_rows], lse_cmp[ch_rows] = o, l
    g_out = bf16_to_f64(step.out[rows])
    g_lse = step.out_lse[rows].cpu().double().numpy()
    for i in range(len(rows)):
        check_out(g_out[i], g_lse[i], out_cmp[i], lse_cmp[i])
    return swapped


@pytest.mark.parametrize("splits", [None, (4, 3)])
def test_index_share_chains_match_oracle(splits):
    """32 requests x 6 causal draft rows: the indexer and top-k run on each
    chain's first row, every row attends that list (chains placed on one
    XCD each); sampled chains 0, 13 and 31 against the oracle."""
    inp = W.make("c3s", device="cuda")
    step = dsa.DecodeStep(inp, *(splits or (None, None)))
    step.run()
    torch.cuda.synchronize()
    dsa.check_status(step.status)
    say(f"c3s: R={inp.n_rows} chains={inp.n_rows // step.index_share} splits=({step.index_splits},{step.attn_splits})")
    swapped = compare_index_share(inp, step, [0, 13, 31])
    say(f"c3s: swapped {swapped}")


def test_index_share_edge_chains_match_oracle():
    """Short chains on small pages: spans from 2 tokens, k above the first
    row's span, 16 heads, chains of 3, one and four attention splits."""
    cfg = W.Config("edge_share", batch=5, kv_lens=(3, 40, 300, 2100, 2500), rows_per_req=3, causal="mtp",
                   page_size=16, mla_heads=16, index_splits=1, attn_splits=4, index_share=3)
    inp = W.to(W.make(cfg), "cuda")
    for splits in ((1, 4), (2, 1)):
        step = dsa.DecodeStep(inp, *splits)
        step.run()
        torch.cuda.synchronize()
        dsa.check_status(step.status)
        compare_index_share(inp, step, list(range(inp.n_rows // 3)))


def test_shared_lists_in_any_order_and_bad_list_ids():
    """row_list in an arbitrary order (no chains: the plain grid) gives each
    row the oracle's attention over its list; a list id out of range writes
    the row empty with DSA_DEV_ROW_RANGE; a list whose entries reach past a
    shorter row's span leaves those entries out with DSA_DEV_TOPK_OOB."""
    inp = W.to(W.make("c0"), "cuda")
    good = run_step(inp, 1, 1)
    # Lists: row 0's and row 1's own, in a shuffled map over 5 query rows of
    # request 1 (each row sees all of request 1's slots).
    rr = torch.tensor([1, 1, 1, 1, 1], dtype=torch.int32, device="cuda")
    rv = torch.full((5,), int(inp.kv_lens[1]), dtype=torch.int32, device="cuda")
    q = inp.q_mla[torch.tensor([1, 0, 1, 0, 1], device="cuda")].contiguous()
    row_list = torch.tensor([1, 0, 1, 1, 0], dtype=torch.int32, device="cuda")
    st = dsa.new_status()
    out, lse, _ = dsa.sparse_mla_decode_shared(q, inp.kv_cache, inp.page_table, rr, rv, row_list, good.topk_idx,
                                               good.topk_count, 1, inp.sm_scale, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    n = W.as_numpy(W.subset(inp, [0, 1]))
    rl = row_list.cpu().numpy()
    idx = good.topk_idx.cpu().numpy()[rl]
    cnt = good.topk_count.cpu().numpy()[rl]
    # request 1 is the subset's request 1; row 0's list (slots < 1500) lies inside its span
    qn = q.cpu().view(torch.int16).numpy().view(np.uint16)
    r_po, r_pl = O.sparse_mla(qn, n["kv_code"], n["kv_scale"], n["page_table"], np.ones(5, dtype=np.int64), idx,
                              cnt, inp.sm_scale, 1, inp.page_size)
    r_out, r_lse = O.lse_merge(r_po, r_pl)
    check_out(bf16_to_f64(out), lse.cpu().double().numpy(), r_out, r_lse)
    # A list id out of range: that row only is empty.
    bad_list = torch.tensor([1, 0, 7, 1, -1], dtype=torch.int32, device="cuda")
    st = dsa.new_status()
    out2, lse2, _ = dsa.sparse_mla_decode_shared(q, inp.kv_cache, inp.page_table, rr, rv, bad_list,
                                                 good.topk_idx, good.topk_count, 1, inp.sm_scale, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == dsa.DEV_ROW_RANGE
    for i in (2, 4):
        assert torch.all(out2[i] == 0) and torch.all(torch.isneginf(lse2[i]))
    for i in (0, 1, 3):
        assert torch.equal(out2[i], out[i])
    # Request 0's rows (span 1500) attending request 1's list (2048 slots of
    # 5000): the count exceeds the span, so the row is written empty.
    rr0 = torch.zeros(2, dtype=torch.int32, device="cuda")
    rv0 = torch.full((2,), 1500, dtype=torch.int32, device="cuda")
    st = dsa.new_status()
    out3, lse3, _ = dsa.sparse_mla_decode_shared(inp.q_mla[:1].repeat(2, 1, 1).contiguous(), inp.kv_cache,
                                                 inp.page_table, rr0, rv0,
                                                 torch.tensor([0, 1], dtype=torch.int32, device="cuda"),
                                                 good.topk_idx, good.topk_count, 1, inp.sm_scale, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & dsa.DEV_TOPK_OOB
    assert torch.equal(out3[0], good.out[0])
    assert torch.all(out3[1] == 0) and torch.all(torch.isneginf(lse3[1]))
