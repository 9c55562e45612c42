"""GPU parity of the physical-row path: dsa_topk_rows emits the selected
slots' rows in the paged caches and dsa_sparse_mla_decode_rows attends them
with no block-table walk.

dsa_topk_rows must select exactly what dsa_topk selects, and its rows must be
the block-table image of those slots (computed here on the host from the
page table); the attention over the rows must equal, bit for bit, the
attention over the slots; and the step through both against the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch

from sparse_attention_decode_dsa_amd import dsa
from sparse_attention_decode_dsa_amd import workload as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def host_rows(idx, cnt, row_req, page_table, page_size, num_pages):
    """Block-table image of each selected slot; -1 after the count and for a
    slot on a page id outside the pool."""
    idx = np.asarray(idx)
    out = np.full_like(idx, -1)
    for r in range(idx.shape[0]):
        b = int(row_req[r])
        for i in range(int(cnt[r])):
            t = int(idx[r, i])
            page = int(page_table[b, t // page_size])
            if 0 <= page < num_pages:
                out[r, i] = page * page_size + t % page_size
    return out


def scores_of(inp, stride):
    st = dsa.new_status()
    sc, _ = dsa.index_scores(inp.q_idx, inp.head_w, inp.k_code, inp.k_scale, inp.page_table, inp.kv_lens,
                             inp.row_req, inp.row_vis, score_stride=stride, status=st)
    torch.cuda.synchronize()
    dsa.check_status(st)
    return sc


def check_topk_rows(inp, stride, n_splits, sc=None):
    sc = scores_of(inp, stride) if sc is None else sc
    k = inp.top_k
    idx, cnt, st = dsa.topk(sc, inp.row_vis, k, n_splits)
    idx2, cnt2, rows, st2 = dsa.topk_rows(sc, inp.row_vis, inp.row_req, inp.page_table, inp.kv_cache.shape[0],
                                          inp.page_size, k, n_splits)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2) and torch.equal(cnt, cnt2)
    want = host_rows(idx.cpu().numpy(), cnt.cpu().numpy(), inp.row_req.cpu().numpy(), inp.page_table.cpu().numpy(),
                     inp.page_size, inp.kv_cache.shape[0])
    np.testing.assert_array_equal(rows.cpu().numpy(), want)
    return idx, cnt, rows, st2


@pytest.mark.parametrize("name,n_splits", [("c0", 1), ("c0", 4), ("c1_l32k", 1), ("c2", 16), ("c3", 4)])
def test_topk_rows_are_the_block_table_image_of_the_selection(name, n_splits):
    inp = W.make(name, device="cuda")
    stride = (int(inp.row_vis.max()) + 63) // 64 * 64
    say(f"{name}: R={inp.n_rows} splits={n_splits}")
    if inp.cfg.group_rows > 1:   # rows scored in groups: scores from the grouped indexer
        st = dsa.new_status()
        sc, _ = dsa.index_scores(inp.q_idx, inp.head_w, inp.k_code, inp.k_scale, inp.page_table, inp.kv_lens,
                                 inp.row_req, inp.row_vis, group_rows=inp.cfg.group_rows, score_stride=stride,
                                 status=st)
        _, _, _, st2 = check_topk_rows(inp, stride, n_splits, sc)
    else:
        _, _, _, st2 = check_topk_rows(inp, stride, n_splits)
    dsa.check_status(st2)


@pytest.mark.parametrize("page_size,kv", [(16, (20000, 3000, 1)), (1024, (5000, 70000, 2049))])
def test_topk_rows_page_sizes_and_long_block_tables(page_size, kv):
    """16-token pages with 1250 pages a request (the block table is read from
    global memory, not staged) and 1024-token pages."""
    cfg = W.Config("rows_edge", batch=len(kv), kv_lens=kv, page_size=page_size, mla_heads=16)
    inp = W.make(cfg, device="cuda")
    stride = (int(inp.row_vis.max()) + 63) // 64 * 64
    n_splits = -(-stride // 32768)   # a split's list holds at most 32768 scores
    say(f"rows P={page_size} kv={kv} max_pages={inp.page_table.shape[1]} splits={n_splits}")
    _, _, _, st = check_topk_rows(inp, stride, n_splits)
    dsa.check_status(st)


def test_topk_rows_bad_page_and_bad_request_are_reported():
    inp = W.make("c0", device="cuda")
    stride = (int(inp.row_vis.max()) + 63) // 64 * 64
    sc = scores_of(inp, stride)
    pt = inp.page_table.clone()
    pt[1, 10] = inp.kv_cache.shape[0] + 3            # a page id outside the pool, inside request 1's span
    bad = dataclasses.replace(inp, page_table=pt)
    idx, cnt, rows, st = check_topk_rows(bad, stride, 1, sc)
    assert int(st.item()) & dsa.DEV_PAGE_OOB
    rr = inp.row_req.clone()
    rr[0] = 7                                          # no such request
    idx, cnt, rows, st = dsa.topk_rows(sc, inp.row_vis, rr, inp.page_table, inp.kv_cache.shape[0], inp.page_size,
                                       inp.top_k, 1)
    torch.cuda.synchronize()
    assert int(st.item()) & dsa.DEV_ROW_RANGE
    assert torch.all(rows[0] == -1)
    want, wcnt, _ = dsa.topk(sc, inp.row_vis, inp.top_k, 1)
    torch.cuda.synchronize()
    assert torch.equal(idx, want) and torch.equal(cnt, wcnt)


@pytest.mark.parametrize("name,n_splits", [("c0", 1), ("c0", 4), ("c1_l32k", 4), ("c2", 32), ("c3", 1)])
def test_attention_over_rows_equals_attention_over_slots(name, n_splits):
    inp = W.make(name, device="cuda")
    stride = (int(inp.row_vis.max()) + 63) // 64 * 64
    st0 = dsa.new_status()
    sc, _ = dsa.index_scores(inp.q_idx, inp.head_w, inp.k_code, inp.k_scale, inp.page_table, inp.kv_lens,
                             inp.row_req, inp.row_vis, group_rows=inp.cfg.group_rows, score_stride=stride,
                             status=st0)
    splits = inp.cfg.index_splits
    idx, cnt, rows, st = dsa.topk_rows(sc, inp.row_vis, inp.row_req, inp.page_table, inp.kv_cache.shape[0],
                                       inp.page_size, inp.top_k, splits)
    a = dsa.sparse_mla_decode(inp.q_mla, inp.kv_cache, inp.page_table, inp.row_req, inp.row_vis, idx, cnt,
                              n_splits, inp.sm_scale)
    b = dsa.sparse_mla_decode_rows(inp.q_mla, inp.kv_cache, inp.row_vis, rows, cnt, n_splits, inp.sm_scale)
    torch.cuda.synchronize()
    dsa.check_status(st0)
    dsa.check_status(st)
    dsa.check_status(a[2])
    dsa.check_status(b[2])
    say(f"{name}: attention splits {n_splits}")
    for x, y in zip(a[:2], b[:2]):
        assert torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x.view(torch.int32),
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))


def test_attention_over_rows_leaves_out_bad_rows():
    """-1 entries are left out quietly (the top-k reported them); entries
    past the pool are left out and set DSA_DEV_TOPK_OOB; the rest attend as
    the slot path over the same surviving entries."""
    inp = W.make("c0", device="cuda")
    stride = (int(inp.row_vis.max()) + 63) // 64 * 64
    sc = scores_of(inp, stride)
    idx, cnt, rows, st = dsa.topk_rows(sc, inp.row_vis, inp.row_req, inp.page_table, inp.kv_cache.shape[0],
                                       inp.page_size, inp.top_k, 1)
    torch.cuda.synchronize()
    r2 = rows.clone()
    r2[0, 5] = -1
    st1 = dsa.new_status()
    dsa.sparse_mla_decode_rows(inp.q_mla, inp.kv_cache, inp.row_vis, r2, cnt, 1, inp.sm_scale, status=st1)
    torch.cuda.synchronize()
    assert int(st1.item()) == 0
    r2[1, 7] = inp.kv_cache.shape[0] * inp.page_size   # one past the pool
    out, lse, st2 = dsa.sparse_mla_decode_rows(inp.q_mla, inp.kv_cache, inp.row_vis, r2, cnt, 1, inp.sm_scale)
    torch.cuda.synchronize()
    assert int(st2.item()) == dsa.DEV_TOPK_OOB
    # The slot path with the same two entries made invalid (past the span).
    i2 = idx.clone()
    i2[0, 5] = int(inp.row_vis[0]) + 1
    i2[1, 7] = int(inp.row_vis[1]) + 1
    want, wlse, _ = dsa.sparse_mla_decode(inp.q_mla, inp.kv_cache, inp.page_table, inp.row_req, inp.row_vis, i2,
                                          cnt, 1, inp.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
    assert torch.equal(lse, wlse)
