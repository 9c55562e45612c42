"""GPU parity of dsa_index_topk: the decode indexer with the top-k's candidate
filter in its epilogue, then the merge of the candidates.

Its results must equal, bit for bit, those of the two calls it replaces
(dsa_index_scores with one row a group, then dsa_topk), and match the oracle
under the rules of tests/parity_util.py.  The inputs are seeded and built on
the CPU; some are shaped so that each way through the merge runs:
  random    scores of the synthetic workload: the usual case (the bin of the
            k-th largest candidate holds at most 64 keys);
  ramp_up   scores rising with the slot, so the row's top k sit in its last
            chunks while every chunk keeps only its expected share: fewer than
            k candidates at or above the highest cut, and the merge selects
            from the scores;
  ramp_down the same with the top k in the first chunks;
  ties      five distinct scores: the k-th largest candidate's bin holds
            thousands of keys, and the general selection runs;
  equal     one score everywhere with k below the chunk length: every chunk
            keeps more than its capacity and reports it, and the merge
            selects from the scores.
Crafted rows use one key code (E4M3FN 1.0) and positive head weights and
queries, so slot t scores 128 * k_scale[t] on both sides, exactly.
"""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from parity_util import check_topk_row
from sparse_attention_decode_dsa_amd import dsa
from sparse_attention_decode_dsa_amd import workload as W

pytestmark = pytest.mark.gpu

E4M3_ONE = 0x38


def say(*a):
    print(*a, flush=True)


def fused(g, k, stride):
    sc, idx, cnt, st = dsa.index_topk(g.q_idx, g.head_w, g.k_code, g.k_scale, g.page_table, g.kv_lens,
                                      g.row_req, g.row_vis, k, score_stride=stride)
    torch.cuda.synchronize()
    return sc, idx, cnt, st


def two_calls(g, k, stride, n_splits=1):
    st = dsa.new_status()
    sc, _ = dsa.index_scores(g.q_idx, g.head_w, g.k_code, g.k_scale, g.page_table, g.kv_lens, g.row_req,
                             g.row_vis, score_stride=stride, status=st)
    idx, cnt, _ = dsa.topk(sc, g.row_vis, k, n_splits, status=st)
    torch.cuda.synchronize()
    return sc, idx, cnt, st


def assert_same(a, b):
    sa, ia, ca, ta = a
    sb, ib, cb, tb = b
    assert torch.equal(sa.view(torch.int32), sb.view(torch.int32)), "scores differ"
    assert torch.equal(ca, cb), "counts differ"
    assert torch.equal(ia, ib), "selections differ"
    assert int(ta.item()) == int(tb.item()), (int(ta.item()), int(tb.item()))


CRAFT = W.Config("craft", batch=3, kv_lens=(20000, 9000, 2100), page_size=64, mla_heads=16)


def crafted(kind, top_k, seed=5):
    inp = W.make(dataclasses.replace(CRAFT, top_k=top_k), seed=seed)
    if kind == "random":
        return inp
    rng = np.random.default_rng(seed)
    kc = inp.k_code.clone()
    ks = inp.k_scale.clone()
    p = inp.page_size
    for b in range(inp.cfg.batch):
        v = int(inp.kv_lens[b])
        t = np.arange(v)
        pages = inp.page_table[b, t // p].long()
        offs = torch.from_numpy(t % p)
        if kind == "ramp_up":
            s = 1.0 + t * 2.0 ** -16
        elif kind == "ramp_down":
            s = 2.0 - t * 2.0 ** -16
        elif kind == "ties":
            s = rng.choice([1.0, 1.25, 1.5, 1.75, 2.0], size=v)
        elif kind == "equal":
            s = np.ones(v)
        else:
            raise ValueError(kind)
        kc[pages, offs] = E4M3_ONE
        ks[pages, offs] = torch.from_numpy(s.astype(np.float32))
    return dataclasses.replace(inp, q_idx=torch.ones_like(inp.q_idx), head_w=torch.full_like(inp.head_w, 1 / 64),
                               k_code=kc, k_scale=ks)


@pytest.mark.parametrize("kind,top_k", [("random", 2048), ("ramp_up", 2048), ("ramp_down", 2048),
                                        ("ties", 2048), ("equal", 512), ("ties", 100), ("random", 1),
                                        ("ramp_up", 8192)])
def test_index_topk_matches_two_calls_and_oracle(kind, top_k):
    inp = crafted(kind, top_k)
    g = W.to(inp, "cuda")
    stride = (int(inp.row_vis.max()) + 63) // 64 * 64
    say(f"index_topk {kind} k={top_k} vis={inp.row_vis.tolist()} stride={stride}")
    a = fused(g, top_k, stride)
    dsa.check_status(a[3])
    assert_same(a, two_calls(g, top_k, stride))
    ref = O.decode_step(W.as_numpy(inp), 1, 1)
    idx, cnt = a[1].cpu().numpy(), a[2].cpu().numpy()
    vis = inp.row_vis.numpy()
    swaps = [check_topk_row(idx[i], cnt[i], ref["topk_idx"][i], ref["topk_count"][i], ref["scores"][i],
                            int(vis[i]), top_k) for i in range(inp.n_rows)]
    say(f"  tie-band swaps per row {swaps}")
    if kind != "random":
        assert swaps == [0] * inp.n_rows   # exact scores on both sides
    if kind == "ramp_up":
        for i, v in enumerate(vis):
            c = min(top_k, int(v))
            np.testing.assert_array_equal(idx[i, :c], np.arange(v - c, v))


@pytest.mark.parametrize("page_size,top_k,stride_pad", [(16, 2048, 0), (1024, 2048, 3), (64, 100, 1),
                                                        (16, 1, 0)])
def test_index_topk_edge_rows(page_size, top_k, stride_pad):
    """Empty, one-token, page-edge and k +- 1 rows; unaligned score strides."""
    cfg = W.Config("edge_fused", batch=10, kv_lens=(0, 1, 63, 64, 65, 2047, 2048, 2049, 5000, 777),
                   page_size=page_size, mla_heads=16, top_k=top_k)
    inp = W.make(cfg)
    g = W.to(inp, "cuda")
    stride = (int(inp.row_vis.max()) + 63) // 64 * 64 + stride_pad
    say(f"index_topk edge P={page_size} k={top_k} stride={stride}")
    a = fused(g, top_k, stride)
    dsa.check_status(a[3])
    assert_same(a, two_calls(g, top_k, stride))
    ref = O.decode_step(W.as_numpy(inp), 1, 1)
    idx, cnt = a[1].cpu().numpy(), a[2].cpu().numpy()
    vis = inp.row_vis.numpy()
    for i in range(inp.n_rows):
        check_topk_row(idx[i], cnt[i], ref["topk_idx"][i], ref["topk_count"][i], ref["scores"][i],
                       int(vis[i]), top_k)


@pytest.mark.parametrize("name,n_splits", [("c1_l32k", 1), ("c1", 1), ("c2", 16)])
def test_index_topk_full_size_equals_two_calls(name, n_splits):
    """Every row of the bulk-decode and long-context workloads at full size,
    in the launch configuration the step uses: the fused call against the two
    calls (the oracle checks sampled rows of the same step elsewhere)."""
    inp = W.make(name, device="cuda")
    st = dsa.DecodeStep(inp, index_topk=True)
    assert st.index_topk
    say(f"{name}: R={inp.n_rows} stride={st.score_stride}")
    a = fused(inp, inp.top_k, st.score_stride)
    dsa.check_status(a[3])
    assert_same(a, two_calls(inp, inp.top_k, st.score_stride, n_splits))


def test_index_topk_phases_apart_equal_the_whole_call():
    """DSA_PHASE_SCORE then DSA_PHASE_SELECT on one workspace gives what one
    call with both gives; a select phase run again gives the same again."""
    inp = W.make("c1", device="cuda")
    st = dsa.DecodeStep(inp, index_topk=True)
    k, stride = inp.top_k, st.score_stride
    want = fused(inp, k, stride)
    ws = torch.empty((dsa.index_topk_workspace_size(inp.n_rows, stride, k),), dtype=torch.uint8, device="cuda")
    args = (inp.q_idx, inp.head_w, inp.k_code, inp.k_scale, inp.page_table, inp.kv_lens, inp.row_req,
            inp.row_vis, k)
    sc, idx, cnt, s1 = dsa.index_topk(*args, score_stride=stride, workspace=ws, phases=dsa.PHASE_SCORE)
    idx.fill_(-7)
    dsa.index_topk(*args, score_stride=stride, scores=sc, workspace=ws, topk_idx=idx, topk_count=cnt,
                   status=s1, phases=dsa.PHASE_SELECT)
    torch.cuda.synchronize()
    assert_same((sc, idx, cnt, s1), want)
    idx2 = torch.full_like(idx, -7)
    dsa.index_topk(*args, score_stride=stride, scores=sc, workspace=ws, topk_idx=idx2, topk_count=cnt,
                   status=s1, phases=dsa.PHASE_SELECT)
    torch.cuda.synchronize()
    assert torch.equal(idx2, want[1])


def test_index_topk_reports_as_the_two_calls_do():
    """NaN scores (row 0: a NaN head weight, which every score of the row
    sums), a bad key scale (row 1) and a span past its request's kv_len (row
    2): the fused call sets the same status bits and writes the same scores
    and selections as the two calls."""
    inp = W.make(dataclasses.replace(CRAFT, top_k=512), seed=9)
    p = inp.page_size
    ks = inp.k_scale.clone()
    ks[int(inp.page_table[1, 100 // p]), 100 % p] = -1.0
    hw = inp.head_w.clone()
    hw[0, 0] = float("nan")
    vis = inp.row_vis.clone()
    vis[2] = int(inp.kv_lens[2]) + 1
    bad = dataclasses.replace(inp, head_w=hw, k_scale=ks, row_vis=vis)
    g = W.to(bad, "cuda")
    stride = (int(inp.row_vis.max()) + 63) // 64 * 64
    a = fused(g, 512, stride)
    b = two_calls(g, 512, stride)
    bits = int(a[3].item())
    assert bits & dsa.DEV_NAN and bits & dsa.DEV_SCALE and bits & dsa.DEV_ROW_RANGE, bits
    assert int(torch.isnan(a[0][0]).sum()) == int(inp.row_vis[0])
    assert_same(a, b)
