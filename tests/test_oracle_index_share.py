"""Pins for the oracle's MTP IndexShare step (one top-k list per chain of
draft rows).

The selection itself is pinned by the top-k tests; here the pins fix what the
sharing adds: with chains of one row it is the plain step; a chain's first
row attends its own list; every other row attends exactly the first row's
slots with its own query, checked against torch's float64
scaled_dot_product_attention over the row's whole span with a mask that
keeps only those slots (keys decoded through torch's fp8 cast, an
independent route).  A mutant that gives each row its own list fails that
pin.
"""
import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O


def _chain_inputs(seed=50, h=2, kv=(41, 29), chain=3, top_k=6, p=4, plant_tail=True):
    """Two requests, `chain` causal rows each (row i of a request sees
    kv - chain + i + 1 slots).  With plant_tail the last chain - 1 slots of
    each request (seen only by the later rows) get large index-key scales,
    so that each later row's own top-k would differ from the first row's."""
    rng = np.random.default_rng(seed)
    n_pages = sum(-(-v // p) for v in kv) + 3
    perm = rng.permutation(n_pages)
    pt = np.full((len(kv), max(-(-v // p) for v in kv)), -1)
    off = 0
    for b, v in enumerate(kv):
        n = -(-v // p)
        pt[b, :n] = perm[off:off + n]
        off += n
    rows = len(kv) * chain
    row_req = np.repeat(np.arange(len(kv)), chain)
    row_vis = np.array([kv[b] - chain + i + 1 for b in range(len(kv)) for i in range(chain)])
    g = torch.Generator().manual_seed(seed)
    qi = torch.randn(rows, 64, 128, generator=g).to(torch.bfloat16)
    qm = torch.randn(rows, h, O.D_QK, generator=g).to(torch.bfloat16)
    k_code = rng.integers(0, 256, size=(n_pages, p, 128), dtype=np.uint8)
    k_code[(k_code & 0x7F) == 0x7F] = 0x30
    kv_code = rng.integers(0, 256, size=(n_pages, p, O.D_QK), dtype=np.uint8)
    kv_code[(kv_code & 0x7F) == 0x7F] = 0x30
    k_scale = rng.uniform(0.001, 0.01, (n_pages, p))
    inp = {
        "q_idx": qi.view(torch.int16).numpy().view(np.uint16),
        "head_w": rng.normal(0, 0.125, size=(rows, 64)),
        "q_mla": qm.view(torch.int16).numpy().view(np.uint16),
        "k_code": k_code, "k_scale": k_scale,
        "kv_code": kv_code, "kv_scale": rng.uniform(0.001, 0.01, (n_pages, p)),
        "page_table": pt, "kv_lens": np.array(kv), "row_req": row_req, "row_vis": row_vis,
        "page_size": p, "top_k": top_k, "sm_scale": 1 / 24,
    }
    if plant_tail:
        for b, v in enumerate(kv):
            for t in range(v - chain + 1, v):
                inp["k_scale"][pt[b, t // p], t % p] *= 1e4
    return inp


def _masked_sdpa(inp, r, slots):
    """Row r's attention over its whole span with every slot outside
    `slots` masked out (float64, torch's fp8 decode)."""
    b = int(inp["row_req"][r])
    v = int(inp["row_vis"][r])
    p = int(inp["page_size"])
    t = np.arange(v)
    phys = inp["page_table"][b][t // p] * p + t % p
    codes = np.ascontiguousarray(inp["kv_code"].reshape(-1, O.D_QK)[phys])
    x = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64)
    x = x * torch.from_numpy(inp["kv_scale"].reshape(-1)[phys])[:, None]
    q = torch.from_numpy(inp["q_mla"][r].view(np.int16)).view(torch.bfloat16).to(torch.float64)
    h = q.shape[0]
    mask = torch.from_numpy(np.isin(t, slots))[None, None, :].expand(h, 1, v)
    o = torch.nn.functional.scaled_dot_product_attention(
        q[:, None], x[None].expand(h, v, O.D_QK).contiguous(),
        x[None, :, :O.D_LATENT].expand(h, v, O.D_LATENT).contiguous(), attn_mask=mask,
        scale=float(inp["sm_scale"]))[:, 0]
    logits = float(inp["sm_scale"]) * (q @ x.T)
    lse = torch.logsumexp(logits.masked_fill(~mask[:, 0], -torch.inf), dim=1)
    return o.numpy(), lse.numpy()


def test_chains_of_one_row_are_the_plain_step():
    inp = _chain_inputs(chain=3)
    a = O.decode_step(inp, 1, 2)
    b = O.decode_step_index_share(inp, 1, 1, 2)
    np.testing.assert_array_equal(a["topk_idx"], b["topk_idx"])
    np.testing.assert_array_equal(a["out"], b["out"])
    np.testing.assert_array_equal(a["lse"], b["lse"])


@pytest.mark.parametrize("chain,splits", [(3, (1, 1)), (3, (2, 3))])
def test_every_row_attends_its_first_rows_slots(chain, splits):
    inp = _chain_inputs(chain=chain)
    res = O.decode_step_index_share(inp, chain, *splits)
    plain = O.decode_step(inp, 1, 1)
    np.testing.assert_array_equal(res["lead_rows"], np.arange(0, len(inp["row_req"]), chain))
    for r in range(len(inp["row_req"])):
        lead = res["row_list"][r]
        sel = res["topk_idx"][lead][: res["topk_count"][lead]]
        o, lse = _masked_sdpa(inp, r, sel)
        np.testing.assert_allclose(res["out"][r], o, rtol=1e-10, atol=1e-13)
        np.testing.assert_allclose(res["lse"][r], lse, rtol=1e-12, atol=1e-12)
        if r % chain == 0:   # a chain's first row attends its own list: the plain step
            np.testing.assert_array_equal(sel, plain["topk_idx"][r][: plain["topk_count"][r]])
            np.testing.assert_allclose(res["out"][r], plain["out"][r], rtol=1e-12, atol=1e-14)


def test_pin_catches_rows_that_keep_their_own_lists():
    inp = _chain_inputs(chain=3)
    res = O.decode_step_index_share(inp, 3)
    own = O.decode_step(inp, 1, 1)           # every row its own selection: no sharing
    caught = 0
    for r in range(len(inp["row_req"])):
        if r % 3 == 0:
            continue
        lead = res["row_list"][r]
        o, _ = _masked_sdpa(inp, r, res["topk_idx"][lead][: res["topk_count"][lead]])
        assert not np.array_equal(np.sort(own["topk_idx"][r]), np.sort(res["topk_idx"][lead]))
        caught += not np.allclose(own["out"][r], o, rtol=1e-6, atol=1e-9)
    assert caught == 4


def test_chains_are_validated():
    inp = _chain_inputs(chain=3)
    with pytest.raises(ValueError):
        O.decode_step_index_share(inp, 4)            # 6 rows are not whole chains of 4
    bad = dict(inp)
    bad["row_req"] = np.array([0, 0, 1, 1, 1, 0])
    with pytest.raises(ValueError):
        O.decode_step_index_share(bad, 3)            # a chain across two requests
    bad = dict(inp)
    bad["row_vis"] = inp["row_vis"][[1, 0, 2, 3, 4, 5]]
    with pytest.raises(ValueError):
        O.decode_step_index_share(bad, 3)            # the first row sees more than the second
