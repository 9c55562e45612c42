"""GPU parity of the cache write (the step before the decode path) against
the oracle, through the C ABI.  Codes and scales are compared bit for bit
over the whole pool, so rows that must not change are checked too."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from sparse_attention_decode_dsa_amd import dsa
from sparse_attention_decode_dsa_amd import workload as W

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _u16(t):
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def write_both(inp, toks, tables=True):
    """The GPU write into device copies of inp's caches, and the oracle's into
    host copies; returns (gpu arrays, oracle arrays, status, written)."""
    kv = inp.kv_cache.cuda().clone()
    kc = inp.k_code.cuda().clone()
    ks = inp.k_scale.cuda().clone()
    cos = toks.rope_cos.cuda() if tables else None
    sin = toks.rope_sin.cuda() if tables else None
    st = dsa.cache_write(toks.latent.cuda(), toks.rope.cuda(), toks.index_k.cuda(), toks.tok_req.cuda(),
                         toks.tok_slot.cuda(), inp.page_table.cuda(), kv, kc, ks, rope_cos=cos, rope_sin=sin)
    torch.cuda.synchronize()
    ref = O.cache_write(_u16(toks.latent), _u16(toks.rope), _u16(toks.index_k),
                        toks.rope_cos.cpu().numpy() if tables else None,
                        toks.rope_sin.cpu().numpy() if tables else None,
                        toks.tok_req.cpu().numpy(), toks.tok_slot.cpu().numpy(), inp.page_table.cpu().numpy(),
                        inp.page_size, inp.kv_cache.cpu().numpy(), inp.k_code.cpu().numpy(),
                        inp.k_scale.cpu().numpy())
    gpu = (kv.cpu().numpy(), kc.cpu().numpy(), ks.cpu().numpy())
    return gpu, ref[:3], int(st.item()), ref[3]


def assert_pools_equal(gpu, ref):
    np.testing.assert_array_equal(gpu[0], ref[0])
    np.testing.assert_array_equal(gpu[1], ref[1])
    np.testing.assert_array_equal(gpu[2].view(np.int32), ref[2].view(np.int32))


def _c0_tokens(inp):
    """Valid tokens at page edges and span ends, then invalid ones: a request
    out of range, a slot past the block table, a slot past the span (page -1)."""
    p = inp.page_size
    kv = inp.kv_lens.tolist()
    req = [0, 0, 0, 1, 1, 1, 0, 2, 1, 0]
    slot = [0, p - 1, kv[0] - 1, p, kv[1] - 1, 3 * p + 7, 777, 5, inp.max_pages * p, kv[0] + 2 * p]
    return req, slot


@pytest.mark.parametrize("tables", [True, False], ids=["rotated", "as_given"])
def test_tiny_pool_bit_exact(tables):
    inp = W.make("c0")
    req, slot = _c0_tokens(inp)
    toks = W.make_new_tokens(inp, req, slot, seed=11)
    gpu, ref, st, written = write_both(inp, toks, tables)
    say(f"  written {written.tolist()} status {st:#x}")
    assert written.tolist() == [True] * 7 + [False] * 3
    assert st == (dsa.DEV_WRITE | dsa.DEV_PAGE_OOB)
    assert_pools_equal(gpu, ref)


@pytest.mark.parametrize("page_size", [16, 1024])
def test_page_sizes_and_empty_call(page_size):
    cfg = W.Config("cw_pages", batch=3, kv_lens=(1, 700, 2049), page_size=page_size, mla_heads=16)
    inp = W.make(cfg)
    kv = inp.kv_lens.tolist()
    req = [0, 1, 1, 2, 2, 2]
    slot = [0, 0, kv[1] - 1, page_size - 1, page_size, kv[2] - 1]
    toks = W.make_new_tokens(inp, req, slot, seed=12)
    gpu, ref, st, written = write_both(inp, toks)
    assert written.all() and st == 0
    assert_pools_equal(gpu, ref)
    # n_tok == 0 enqueues nothing and leaves the pool alone
    empty = W.make_new_tokens(inp, [], [], seed=13)
    g2, r2, st2, w2 = write_both(inp, empty)
    assert st2 == 0 and len(w2) == 0
    assert_pools_equal(g2, (inp.kv_cache.numpy(), inp.k_code.numpy(), inp.k_scale.numpy()))


def test_bulk_decode_batch_at_the_last_slots():
    """The launch bench.py times: one new token per request of the 64 x 32768
    bulk-decode workload, at slot kv_len - 1, compared over the whole pool."""
    inp = W.make("c1_l32k")
    req = list(range(inp.kv_lens.shape[0]))
    slot = (inp.kv_lens - 1).tolist()
    toks = W.make_new_tokens(inp, req, slot, seed=14)
    say(f"  {len(req)} tokens, pool {tuple(inp.kv_cache.shape)}")
    gpu, ref, st, written = write_both(inp, toks)
    assert written.all() and st == 0
    assert_pools_equal(gpu, ref)


def test_decode_step_over_written_caches():
    """Write, then decode: the step over the caches the oracle wrote (equal to
    the GPU's, checked above) matches the oracle's step."""
    from test_parity_gpu import compare_step, mla_on_oracle_selection, run_step
    inp = W.make("c0")
    kv = inp.kv_lens.tolist()
    toks = W.make_new_tokens(inp, [0, 1], [kv[0] - 1, kv[1] - 1], seed=15)
    gpu, ref, st, written = write_both(inp, toks)
    assert written.all() and st == 0
    assert_pools_equal(gpu, ref)
    new = dataclasses.replace(inp, kv_cache=torch.from_numpy(ref[0]), k_code=torch.from_numpy(ref[1]),
                              k_scale=torch.from_numpy(ref[2]))
    g = W.to(new, "cuda")
    step = run_step(g)
    ref_step, sub, _ = compare_step(g, step, range(g.n_rows), max_swap_rows=1)
    # every row's attention over the written caches, on the oracle's selection
    mla_on_oracle_selection(sub, ref_step, 4)
