"""Host-side checks of the seeded input generator (no GPU, no method arithmetic)."""
import numpy as np
import torch

from sparse_attention_decode_dsa_amd import workload as W
from oracle import dsa_oracle as O


def test_c0_shapes_tables_and_determinism():
    a = W.make("c0")
    b = W.make("c0")
    for f in ("q_idx", "head_w", "q_mla", "k_code", "k_scale", "kv_code", "kv_scale", "page_table"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    assert a.page_size == 64 and a.n_pages == 256 and a.mla_heads == 16
    assert a.kv_lens.tolist() == [1500, 5000]
    pt = a.page_table.numpy()
    assert (pt[0] >= 0).sum() == 24 and (pt[1] >= 0).sum() == 79
    assert np.all(pt[0, 24:] == -1)
    used = pt[pt >= 0]
    assert len(np.unique(used)) == len(used)            # disjoint page ranges
    # poison: tail of the last page and every unused page
    assert float(a.k_scale[pt[0, 23], 1500 - 23 * 64]) == W.POISON_SCALE
    assert float(a.k_scale[pt[0, 23], 1500 - 23 * 64 - 1]) < 1.0
    unused = np.setdiff1d(np.arange(256), used)
    assert torch.all(a.kv_scale[torch.from_numpy(unused)] == W.POISON_SCALE)
    # fp8 codes are never NaN
    assert not torch.any((a.k_code & 0x7F) == 0x7F)
    assert not torch.any((a.kv_code & 0x7F) == 0x7F)


def test_packed_mla_cache_layout():
    a = W.make("c0")
    assert a.kv_cache.shape == (256, 64, 640) and a.kv_cache.dtype == torch.uint8
    # codes are bytes 0..575, the fp32 scale bytes 576..579 (little-endian), pad 0x7F
    raw = a.kv_cache.numpy()
    assert np.array_equal(a.kv_code.numpy(), raw[..., :576])
    sc = raw[..., 576:580].copy().view("<f4")[..., 0]
    assert np.array_equal(a.kv_scale.numpy(), sc)
    assert np.all(raw[..., 580:] == 0x7F)
    assert np.all(sc > 0) and np.all(np.isfinite(sc))


def test_row_geometry_of_mtp_and_prefill():
    c3 = W.Config("t3", batch=3, kv_lens=(100, 300, 260), rows_per_req=6, causal="mtp",
                  page_size=64, mla_heads=16)
    x = W.make(c3)
    assert x.row_req.tolist() == sum(([i] * 6 for i in range(3)), [])
    assert x.row_vis.tolist()[:6] == [95, 96, 97, 98, 99, 100]
    c4 = W.Config("t4", batch=1, kv_lens=(300,), rows_per_req=10, causal="prefill", prefix=290,
                  page_size=64, mla_heads=16)
    y = W.make(c4)
    assert y.row_vis.tolist() == list(range(291, 301))


def test_subset_preserves_rows_bit_for_bit():
    a = W.make("c0")
    full = O.decode_step(W.as_numpy(a), 4, 4)
    s = W.subset(a, [1])
    part = O.decode_step(W.as_numpy(s), 4, 4)
    np.testing.assert_array_equal(part["topk_idx"][0], full["topk_idx"][1])
    np.testing.assert_array_equal(part["out"][0], full["out"][1])


def test_c0_request0_is_dense():
    a = W.make("c0")
    res = O.decode_step(W.as_numpy(a), 4, 4, rows=[0])
    assert res["topk_count"][0] == 1500
    np.testing.assert_array_equal(res["topk_idx"][0, :1500], np.arange(1500))


def test_planted_slots_scale_both_caches():
    cfg = W.Config("tp", batch=2, kv_lens=(700, 900), page_size=64, mla_heads=16, planted=4)
    base = W.make(W.Config("tp", batch=2, kv_lens=(700, 900), page_size=64, mla_heads=16))
    pl = W.make(cfg)
    # the draws before planting are identical, so the boosted entries are exactly x8
    ratio = pl.k_scale / base.k_scale
    boosted = (ratio != 1).nonzero()
    assert boosted.shape[0] == 8
    assert torch.all(ratio[ratio != 1] == 8.0)
    assert torch.equal(pl.kv_scale / base.kv_scale, ratio)
