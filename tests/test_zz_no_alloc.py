"""dsa_topk_noalloc (candidates in the library's fixed device array) against
dsa_topk (candidates in a caller workspace): the same selection bit for bit,
on two calls in a row, the second with a smaller input, through the C ABI."""
import numpy as np
import pytest
import torch

from sparse_attention_decode_dsa_amd import dsa

pytestmark = pytest.mark.gpu


def _scores(rng, r, stride, vis):
    s = rng.normal(size=(r, stride)).astype(np.float32)
    ties = rng.random((r, stride)) < 0.3
    s[ties] = rng.choice(np.array([-0.5, 0.0, 0.75, 1.5], dtype=np.float32), size=ties.sum())
    for i, v in enumerate(vis):
        s[i, v:] = -np.inf
    return torch.from_numpy(s).cuda()


def _both(scores, vis, k, n_splits):
    v = torch.tensor(vis, dtype=torch.int32).cuda()
    st_a, st_b = dsa.new_status(), dsa.new_status()
    want_idx, want_cnt, _ = dsa.topk(scores, v, k, n_splits, status=st_a)
    got_idx, got_cnt, _ = dsa.topk_noalloc(scores, v, k, n_splits, status=st_b)
    torch.cuda.synchronize()
    assert int(st_a.item()) == 0 and int(st_b.item()) == 0
    assert torch.equal(got_cnt, want_cnt)
    assert torch.equal(got_idx, want_idx)
    return got_idx, got_cnt


def test_noalloc_matches_workspace_topk_on_two_calls():
    rng = np.random.default_rng(77)
    # First call: long rows, 16 splits (2 MiB of candidates in the array).
    vis1 = [131072, 9600, 38000, 77000, 0, 1, 2048, 2049]
    s1 = _scores(rng, len(vis1), 131072, vis1)
    print("call 1: 8 rows, stride 131072, k 2048, 16 splits", flush=True)
    idx1, cnt1 = _both(s1, vis1, 2048, 16)
    assert cnt1.tolist() == [min(2048, v) for v in vis1]
    # Second call: fewer, shorter rows and another k; the array still holds
    # the first call's candidates, which must not leak into this result.
    vis2 = [5000, 100, 3333]
    s2 = _scores(rng, len(vis2), 6000, vis2)
    print("call 2: 3 rows, stride 6000, k 100, 4 splits", flush=True)
    idx2, cnt2 = _both(s2, vis2, 100, 4)
    assert cnt2.tolist() == [100, 100, 100]
    # One split needs no candidates at all.
    _both(s2, vis2, 100, 1)


def test_noalloc_rejects_a_call_beyond_its_array():
    # 1024 rows x 16 splits x 2048 candidates x 8 bytes = 256 MiB > 16 MiB.
    s = torch.zeros((1024, 64), dtype=torch.float32, device="cuda")
    v = torch.full((1024,), 64, dtype=torch.int32, device="cuda")
    with pytest.raises(dsa.DsaError, match="DSA_ERR_SCRATCH"):
        dsa.topk_noalloc(s, v, 2048, 16)
