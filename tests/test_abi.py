"""CPU checks of the C ABI: libdsa.so loads, exports every function that
include/dsa.h declares, and rejects invalid arguments with the documented
status before any HIP call (no compute is launched here)."""
import ctypes
import os
import re

import pytest

from sparse_attention_decode_dsa_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

OK, NULL, SHAPE, UNSUP, WS, SCRATCH = 0, -1, -2, -3, -4, -6
P = 0x1000  # a non-NULL dummy device pointer; never dereferenced on these paths


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(dsa_\w+)\s*\(", src, flags=re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(dsa.lib_path()):
        pytest.fail("libdsa.so is not built; run __graft_entry__.build()")
    return dsa.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared()
    assert {"dsa_abi_version", "dsa_status_string", "dsa_quantize_q", "dsa_index_scores",
            "dsa_topk_workspace_size", "dsa_topk", "dsa_sparse_mla_decode", "dsa_lse_merge",
            "dsa_cache_write", "dsa_lse_merge_project"} <= set(names)
    raw = ctypes.CDLL(dsa.lib_path())
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(dsa._SIGS), "binding and header disagree"


def test_abi_version_and_status_strings(L):
    assert L.dsa_abi_version() == dsa.ABI_VERSION
    hdr = open(HEADER).read()
    assert f"#define DSA_ABI_VERSION {dsa.ABI_VERSION}" in hdr
    for code in (OK, NULL, SHAPE, UNSUP, WS, -5, SCRATCH):
        assert dsa.status_string(code).startswith("DSA_")
    assert dsa.status_string(12345) == "unknown"


def _idx(L, **kw):
    a = dict(q=P, head_w=P, k_code=P, k_scale=P, page_table=P, kv_lens=P,
             row_req=P, row_vis=P, n_rows=4, batch=2, num_pages=10, max_pages=5, page_size=256,
             n_heads=64, head_dim=128, group_rows=1, flags=0, scores=P, score_stride=1280, status=P,
             stream=None)
    a.update(kw)
    return L.dsa_index_scores(*a.values())


def test_index_scores_validation(L):
    assert _idx(L, flags=2) == SHAPE                            # unknown flag bits
    assert _idx(L, flags=1, group_rows=2) == SHAPE              # whole-row loads: one row a group
    assert _idx(L, flags=1, n_rows=0) == OK
    assert _idx(L, n_heads=32) == UNSUP
    assert _idx(L, head_dim=64) == UNSUP
    assert _idx(L, page_size=100) == UNSUP
    assert _idx(L, page_size=8) == UNSUP
    assert _idx(L, page_size=0) == SHAPE
    assert _idx(L, n_rows=-1) == SHAPE
    assert _idx(L, batch=0) == SHAPE
    assert _idx(L, group_rows=3) == SHAPE      # 4 rows not divisible by 3
    assert _idx(L, group_rows=9, n_rows=9) == SHAPE
    assert _idx(L, score_stride=0) == SHAPE
    assert _idx(L, q=None) == NULL
    assert _idx(L, status=None) == NULL
    assert _idx(L, n_rows=0) == OK             # nothing to enqueue


def _tk(L, **kw):
    a = dict(scores=P, score_stride=32768, row_vis=P, n_rows=4, top_k=2048, n_splits=1,
             workspace=None, workspace_bytes=0, topk_idx=P, topk_count=P, status=P, stream=None)
    a.update(kw)
    return L.dsa_topk(*a.values())


def test_topk_validation_and_workspace(L):
    assert L.dsa_topk_workspace_size(4, 2048, 1) == 0
    need = L.dsa_topk_workspace_size(4, 2048, 16)
    # candidate keys and slots, then a count, a cut and a 512-bin histogram per split
    assert need == 4 * 16 * 2048 * 8 + 4 * 16 * (3 + 512) * 4
    assert _tk(L, top_k=0) == SHAPE
    assert _tk(L, top_k=8193) == SHAPE
    assert _tk(L, score_stride=32769) == SHAPE                   # one split longer than 32768
    assert _tk(L, n_splits=65) == SHAPE
    assert _tk(L, n_splits=17, score_stride=131072) == SHAPE    # 17 * 2048 candidates > 32768
    assert _tk(L, n_splits=16, score_stride=131072) == WS       # no workspace
    assert _tk(L, n_splits=16, score_stride=131072, workspace=P, workspace_bytes=need - 1) == WS
    assert _tk(L, scores=None) == NULL
    assert _tk(L, n_rows=0) == OK


def _mla(L, **kw):
    a = dict(q=P, kv_cache=P, page_table=P, row_req=P, row_vis=P, topk_idx=P,
             topk_count=P, n_rows=4, batch=4, num_pages=100, max_pages=20, page_size=256,
             n_heads=32, top_k=2048, n_splits=4, sm_scale=0.04, part_o=P, part_lse=P, out=None,
             out_lse=None, status=P, stream=None)
    a.update(kw)
    return L.dsa_sparse_mla_decode(*a.values())


def test_sparse_mla_validation(L):
    assert _mla(L, n_heads=128) == UNSUP
    assert _mla(L, n_heads=0) == SHAPE
    assert _mla(L, n_splits=0) == SHAPE
    assert _mla(L, n_splits=65) == SHAPE
    assert _mla(L, sm_scale=float("nan")) == SHAPE
    assert _mla(L, sm_scale=float("inf")) == SHAPE
    assert _mla(L, part_o=None) == NULL                      # split path needs partials
    assert _mla(L, part_o=P + 2) == SHAPE                    # bf16 partials go out 4 bytes a lane
    assert _mla(L, n_splits=1, out=None) == NULL             # lone split needs out
    assert _mla(L, page_size=48) == UNSUP
    assert _mla(L, q=None) == NULL
    assert _mla(L, n_rows=0) == OK


def test_lse_merge_and_quantize_validation(L):
    m = L.dsa_lse_merge
    assert m(P, P, 4, 32, 4, 256, P, None, None) == UNSUP
    assert m(P, P, 4, 32, 0, 512, P, None, None) == SHAPE
    assert m(P, P, 4, 32, 65, 512, P, None, None) == SHAPE
    assert m(None, P, 4, 32, 4, 512, P, None, None) == NULL
    assert m(P, P, 4, 32, 4, 512, None, None, None) == NULL
    assert m(P + 8, P, 4, 32, 4, 512, P, None, None) == SHAPE   # 16-byte aligned partials and output
    assert m(P, P, 4, 32, 4, 512, P + 2, None, None) == SHAPE
    assert m(P, P, 0, 32, 4, 512, P, None, None) == OK
    q = L.dsa_quantize_q
    assert q(P, 4, 64, 64, P, P, None) == UNSUP
    assert q(P, -1, 64, 128, P, P, None) == SHAPE
    assert q(None, 4, 64, 128, P, P, None) == NULL
    assert q(P, 0, 64, 128, P, P, None) == OK


def _cw(L, **kw):
    a = dict(latent=P, rope=P, index_k=P, rope_cos=None, rope_sin=None, max_pos=0, tok_req=P, tok_slot=P,
             n_tok=4, page_table=P, batch=2, num_pages=10, max_pages=5, page_size=256, kv_cache=P,
             k_code=P, k_scale=P, status=P, stream=None)
    a.update(kw)
    return L.dsa_cache_write(*a.values())


def test_cache_write_validation(L):
    assert _cw(L, n_tok=-1) == SHAPE
    assert _cw(L, page_size=100) == UNSUP
    assert _cw(L, batch=0) == SHAPE
    assert _cw(L, rope_cos=P) == NULL                         # one table without the other
    assert _cw(L, rope_cos=P, rope_sin=P, max_pos=0) == SHAPE
    assert _cw(L, latent=None) == NULL
    assert _cw(L, kv_cache=None) == NULL
    assert _cw(L, status=None) == NULL
    assert _cw(L, latent=P + 8) == SHAPE                      # rows must be 16-byte aligned
    assert _cw(L, kv_cache=P + 4) == SHAPE
    assert _cw(L, n_tok=0) == OK                              # nothing to enqueue
    assert _cw(L, n_tok=0, latent=None, kv_cache=None) == OK  # empty batches may pass NULL arrays
    assert _cw(L, n_tok=0, rope_cos=P, rope_sin=P, max_pos=64) == OK


def _mp(L, **kw):
    a = dict(part_o=P, part_lse=P, n_rows=4, n_heads=32, n_splits=4, d_latent=512, w_uv=P, d_v=128,
             out=P, out_lse=None, stream=None)
    a.update(kw)
    return L.dsa_lse_merge_project(*a.values())


def test_lse_merge_project_validation(L):
    assert _mp(L, d_v=64) == UNSUP
    assert _mp(L, d_latent=576) == UNSUP
    assert _mp(L, n_splits=0) == SHAPE
    assert _mp(L, n_splits=65) == SHAPE
    assert _mp(L, n_heads=0) == SHAPE
    assert _mp(L, n_rows=-1) == SHAPE
    assert _mp(L, w_uv=None) == NULL
    assert _mp(L, out=None) == NULL
    assert _mp(L, part_o=P + 4) == SHAPE        # 16-byte aligned partials
    assert _mp(L, w_uv=P + 8) == SHAPE          # 16-byte aligned weights
    assert _mp(L, n_rows=0) == OK


def test_topk_noalloc_validation(L):
    """The no-allocation top-k applies dsa_topk's rules, then rejects a call
    whose candidates exceed its fixed array, all before any HIP call."""
    def call(**kw):
        a = dict(scores=P, score_stride=4096, row_vis=P, n_rows=8, top_k=2048, n_splits=4,
                 topk_idx=P, topk_count=P, status=P, stream=None)
        a.update(kw)
        return L.dsa_topk_noalloc(*a.values())
    assert call(n_rows=-1) == SHAPE
    assert call(top_k=0) == SHAPE
    assert call(n_splits=65) == SHAPE
    assert call(scores=None) == NULL
    assert call(n_rows=0) == OK
    # 1024 rows x 16 splits x 2048 candidates x 8 bytes = 256 MiB > 16 MiB
    assert call(n_rows=1024, n_splits=16, score_stride=64) == SCRATCH
    hdr = open(HEADER).read()
    assert "#define DSA_NOALLOC_SCRATCH_BYTES (16u << 20)" in hdr


def test_bandwidth_library_exports_its_header():
    """libdsa_bw.so (the benchmark's plain read and copy kernels) exports what
    include/dsa_bw.h declares and rejects bad arguments before any launch."""
    from sparse_attention_decode_dsa_amd import build as B
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "dsa_bw.h")).read(), flags=re.S)
    names = set(re.findall(r"^\s*int\s+(dsa_bw_\w+)\s*\(", src, flags=re.M))
    assert names == {"dsa_bw_stream_read", "dsa_bw_stream_read_nt", "dsa_bw_copy"}
    L = ctypes.CDLL(B.BW_LIB)
    for n in names:
        assert hasattr(L, n)
    L.dsa_bw_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p,
                                     ctypes.c_void_p]
    L.dsa_bw_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]
    L.dsa_bw_stream_read_nt.argtypes = L.dsa_bw_stream_read.argtypes
    for read in (L.dsa_bw_stream_read, L.dsa_bw_stream_read_nt):
        assert read(None, 4096, 8, P, None) == -1
        assert read(P, 4095, 8, P, None) == -1
        assert read(P, 4096, 0, P, None) == -1
    assert L.dsa_bw_copy(P, P + 8, 4096, 8, None) == -1


def _itk(L, **kw):
    a = dict(q=P, head_w=P, k_code=P, k_scale=P, page_table=P, kv_lens=P, row_req=P, row_vis=P, n_rows=4,
             batch=2, num_pages=200, max_pages=128, page_size=256, n_heads=64, head_dim=128, scores=P,
             score_stride=32768, top_k=2048, phases=3, workspace=P, workspace_bytes=1 << 30, topk_idx=P,
             topk_count=P, status=P, stream=None)
    a.update(kw)
    return L.dsa_index_topk(*a.values())


def test_index_topk_validation_and_workspace(L):
    """dsa_index_topk applies dsa_index_scores' rules, the top-k's, its own
    phase and chunk-count rules, then checks the workspace, all before any
    HIP call."""
    # 4 rows x 32768 slots: 1024-token chunks (the indexer's smallest), 32 a
    # row, each holding up to min(1024, k) candidate keys and slots, a count
    # and a cut.
    assert L.dsa_index_topk_workspace_size(4, 32768, 2048) == 4 * 32 * (2 * 1024 + 2) * 4
    # 64 rows x 32768 slots: 4096-token chunks, 8 a row, k = 2048 candidates each.
    assert L.dsa_index_topk_workspace_size(64, 32768, 2048) == 64 * 8 * (2 * 2048 + 2) * 4
    assert L.dsa_index_topk_workspace_size(0, 32768, 2048) == 0
    need = L.dsa_index_topk_workspace_size(4, 32768, 2048)
    assert _itk(L, n_heads=32) == UNSUP
    assert _itk(L, page_size=100) == UNSUP
    assert _itk(L, n_rows=-1) == SHAPE
    assert _itk(L, top_k=0) == SHAPE
    assert _itk(L, top_k=8193) == SHAPE
    assert _itk(L, phases=0) == SHAPE
    assert _itk(L, phases=4) == SHAPE
    assert _itk(L, n_rows=1, score_stride=8192 * 1024 + 1, max_pages=40000) == SHAPE   # 1025 chunks
    assert _itk(L, q=None) == NULL
    assert _itk(L, scores=None) == NULL
    assert _itk(L, topk_idx=None) == NULL
    assert _itk(L, topk_count=None) == NULL
    assert _itk(L, workspace=None) == WS
    assert _itk(L, workspace_bytes=need - 1) == WS
    assert _itk(L, workspace=P + 2) == WS
    assert _itk(L, n_rows=0) == OK


def test_rows_entry_points_validation(L):
    """dsa_topk_rows applies dsa_topk's rules and the page geometry, then
    needs its request, block-table and rows arrays; dsa_sparse_mla_decode_rows
    applies the attention's rules without a block table."""
    def tk(**kw):
        a = dict(scores=P, score_stride=32768, row_vis=P, row_req=P, page_table=P, batch=4, num_pages=600,
                 max_pages=128, page_size=256, n_rows=4, top_k=2048, n_splits=1, workspace=None,
                 workspace_bytes=0, topk_idx=P, topk_count=P, topk_rows=P, status=P, stream=None)
        a.update(kw)
        return L.dsa_topk_rows(*a.values())
    assert tk(top_k=0) == SHAPE
    assert tk(n_splits=65) == SHAPE
    assert tk(page_size=100) == UNSUP
    assert tk(batch=0) == SHAPE
    assert tk(row_req=None) == NULL
    assert tk(page_table=None) == NULL
    assert tk(topk_rows=None) == NULL
    assert tk(scores=None) == NULL
    assert tk(n_splits=16, score_stride=131072) == WS
    assert tk(n_rows=0) == OK

    def mla(**kw):
        a = dict(q=P, kv_cache=P, row_vis=P, topk_rows=P, topk_count=P, n_rows=4, num_pages=100,
                 page_size=256, n_heads=32, top_k=2048, n_splits=4, sm_scale=0.04, part_o=P, part_lse=P,
                 out=None, out_lse=None, status=P, stream=None)
        a.update(kw)
        return L.dsa_sparse_mla_decode_rows(*a.values())
    assert mla(n_heads=128) == UNSUP
    assert mla(n_splits=0) == SHAPE
    assert mla(sm_scale=float("nan")) == SHAPE
    assert mla(page_size=48) == UNSUP
    assert mla(topk_rows=None) == NULL
    assert mla(part_o=None) == NULL
    assert mla(n_splits=1) == NULL          # a lone split needs out
    assert mla(row_vis=None) == NULL
    assert mla(n_rows=0) == OK
