"""Thin Python binding of libdsa.so (include/dsa.h), same names as the C ABI.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI.  Tensors must be contiguous CUDA (HIP) tensors of
the documented dtypes; outputs are allocated with torch when not given.  A
nonzero host status raises DsaError; device-detected faults accumulate in an
int32 status tensor that ``check_status`` turns into DsaError.

There is no fallback: if libdsa.so is missing or was built for another ABI,
loading fails loudly.
"""

from __future__ import annotations

import ctypes
import os

import torch

ABI_VERSION = 12
_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DEV_BITS = {1: "PAGE_OOB", 2: "TOPK_OOB", 4: "ROW_RANGE", 8: "GROUP", 16: "NAN", 32: "WRITE", 64: "SCALE"}
DEV_PAGE_OOB, DEV_TOPK_OOB, DEV_ROW_RANGE, DEV_GROUP, DEV_NAN, DEV_WRITE, DEV_SCALE = 1, 2, 4, 8, 16, 32, 64
PHASE_SCORE, PHASE_SELECT = 1, 2   # dsa_index_topk's halves


class DsaError(RuntimeError):
    """A libdsa.so call was rejected, or a kernel reported a device fault."""


_i32 = ctypes.c_int32
_p = ctypes.c_void_p
_f32 = ctypes.c_float
_SIGS = {
    "dsa_abi_version": ([], ctypes.c_int),
    "dsa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "dsa_quantize_q": ([_p, _i32, _i32, _i32, _p, _p, _p], ctypes.c_int),
    "dsa_index_scores": ([_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                          _i32, _i32, _i32, _p, _i32, _p, _p], ctypes.c_int),
    "dsa_index_topk_workspace_size": ([_i32, _i32, _i32], ctypes.c_size_t),
    "dsa_index_topk": ([_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                        _p, _i32, _i32, _i32, _p, ctypes.c_size_t, _p, _p, _p, _p], ctypes.c_int),
    "dsa_topk_workspace_size": ([_i32, _i32, _i32], ctypes.c_size_t),
    "dsa_topk": ([_p, _i32, _p, _i32, _i32, _i32, _p, ctypes.c_size_t, _p, _p, _p, _p], ctypes.c_int),
    "dsa_topk_noalloc": ([_p, _i32, _p, _i32, _i32, _i32, _p, _p, _p, _p], ctypes.c_int),
    "dsa_topk_rows": ([_p, _i32, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _p, ctypes.c_size_t,
                       _p, _p, _p, _p, _p], ctypes.c_int),
    "dsa_sparse_mla_decode_rows": ([_p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _p, _p, _p,
                                    _p, _p, _p], ctypes.c_int),
    "dsa_sparse_mla_decode": ([_p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                               _i32, _i32, _f32, _p, _p, _p, _p, _p, _p], ctypes.c_int),
    "dsa_sparse_mla_decode_shared": ([_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32,
                                      _i32, _i32, _i32, _f32, _p, _p, _p, _p, _p, _p], ctypes.c_int),
    "dsa_lse_merge": ([_p, _p, _i32, _i32, _i32, _i32, _p, _p, _p], ctypes.c_int),
    "dsa_lse_merge_project": ([_p, _p, _i32, _i32, _i32, _i32, _p, _i32, _p, _p, _p], ctypes.c_int),
    "dsa_cache_write": ([_p, _p, _p, _p, _p, _i32, _p, _p, _i32, _p, _i32, _i32, _i32, _i32,
                         _p, _p, _p, _p, _p], ctypes.c_int),
}

_lib = None


def lib_path() -> str:
    return _LIB_PATH


def lib() -> ctypes.CDLL:
    """Load libdsa.so once and check its ABI version."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise DsaError(f"{_LIB_PATH} is not built; run `python -m sparse_attention_decode_dsa_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        v = L.dsa_abi_version()
        if v != ABI_VERSION:
            raise DsaError(f"libdsa.so ABI version {v}, binding expects {ABI_VERSION}")
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().dsa_status_string(code).decode()


def _check(rc: int, what: str):
    if rc != 0:
        raise DsaError(f"{what}: {status_string(rc)} ({rc})")


def _ptr(t: torch.Tensor | None, dtype=None, name="tensor", shape=None) -> int | None:
    """Device address of t after checking where it lives, its layout, dtype
    and, given `shape` (None entries match any size), its shape, so that no
    call hands the library a buffer smaller than the sizes it is told."""
    if t is None:
        return None
    if not t.is_cuda:
        raise DsaError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise DsaError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise DsaError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and (t.dim() != len(shape) or
                              any(w is not None and int(d) != int(w) for d, w in zip(t.shape, shape))):
        raise DsaError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t.data_ptr()


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


_FP8 = (torch.uint8, torch.float8_e4m3fn)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def new_status(device=None) -> torch.Tensor:
    return torch.zeros(1, dtype=torch.int32, device=device or "cuda")


def check_status(status: torch.Tensor):
    """Raise DsaError if any kernel ORed a fault bit into ``status`` (syncs)."""
    v = int(status.item())
    if v:
        names = [n for b, n in DEV_BITS.items() if v & b]
        raise DsaError(f"device status {v:#x}: {', '.join(names)}")


def quantize_q(q_bf16, q_code=None, q_scale=None, stream=None):
    """bf16 [R, H, 128] -> (fp8 codes uint8 [R, H, 128], scales f32 [R, H])."""
    r, h, d = q_bf16.shape
    if q_code is None:
        q_code = torch.empty((r, h, d), dtype=torch.uint8, device=q_bf16.device)
    if q_scale is None:
        q_scale = torch.empty((r, h), dtype=torch.float32, device=q_bf16.device)
    _check(lib().dsa_quantize_q(_ptr(q_bf16, _BF16, "q_bf16"), r, h, d, _ptr(q_code, _FP8, "q_code", (r, h, d)),
                                _ptr(q_scale, torch.float32, "q_scale", (r, h)), _stream(stream)),
           "dsa_quantize_q")
    return q_code, q_scale


def index_scores(q, head_w, k_code, k_scale, page_table, kv_lens, row_req, row_vis,
                 group_rows: int = 1, score_stride: int | None = None, scores=None, status=None,
                 stream=None, whole_rows: bool = False):
    """fp8 indexer scores [R, score_stride] f32 (-inf past each row's span) of
    the bf16 queries q [R, 64, 128] (quantized in the kernel as quantize_q does).
    whole_rows: the caller's word that every row spans at least 3/4 of
    score_stride (one row a group); the keys are then read whole-row with the
    non-temporal hint.  Same scores either way."""
    r, h, d = q.shape
    n_pages, p, dk = k_code.shape
    batch, max_pages = page_table.shape
    if score_stride is None:
        score_stride = scores.shape[1] if scores is not None else max_pages * p
    if scores is None:
        scores = torch.empty((r, score_stride), dtype=torch.float32, device=q.device)
    if status is None:
        status = new_status(q.device)
    _check(lib().dsa_index_scores(
        _ptr(q, _BF16, "q"), _ptr(head_w, torch.float32, "head_w", (r, h)), _ptr(k_code, _FP8, "k_code"),
        _ptr(k_scale, torch.float32, "k_scale", (n_pages, p)), _ptr(page_table, torch.int32, "page_table"),
        _ptr(kv_lens, torch.int32, "kv_lens", (batch,)), _ptr(row_req, torch.int32, "row_req", (r,)),
        _ptr(row_vis, torch.int32, "row_vis", (r,)), r, batch, n_pages, max_pages, p, h, d, group_rows,
        1 if whole_rows else 0, _ptr(scores, torch.float32, "scores", (r, score_stride)), score_stride,
        _ptr(status, torch.int32, "status", (None,)), _stream(stream)), "dsa_index_scores")
    return scores, status


def index_topk_workspace_size(n_rows: int, score_stride: int, top_k: int) -> int:
    return int(lib().dsa_index_topk_workspace_size(n_rows, score_stride, top_k))


def index_topk(q, head_w, k_code, k_scale, page_table, kv_lens, row_req, row_vis, top_k: int,
               score_stride: int | None = None, scores=None, workspace=None, topk_idx=None, topk_count=None,
               status=None, stream=None, phases: int = 3):
    """Decode rows' indexer scores and their exact top-k in one call
    (dsa_index_topk) -> (scores, topk_idx, topk_count, status), the same
    results as index_scores (one row a group) followed by topk.  phases:
    PHASE_SCORE | PHASE_SELECT (both), or one of them on its own."""
    r, h, d = q.shape
    n_pages, p, dk = k_code.shape
    batch, max_pages = page_table.shape
    dev = q.device
    if score_stride is None:
        score_stride = scores.shape[1] if scores is not None else max_pages * p
    if scores is None:
        scores = torch.empty((r, score_stride), dtype=torch.float32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((r, top_k), dtype=torch.int32, device=dev)
    if topk_count is None:
        topk_count = torch.empty((r,), dtype=torch.int32, device=dev)
    if status is None:
        status = new_status(dev)
    if workspace is None:
        workspace = torch.empty((max(index_topk_workspace_size(r, score_stride, top_k), 1),),
                                dtype=torch.uint8, device=dev)
    _check(lib().dsa_index_topk(
        _ptr(q, _BF16, "q"), _ptr(head_w, torch.float32, "head_w", (r, h)), _ptr(k_code, _FP8, "k_code"),
        _ptr(k_scale, torch.float32, "k_scale", (n_pages, p)), _ptr(page_table, torch.int32, "page_table"),
        _ptr(kv_lens, torch.int32, "kv_lens", (batch,)), _ptr(row_req, torch.int32, "row_req", (r,)),
        _ptr(row_vis, torch.int32, "row_vis", (r,)), r, batch, n_pages, max_pages, p, h, d,
        _ptr(scores, torch.float32, "scores", (r, score_stride)), score_stride, top_k, phases,
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _ptr(topk_idx, torch.int32, "topk_idx", (r, top_k)), _ptr(topk_count, torch.int32, "topk_count", (r,)),
        _ptr(status, torch.int32, "status", (None,)), _stream(stream)),
        "dsa_index_topk")
    return scores, topk_idx, topk_count, status


def topk_workspace_size(n_rows: int, top_k: int, n_splits: int) -> int:
    return int(lib().dsa_topk_workspace_size(n_rows, top_k, n_splits))


def topk(scores, row_vis, top_k: int, n_splits: int = 1, workspace=None, topk_idx=None,
         topk_count=None, status=None, stream=None):
    """Exact top-k per row -> (topk_idx i32 [R, k] ascending then -1, topk_count i32 [R])."""
    r, stride = scores.shape
    dev = scores.device
    if topk_idx is None:
        topk_idx = torch.empty((r, top_k), dtype=torch.int32, device=dev)
    if topk_count is None:
        topk_count = torch.empty((r,), dtype=torch.int32, device=dev)
    if status is None:
        status = new_status(dev)
    need = topk_workspace_size(r, top_k, n_splits)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_ptr = _ptr(workspace, None, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dsa_topk(_ptr(scores, torch.float32, "scores"), stride,
                          _ptr(row_vis, torch.int32, "row_vis", (r,)), r, top_k, n_splits, ws_ptr, ws_bytes,
                          _ptr(topk_idx, torch.int32, "topk_idx", (r, top_k)),
                          _ptr(topk_count, torch.int32, "topk_count", (r,)),
                          _ptr(status, torch.int32, "status", (None,)), _stream(stream)), "dsa_topk")
    return topk_idx, topk_count, status


def topk_rows(scores, row_vis, row_req, page_table, num_pages: int, page_size: int, top_k: int,
              n_splits: int = 1, workspace=None, topk_idx=None, topk_count=None, topk_rows=None, status=None,
              stream=None):
    """topk() that also returns each selected slot's physical row in the paged
    caches (dsa_topk_rows) -> (topk_idx, topk_count, topk_rows, status)."""
    r, stride = scores.shape
    dev = scores.device
    batch, max_pages = page_table.shape
    if topk_idx is None:
        topk_idx = torch.empty((r, top_k), dtype=torch.int32, device=dev)
    if topk_count is None:
        topk_count = torch.empty((r,), dtype=torch.int32, device=dev)
    if topk_rows is None:
        topk_rows = torch.empty((r, top_k), dtype=torch.int32, device=dev)
    if status is None:
        status = new_status(dev)
    need = topk_workspace_size(r, top_k, n_splits)
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
    ws_ptr = _ptr(workspace, None, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().dsa_topk_rows(_ptr(scores, torch.float32, "scores"), stride,
                               _ptr(row_vis, torch.int32, "row_vis", (r,)),
                               _ptr(row_req, torch.int32, "row_req", (r,)),
                               _ptr(page_table, torch.int32, "page_table"), batch, num_pages, max_pages, page_size,
                               r, top_k, n_splits, ws_ptr, ws_bytes,
                               _ptr(topk_idx, torch.int32, "topk_idx", (r, top_k)),
                               _ptr(topk_count, torch.int32, "topk_count", (r,)),
                               _ptr(topk_rows, torch.int32, "topk_rows", (r, top_k)),
                               _ptr(status, torch.int32, "status", (None,)), _stream(stream)), "dsa_topk_rows")
    return topk_idx, topk_count, topk_rows, status


def topk_noalloc(scores, row_vis, top_k: int, n_splits: int = 1, topk_idx=None, topk_count=None,
                 status=None, stream=None):
    """topk() with the candidates in the library's fixed device array instead
    of a workspace (dsa_topk_noalloc); the same results."""
    r, stride = scores.shape
    dev = scores.device
    if topk_idx is None:
        topk_idx = torch.empty((r, top_k), dtype=torch.int32, device=dev)
    if topk_count is None:
        topk_count = torch.empty((r,), dtype=torch.int32, device=dev)
    if status is None:
        status = new_status(dev)
    _check(lib().dsa_topk_noalloc(_ptr(scores, torch.float32, "scores"), stride,
                                  _ptr(row_vis, torch.int32, "row_vis", (r,)), r, top_k, n_splits,
                                  _ptr(topk_idx, torch.int32, "topk_idx", (r, top_k)),
                                  _ptr(topk_count, torch.int32, "topk_count", (r,)),
                                  _ptr(status, torch.int32, "status", (None,)), _stream(stream)), "dsa_topk_noalloc")
    return topk_idx, topk_count, status


def sparse_mla_decode(q, kv_cache, page_table, row_req, row_vis, topk_idx, topk_count,
                      n_splits: int = 1, sm_scale: float = 1.0 / 24.0, part_o=None, part_lse=None,
                      out=None, out_lse=None, status=None, stream=None):
    """Split-K sparse MLA of the bf16 query q [R, H, 576].  n_splits == 1 -> (out bf16 [R,H,512], out_lse f32
    [R,H]); otherwise -> (part_o bf16 [R,H,S,512], part_lse f32 [R,H,S]).
    kv_cache is the packed uint8 [NP, P, 640] MLA cache (codes, fp32 scale at
    byte 576, pad)."""
    r, h, dq = q.shape
    if dq != 576:
        raise DsaError(f"q heads must hold 576 values (512 latent + 64 rope), got {dq}")
    n_pages, p, row_bytes = kv_cache.shape
    if row_bytes != 640:
        raise DsaError(f"kv_cache rows must be 640 bytes, got {row_bytes}")
    batch, max_pages = page_table.shape
    top_k = topk_idx.shape[1]
    dev = q.device
    if status is None:
        status = new_status(dev)
    if n_splits == 1:
        if out is None:
            out = torch.empty((r, h, 512), dtype=torch.bfloat16, device=dev)
        if out_lse is None:
            out_lse = torch.empty((r, h), dtype=torch.float32, device=dev)
    else:
        if part_o is None:
            part_o = torch.empty((r, h, n_splits, 512), dtype=torch.bfloat16, device=dev)
        if part_lse is None:
            part_lse = torch.empty((r, h, n_splits), dtype=torch.float32, device=dev)
    _check(lib().dsa_sparse_mla_decode(
        _ptr(q, _BF16, "q"), _ptr(kv_cache, torch.uint8, "kv_cache"),
        _ptr(page_table, torch.int32, "page_table"), _ptr(row_req, torch.int32, "row_req", (r,)),
        _ptr(row_vis, torch.int32, "row_vis", (r,)), _ptr(topk_idx, torch.int32, "topk_idx", (r, top_k)),
        _ptr(topk_count, torch.int32, "topk_count", (r,)), r, batch, n_pages, max_pages, p, h, top_k,
        n_splits, float(sm_scale),
        _ptr(part_o, torch.bfloat16, "part_o", (r, h, n_splits, 512)) if n_splits > 1 else None,
        _ptr(part_lse, torch.float32, "part_lse", (r, h, n_splits)) if n_splits > 1 else None,
        _ptr(out, _BF16, "out", (r, h, 512)) if n_splits == 1 else None,
        _ptr(out_lse, torch.float32, "out_lse", (r, h)) if n_splits == 1 else None,
        _ptr(status, torch.int32, "status", (None,)), _stream(stream)), "dsa_sparse_mla_decode")
    if n_splits == 1:
        return out, out_lse, status
    return part_o, part_lse, status


def sparse_mla_decode_rows(q, kv_cache, row_vis, topk_rows, topk_count, n_splits: int, sm_scale: float,
                           part_o=None, part_lse=None, out=None, out_lse=None, status=None, stream=None):
    """sparse_mla_decode over physical rows (dsa_sparse_mla_decode_rows); the
    same returns."""
    r, h, dq = q.shape
    if dq != 576:
        raise DsaError(f"q heads must hold 576 values (512 latent + 64 rope), got {dq}")
    n_pages, p, row_bytes = kv_cache.shape
    if row_bytes != 640:
        raise DsaError(f"kv_cache rows must be 640 bytes, got {row_bytes}")
    top_k = topk_rows.shape[1]
    dev = q.device
    if status is None:
        status = new_status(dev)
    if n_splits == 1:
        if out is None:
            out = torch.empty((r, h, 512), dtype=torch.bfloat16, device=dev)
        if out_lse is None:
            out_lse = torch.empty((r, h), dtype=torch.float32, device=dev)
    else:
        if part_o is None:
            part_o = torch.empty((r, h, n_splits, 512), dtype=torch.bfloat16, device=dev)
        if part_lse is None:
            part_lse = torch.empty((r, h, n_splits), dtype=torch.float32, device=dev)
    _check(lib().dsa_sparse_mla_decode_rows(
        _ptr(q, _BF16, "q"), _ptr(kv_cache, torch.uint8, "kv_cache"), _ptr(row_vis, torch.int32, "row_vis", (r,)),
        _ptr(topk_rows, torch.int32, "topk_rows", (r, top_k)), _ptr(topk_count, torch.int32, "topk_count", (r,)),
        r, n_pages, p, h,
        top_k, n_splits, float(sm_scale),
        _ptr(part_o, torch.bfloat16, "part_o", (r, h, n_splits, 512)) if n_splits > 1 else None,
        _ptr(part_lse, torch.float32, "part_lse", (r, h, n_splits)) if n_splits > 1 else None,
        _ptr(out, _BF16, "out", (r, h, 512)) if n_splits == 1 else None,
        _ptr(out_lse, torch.float32, "out_lse", (r, h)) if n_splits == 1 else None,
        _ptr(status, torch.int32, "status", (None,)), _stream(stream)), "dsa_sparse_mla_decode_rows")
    if n_splits == 1:
        return out, out_lse, status
    return part_o, part_lse, status


def sparse_mla_decode_shared(q, kv_cache, page_table, row_req, row_vis, row_list, topk_idx, topk_count,
                             n_splits: int = 1, sm_scale: float = 1.0 / 24.0, part_o=None, part_lse=None,
                             out=None, out_lse=None, status=None, stream=None):
    """sparse_mla_decode where row r attends list row_list[r] of topk_idx
    [n_lists, k] / topk_count [n_lists] (MTP IndexShare).  Returns as
    sparse_mla_decode."""
    r, h, dq = q.shape
    if dq != 576:
        raise DsaError(f"q heads must hold 576 values (512 latent + 64 rope), got {dq}")
    n_pages, p, row_bytes = kv_cache.shape
    if row_bytes != 640:
        raise DsaError(f"kv_cache rows must be 640 bytes, got {row_bytes}")
    batch, max_pages = page_table.shape
    n_lists, top_k = topk_idx.shape
    dev = q.device
    if status is None:
        status = new_status(dev)
    if n_splits == 1:
        if out is None:
            out = torch.empty((r, h, 512), dtype=torch.bfloat16, device=dev)
        if out_lse is None:
            out_lse = torch.empty((r, h), dtype=torch.float32, device=dev)
    else:
        if part_o is None:
            part_o = torch.empty((r, h, n_splits, 512), dtype=torch.bfloat16, device=dev)
        if part_lse is None:
            part_lse = torch.empty((r, h, n_splits), dtype=torch.float32, device=dev)
    _check(lib().dsa_sparse_mla_decode_shared(
        _ptr(q, _BF16, "q"), _ptr(kv_cache, torch.uint8, "kv_cache"),
        _ptr(page_table, torch.int32, "page_table"), _ptr(row_req, torch.int32, "row_req", (r,)),
        _ptr(row_vis, torch.int32, "row_vis", (r,)), _ptr(row_list, torch.int32, "row_list", (r,)),
        _ptr(topk_idx, torch.int32, "topk_idx"), _ptr(topk_count, torch.int32, "topk_count", (n_lists,)), n_lists,
        r, batch, n_pages, max_pages, p, h, top_k, n_splits, float(sm_scale),
        _ptr(part_o, torch.bfloat16, "part_o", (r, h, n_splits, 512)) if n_splits > 1 else None,
        _ptr(part_lse, torch.float32, "part_lse", (r, h, n_splits)) if n_splits > 1 else None,
        _ptr(out, _BF16, "out", (r, h, 512)) if n_splits == 1 else None,
        _ptr(out_lse, torch.float32, "out_lse", (r, h)) if n_splits == 1 else None,
        _ptr(status, torch.int32, "status", (None,)), _stream(stream)), "dsa_sparse_mla_decode_shared")
    if n_splits == 1:
        return out, out_lse, status
    return part_o, part_lse, status


def lse_merge(part_o, part_lse, out=None, out_lse=None, stream=None):
    """Merge split partials -> (out bf16 [R,H,512], out_lse f32 [R,H])."""
    r, h, s, dv = part_o.shape
    dev = part_o.device
    if out is None:
        out = torch.empty((r, h, dv), dtype=torch.bfloat16, device=dev)
    if out_lse is None:
        out_lse = torch.empty((r, h), dtype=torch.float32, device=dev)
    _check(lib().dsa_lse_merge(_ptr(part_o, torch.bfloat16, "part_o"),
                               _ptr(part_lse, torch.float32, "part_lse", (r, h, s)), r, h, s, dv,
                               _ptr(out, _BF16, "out", (r, h, dv)), _ptr(out_lse, torch.float32, "out_lse", (r, h)),
                               _stream(stream)), "dsa_lse_merge")
    return out, out_lse


def lse_merge_project(part_o, part_lse, w_uv, out=None, out_lse=None, stream=None):
    """Merge split partials, then project with W_UV bf16 [H, 128, 512] ->
    (out bf16 [R, H, 128], out_lse f32 [R, H])."""
    r, h, s, dl = part_o.shape
    dv = w_uv.shape[1]
    dev = part_o.device
    if out is None:
        out = torch.empty((r, h, dv), dtype=torch.bfloat16, device=dev)
    if out_lse is None:
        out_lse = torch.empty((r, h), dtype=torch.float32, device=dev)
    _check(lib().dsa_lse_merge_project(_ptr(part_o, torch.bfloat16, "part_o"),
                                       _ptr(part_lse, torch.float32, "part_lse", (r, h, s)), r, h, s, dl,
                                       _ptr(w_uv, _BF16, "w_uv", (h, dv, dl)), dv, _ptr(out, _BF16, "out", (r, h, dv)),
                                       _ptr(out_lse, torch.float32, "out_lse", (r, h)), _stream(stream)),
           "dsa_lse_merge_project")
    return out, out_lse


def cache_write(latent, rope, index_k, tok_req, tok_slot, page_table, kv_cache, k_code, k_scale,
                rope_cos=None, rope_sin=None, status=None, stream=None):
    """New tokens into the paged caches, in place: latent bf16 [n, 512], rope
    bf16 [n, 64] (rotated by rope_cos / rope_sin f32 [max_pos, 32] at each
    token's slot, or stored as given), index_k bf16 [n, 128]; returns status."""
    n = latent.shape[0]
    n_pages, p, _ = kv_cache.shape
    batch, max_pages = page_table.shape
    if status is None:
        status = new_status(latent.device)
    max_pos = rope_cos.shape[0] if rope_cos is not None else 0
    _check(lib().dsa_cache_write(
        _ptr(latent, _BF16, "latent", (n, 512)), _ptr(rope, _BF16, "rope", (n, 64)),
        _ptr(index_k, _BF16, "index_k", (n, 128)),
        _ptr(rope_cos, torch.float32, "rope_cos", (max_pos, 32)),
        _ptr(rope_sin, torch.float32, "rope_sin", (max_pos, 32)), max_pos,
        _ptr(tok_req, torch.int32, "tok_req", (n,)), _ptr(tok_slot, torch.int32, "tok_slot", (n,)), n,
        _ptr(page_table, torch.int32, "page_table"), batch, n_pages, max_pages, p,
        _ptr(kv_cache, torch.uint8, "kv_cache", (n_pages, p, 640)), _ptr(k_code, _FP8, "k_code", (n_pages, p, 128)),
        _ptr(k_scale, torch.float32, "k_scale", (n_pages, p)), _ptr(status, torch.int32, "status", (None,)),
        _stream(stream)), "dsa_cache_write")
    return status


class DecodeStep:
    """All buffers of one DSA decode step for fixed inputs, allocated once;
    ``run()`` enqueues scores -> top-k -> sparse MLA -> merge on the given
    (else the current) stream without allocating or synchronising."""

    def __init__(self, inp, index_splits: int | None = None, attn_splits: int | None = None,
                 group_rows: int | None = None, score_stride: int | None = None,
                 index_share: int | None = None, index_topk: bool | None = None,
                 phys_rows: bool | None = None, whole_rows: bool = False):
        self.inp = inp
        cfg = inp.cfg
        self.index_splits = index_splits or cfg.index_splits
        self.attn_splits = attn_splits or cfg.attn_splits
        self.group_rows = group_rows or cfg.group_rows
        # index_topk: rows scored one at a time take scores and top-k in one
        # call (dsa_index_topk); the default is the configuration's (the two
        # calls, which measure as fast at the step level).
        if index_topk is None:
            index_topk = index_splits is None and cfg.index_topk
        self.index_topk = bool(index_topk) and self.group_rows == 1
        # phys_rows: the top-k also emits each selected slot's physical row
        # (dsa_topk_rows) and the attention gathers those rows directly
        # (dsa_sparse_mla_decode_rows); for rows that select their own lists
        # with dsa_topk.
        # MTP IndexShare: chains of `index_share` consecutive rows; only each
        # chain's first row is scored and selected, and every row attends
        # that list.  The first rows' inputs are gathered once, here.
        self.index_share = index_share if index_share is not None else cfg.index_share
        dev = inp.q_idx.device
        r = inp.n_rows
        h = inp.mla_heads
        k = inp.top_k
        if self.index_share > 1:
            c = self.index_share
            if r % c or self.group_rows != 1:
                raise DsaError("index sharing needs whole chains and one row per scoring group")
            self.lead_q = inp.q_idx[::c].contiguous()
            self.lead_w = inp.head_w[::c].contiguous()
            self.lead_req = inp.row_req[::c].contiguous()
            self.lead_vis = inp.row_vis[::c].contiguous()
            self.row_list = (torch.arange(r, device=dev, dtype=torch.int32) // c).contiguous()
        else:
            self.lead_q, self.lead_w, self.lead_req, self.lead_vis = inp.q_idx, inp.head_w, inp.row_req, inp.row_vis
            self.row_list = None
        n_sel = self.lead_q.shape[0]
        # Rows start 16-byte aligned (the top-k then reads them in 16-byte loads).
        self.score_stride = score_stride or max(64, (int(self.lead_vis.max()) + 63) // 64 * 64)
        # whole_rows (opt-in): the indexer's whole-row, non-temporal key loads,
        # taken only when every row spans at least 3/4 of the stride (lengths
        # known here, on the host).  Off by default: measured steps come out
        # from 3 us faster to 0.6 us slower depending on the box, and the
        # indexer alone is slower with them.
        self.whole_rows = (bool(whole_rows) and self.group_rows == 1 and n_sel > 0
                           and 4 * int(self.lead_vis.min()) >= 3 * self.score_stride)
        self.scores = torch.empty((n_sel, self.score_stride), dtype=torch.float32, device=dev)
        if self.index_topk:
            need = index_topk_workspace_size(n_sel, self.score_stride, k)
        else:
            need = topk_workspace_size(n_sel, k, self.index_splits)
        self.workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
        self.topk_idx = torch.empty((n_sel, k), dtype=torch.int32, device=dev)
        if phys_rows is None:
            phys_rows = cfg.phys_rows
        self.phys_rows = bool(phys_rows) and not self.index_topk and self.index_share <= 1
        self.topk_rows = torch.empty((n_sel, k), dtype=torch.int32, device=dev) if self.phys_rows else None
        self.topk_count = torch.empty((n_sel,), dtype=torch.int32, device=dev)
        s = self.attn_splits
        self.part_o = torch.empty((r, h, s, 512), dtype=torch.bfloat16, device=dev) if s > 1 else None
        self.part_lse = torch.empty((r, h, s), dtype=torch.float32, device=dev) if s > 1 else None
        self.out = torch.empty((r, h, 512), dtype=torch.bfloat16, device=dev)
        self.out_lse = torch.empty((r, h), dtype=torch.float32, device=dev)
        self.status = new_status(dev)

    def run(self, stream=None):
        i = self.inp
        if self.index_topk:
            index_topk(self.lead_q, self.lead_w, i.k_code, i.k_scale, i.page_table, i.kv_lens,
                       self.lead_req, self.lead_vis, i.top_k, score_stride=self.score_stride,
                       scores=self.scores, workspace=self.workspace, topk_idx=self.topk_idx,
                       topk_count=self.topk_count, status=self.status, stream=stream)
        else:
            index_scores(self.lead_q, self.lead_w, i.k_code, i.k_scale, i.page_table,
                         i.kv_lens, self.lead_req, self.lead_vis, group_rows=self.group_rows,
                         score_stride=self.score_stride, scores=self.scores, status=self.status,
                         stream=stream, whole_rows=self.whole_rows)
            if self.phys_rows:
                topk_rows(self.scores, self.lead_vis, self.lead_req, i.page_table, i.kv_cache.shape[0],
                          i.kv_cache.shape[1], i.top_k, self.index_splits, workspace=self.workspace,
                          topk_idx=self.topk_idx, topk_count=self.topk_count, topk_rows=self.topk_rows,
                          status=self.status, stream=stream)
            else:
                topk(self.scores, self.lead_vis, i.top_k, self.index_splits, workspace=self.workspace,
                     topk_idx=self.topk_idx, topk_count=self.topk_count, status=self.status, stream=stream)
        if self.row_list is not None:
            s = self.attn_splits
            sparse_mla_decode_shared(i.q_mla, i.kv_cache, i.page_table, i.row_req, i.row_vis,
                                           self.row_list, self.topk_idx, self.topk_count, s, i.sm_scale,
                                           part_o=self.part_o, part_lse=self.part_lse, out=self.out,
                                           out_lse=self.out_lse, status=self.status, stream=stream)
            if s > 1:
                lse_merge(self.part_o, self.part_lse, out=self.out, out_lse=self.out_lse, stream=stream)
            return self.out, self.out_lse
        if self.phys_rows:
            s = self.attn_splits
            sparse_mla_decode_rows(i.q_mla, i.kv_cache, i.row_vis, self.topk_rows, self.topk_count, s, i.sm_scale,
                                   part_o=self.part_o, part_lse=self.part_lse, out=self.out, out_lse=self.out_lse,
                                   status=self.status, stream=stream)
            if s > 1:
                lse_merge(self.part_o, self.part_lse, out=self.out, out_lse=self.out_lse, stream=stream)
        elif self.attn_splits == 1:
            sparse_mla_decode(i.q_mla, i.kv_cache, i.page_table, i.row_req,
                              i.row_vis, self.topk_idx, self.topk_count, 1, i.sm_scale, out=self.out,
                              out_lse=self.out_lse, status=self.status, stream=stream)
        else:
            sparse_mla_decode(i.q_mla, i.kv_cache, i.page_table, i.row_req,
                              i.row_vis, self.topk_idx, self.topk_count, self.attn_splits, i.sm_scale,
                              part_o=self.part_o, part_lse=self.part_lse, status=self.status,
                              stream=stream)
            lse_merge(self.part_o, self.part_lse, out=self.out, out_lse=self.out_lse, stream=stream)
        return self.out, self.out_lse
