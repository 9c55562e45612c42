"""Plain, slow, fp64 CPU oracle for one DSA sparse decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (its own fp8 and bf16 decoders, no torch in any computation) and it
imports nothing from the product package.

What it computes, and where the pages state it.  Page "[ROCm] Support decode
context parallel (DCP) for GLM-5 / DeepSeek-V3.2" (sgl-project/sglang PR
#42618) is the subject:

* Motivation: DSA keeps the 2048 highest-scoring tokens of the whole sequence
  before attention runs.
* Modifications, "Indexer decode": an fp8 index key per cached token is scored
  and a local top-k is taken per shard; the shards' candidates are merged into
  the exact global top-k.  Here the shards are contiguous splits of one row.
* Modifications, "Sparse decode" and the split-K commit note: attention runs
  only over the selected slots, split along the selected list, each split
  returning a partial output and a natural-log LSE; the partials are merged by
  LSE; with a single split the partial already is the result.
* Page "DeepSeek V4 DSpark Internals" (pypto.ai), kernel mapping: block tables
  hold -1 past each request's span.
* The step before the path, the cache write: Modifications ("Writes", and the
  fused rope + KV-cache write named under "Disabled under DCP") and Future
  work (the write location computed once per step and fused into the write
  kernels).  New tokens' MLA rows (rope part rotated) and index keys are
  quantized to fp8 with one fp32 scale per token and stored at their slots.
* The step after the path: Future work, projecting V (W_UV) before the LSE
  merge; here the merge is followed by the projection, which is the same
  linear map applied once.
* MTP IndexShare: Modifications, "MTP / EAGLE", and the chain-EAGLE commit
  note name an option that shares the index across MTP iterations; read here
  as one top-k list, selected for a chain's first draft row, attended by every
  row of the chain (``decode_step_index_share``).

The pages never print the formulas.  The readings taken here are the plainest
ones consistent with the configurations: indexer score
``s_t = sum_h w_h * relu(q_h . k_t)`` with one 128-wide key per token shared by
all heads; absorbed MLA with keys = the 576-wide latent+rope row and values =
its first 512 entries; logits scaled by ``sm_scale``; everything decoded from
fp8 E4M3FN codes times one fp32 scale per token.

Every function below states in its docstring which of these it follows.  The
functions that have no independent pin are marked "parity unpinned"; at present
none is.
"""

from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------------------
# Number formats
# ---------------------------------------------------------------------------

FP8_MAX = 448.0  # largest finite E4M3FN value: S.1111.110 = 1.75 * 2^8


def fp8_e4m3fn_decode(codes) -> np.ndarray:
    """Decode OCP FP8 E4M3FN codes to float64 from the format's definition.

    Layout: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits.  Exponent
    field 0 is subnormal, value (m/8) * 2^-6.  Otherwise (1 + m/8) * 2^(e-7).
    There is no infinity; S.1111.111 is NaN, which no valid cache holds, so it
    is rejected.  (The configurations name ``fp8_e4m3``; on gfx950 that is the
    OCP "FN" variant, not the FNUZ one.)
    """
    c = np.asarray(codes, dtype=np.uint8)
    if np.any((c & 0x7F) == 0x7F):
        raise ValueError("E4M3FN NaN code in fp8 input")
    sign = (c >> 7).astype(np.int64)
    exp = ((c >> 3) & 0xF).astype(np.int64)
    man = (c & 0x7).astype(np.float64)
    sub = man / 8.0 * 2.0 ** -6
    norm = (1.0 + man / 8.0) * np.exp2((exp - 7).astype(np.float64))
    mag = np.where(exp == 0, sub, norm)
    return np.where(sign == 1, -mag, mag)


def bf16_decode(bits) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64: they are the top 16
    bits of an IEEE binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _e4m3fn_grid() -> np.ndarray:
    """The 127 non-negative finite E4M3FN values, indexed by their code."""
    return fp8_e4m3fn_decode(np.arange(0, 127, dtype=np.uint8))


def fp8_e4m3fn_encode_rne(x) -> np.ndarray:
    """Round float64 values with |x| <= 448 to the nearest E4M3FN code, ties
    to the code with an even mantissa (round-to-nearest-even).  The sign bit
    follows the IEEE sign of x, so -0.0 and tiny negatives give code 0x80."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(~np.isfinite(x)) or np.any(np.abs(x) > FP8_MAX):
        raise ValueError("value outside the E4M3FN finite range")
    grid = _e4m3fn_grid()
    a = np.abs(x)
    hi = np.searchsorted(grid, a, side="left")  # first grid value >= a
    hi = np.minimum(hi, len(grid) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    mag = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), mag | np.uint8(0x80), mag).astype(np.uint8)


# ---------------------------------------------------------------------------
# Indexer query quantization (input side of the fp8 indexer)
# ---------------------------------------------------------------------------


def quantize_q(q_bf16_bits) -> tuple[np.ndarray, np.ndarray]:
    """Quantize the bf16 indexer queries to fp8 E4M3FN codes with one
    power-of-two fp32 scale per (row, head).

    The indexer of the subject page is an fp8 indexer and the configurations
    give the query as bf16, so the query is brought to fp8 before the fp8
    contraction.  Reading used here: scale = 2^ceil(log2(amax / 448)), a power
    of two so that q / scale is exact, then round-to-nearest-even onto the
    E4M3FN grid; an all-zero head gets scale 1.

    Input: uint16 [R, Hi, Di].  Returns (codes uint8 [R, Hi, Di],
    scale float64 [R, Hi]).
    """
    q = bf16_decode(q_bf16_bits)
    amax = np.max(np.abs(q), axis=-1)
    scale = np.ones_like(amax)
    nz = amax > 0
    # amax / 448 is a ratio of an 8-bit significand and 7*2^6; it is exact when
    # it is a power of two and at least 2^-8 relative away from one otherwise,
    # so log2 followed by ceil lands on the right integer in float64.
    scale[nz] = np.exp2(np.ceil(np.log2(amax[nz] / FP8_MAX)))
    codes = fp8_e4m3fn_encode_rne(q / scale[..., None])
    return codes, scale


# ---------------------------------------------------------------------------
# Cache write (the step before the path: new tokens into the paged caches)
# ---------------------------------------------------------------------------

D_LATENT_W = 512   # latent entries of an MLA row
D_ROPE_W = 64      # rope entries of an MLA row, rotated before they are stored
D_INDEX_W = 128    # entries of an index key
KV_ROW_BYTES_W = 640   # bytes of an MLA cache row: 576 codes, fp32 scale at 576, pad


def rope_interleaved_f32(rope_bits, cos, sin, pos) -> np.ndarray:
    """Rotary embedding of the rope part of new MLA rows, in float32.

    The page "[ROCm] Support decode context parallel (DCP) for GLM-5 /
    DeepSeek-V3.2" names a fused rope + KV-cache write (Modifications,
    "Disabled under DCP") but not the rotation.  Reading taken here: the 64
    rope entries form 32 pairs (2j, 2j+1), and pair j of a token at position
    p is turned by the angle whose cosine and sine the caller tabulates at
    cos[p, j], sin[p, j]:
        y[2j]   = x[2j] * c - x[2j+1] * s
        y[2j+1] = x[2j] * s + x[2j+1] * c
    each product rounded to float32, then the sum or difference (no fused
    multiply-add), which fixes every bit of the result.  The position of a
    token is the slot it is written to.

    rope_bits uint16 [n, 64] bf16; cos, sin float32 [max_pos, 32]; pos [n].
    Returns float32 [n, 64].
    """
    x = bf16_decode(rope_bits).astype(np.float32)
    pos = np.asarray(pos, dtype=np.int64)
    c = np.asarray(cos, dtype=np.float32)[pos]
    s = np.asarray(sin, dtype=np.float32)[pos]
    x0, x1 = x[:, 0::2], x[:, 1::2]
    y = np.empty_like(x)
    y[:, 0::2] = (x0 * c) - (x1 * s)
    y[:, 1::2] = (x0 * s) + (x1 * c)
    return y


def quantize_rows_f32(v) -> tuple[np.ndarray, np.ndarray]:
    """E4M3FN codes and one fp32 scale per row, the rule the caches are
    written with: scale = max|x| / 448 (1 for an all-zero row) and
    code = RNE(clamp(x / scale, -448, 448)), the division and the scale in
    float32, so that the decision of every code is taken in float32.

    The pages fix only "fp8 rows with an fp32 scale per token"; max|x| / 448
    is the plainest scale that uses the format's whole range.
    v float32 [n, d].  Returns (codes uint8 [n, d], scale float32 [n]).
    """
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v), axis=1)
    scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(v / scale[:, None], np.float32(-FP8_MAX), np.float32(FP8_MAX))
    return fp8_e4m3fn_encode_rne(y.astype(np.float64)), scale


def cache_write(latent_bits, rope_bits, index_bits, cos, sin, tok_req, tok_slot, page_table,
                page_size: int, kv_cache, k_code, k_scale):
    """Write new tokens into the paged caches.

    Token i belongs to request tok_req[i] and is stored at logical slot
    tok_slot[i] (its position): physical row page_table[b][t / P] * P + t % P
    (page "DeepSeek V4 DSpark Internals", kernel mapping).  Its MLA row is
    the 512 latent entries followed by the 64 rope entries rotated as in
    rope_interleaved_f32 (no rotation when cos is None), quantized as in
    quantize_rows_f32 into bytes 0..575 of the row with the scale at bytes
    576..579; bytes 580..639 are left as they are.  Its 128-entry index key
    is quantized the same way into k_code / k_scale, unrotated (the pages say
    nothing of a rotation of the index key; a caller rotates it beforehand).
    A token whose request, slot or page id is out of range, or whose position
    lies past the rotation tables, writes nothing.

    Inputs are not modified.  Returns (kv_cache, k_code, k_scale, written)
    with written bool [n].
    """
    latent_bits = np.asarray(latent_bits, dtype=np.uint16)
    rope_bits = np.asarray(rope_bits, dtype=np.uint16)
    index_bits = np.asarray(index_bits, dtype=np.uint16)
    tok_req = np.asarray(tok_req, dtype=np.int64)
    tok_slot = np.asarray(tok_slot, dtype=np.int64)
    page_table = np.asarray(page_table, dtype=np.int64)
    kv = np.array(kv_cache, dtype=np.uint8, copy=True)
    kc = np.array(k_code, dtype=np.uint8, copy=True)
    ks = np.array(k_scale, dtype=np.float32, copy=True)
    n_pages = kv.shape[0]
    batch, max_pages = page_table.shape
    n = len(tok_req)
    written = np.zeros(n, dtype=bool)
    if n == 0:
        return kv, kc, ks, written
    if cos is None:
        rope = bf16_decode(rope_bits).astype(np.float32)
    else:
        pos = np.clip(tok_slot, 0, np.asarray(cos).shape[0] - 1)
        rope = rope_interleaved_f32(rope_bits, cos, sin, pos)
    mla = np.concatenate([bf16_decode(latent_bits).astype(np.float32), rope], axis=1)
    mla_codes, mla_scale = quantize_rows_f32(mla)
    idx_codes, idx_scale = quantize_rows_f32(bf16_decode(index_bits).astype(np.float32))
    for i in range(n):
        b, t = int(tok_req[i]), int(tok_slot[i])
        if not (0 <= b < batch and 0 <= t < max_pages * page_size):
            continue
        if cos is not None and t >= np.asarray(cos).shape[0]:
            continue
        page = int(page_table[b, t // page_size])
        if not (0 <= page < n_pages):
            continue
        off = t % page_size
        kv[page, off, :D_LATENT_W + D_ROPE_W] = mla_codes[i]
        kv[page, off, D_LATENT_W + D_ROPE_W:D_LATENT_W + D_ROPE_W + 4] = \
            np.frombuffer(np.float32(mla_scale[i]).tobytes(), dtype=np.uint8)
        kc[page, off] = idx_codes[i]
        ks[page, off] = idx_scale[i]
        written[i] = True
    return kv, kc, ks, written


# ---------------------------------------------------------------------------
# Paged addressing
# ---------------------------------------------------------------------------


def physical_rows(page_table_row, n_slots: int, page_size: int, n_pages: int) -> np.ndarray:
    """Map logical slots 0..n_slots-1 of one request to flat physical rows
    ``page * page_size + slot % page_size`` through its block table.

    Entries past the request's span are -1 (page "DeepSeek V4 DSpark
    Internals", kernel mapping); a slot inside the span must land on a valid
    page, which is asserted.
    """
    t = np.arange(n_slots, dtype=np.int64)
    pages = np.asarray(page_table_row, dtype=np.int64)[t // page_size]
    if np.any(pages < 0) or np.any(pages >= n_pages):
        raise ValueError("slot inside the span maps to an invalid page")
    return pages * page_size + t % page_size


def _check_rows(row_req, row_vis, kv_lens, max_pages, page_size):
    row_req = np.asarray(row_req, dtype=np.int64)
    row_vis = np.asarray(row_vis, dtype=np.int64)
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    if np.any(row_vis < 0) or np.any(row_vis > kv_lens[row_req]):
        raise ValueError("row_vis must lie in [0, kv_len of its request]")
    if np.any(kv_lens > max_pages * page_size):
        raise ValueError("kv_len exceeds the block table")
    return row_req, row_vis


# ---------------------------------------------------------------------------
# Indexer scores
# ---------------------------------------------------------------------------


def index_scores(q_code, q_scale, head_w, k_code, k_scale, page_table, kv_lens,
                 row_req, row_vis, page_size: int, score_len: int) -> np.ndarray:
    """Lightning-indexer scores for every visible slot of every query row.

    Follows the subject page's "Indexer decode" modification (score the cached
    index keys), under the reading ``s_t = sum_h w[r,h] * relu(q_h . k_t)``:
    k_t = dec(k_code[t]) * k_scale[t] (one key and one scale per token, shared
    by all heads), q_h = dec(q_code[r,h]) * q_scale[r,h].  Literal order:
    dequantize, dot, ReLU, weight, sum.  Slots t >= row_vis[r] score -inf.

    Shapes: q_code uint8 [R,Hi,Di], q_scale [R,Hi], head_w [R,Hi],
    k_code uint8 [NP,P,Di], k_scale [NP,P], page_table int [B,max_pages].
    Returns float64 [R, score_len].
    """
    q_code = np.asarray(q_code)
    k_code = np.asarray(k_code)
    n_pages = k_code.shape[0]
    di = k_code.shape[-1]
    page_table = np.asarray(page_table)
    row_req, row_vis = _check_rows(row_req, row_vis, kv_lens, page_table.shape[1], page_size)
    k_flat = k_code.reshape(-1, di)
    ks_flat = np.asarray(k_scale, dtype=np.float64).reshape(-1)
    w = np.asarray(head_w, dtype=np.float64)
    qs = np.asarray(q_scale, dtype=np.float64)
    out = np.full((q_code.shape[0], score_len), -np.inf)
    for r in range(q_code.shape[0]):
        v = int(row_vis[r])
        if v == 0:
            continue
        if v > score_len:
            raise ValueError("score_len shorter than a row's visible span")
        phys = physical_rows(page_table[row_req[r]], v, page_size, n_pages)
        keys = fp8_e4m3fn_decode(k_flat[phys]) * ks_flat[phys][:, None]   # [V, Di]
        q = fp8_e4m3fn_decode(q_code[r]) * qs[r][:, None]                 # [Hi, Di]
        dots = q @ keys.T                                                 # [Hi, V]
        out[r, :v] = w[r] @ np.maximum(dots, 0.0)
    return out


# ---------------------------------------------------------------------------
# Top-k selection
# ---------------------------------------------------------------------------


def _order_desc_slot_asc(scores: np.ndarray, slots: np.ndarray) -> np.ndarray:
    """Positions sorted by (score descending, slot ascending): the total order
    used for selection, so equal scores keep the lower slot."""
    return np.lexsort((slots, -scores))


def topk_global(scores_row, n_vis: int, top_k: int) -> tuple[np.ndarray, int]:
    """Exact top-k of slots 0..n_vis-1 of one row under (score desc, slot asc).

    Subject page, Motivation: DSA keeps the top 2048 tokens of the whole
    sequence; a row shorter than k keeps every slot.  Output: int64 [top_k],
    the selected slots in ascending order followed by -1, and the count
    min(top_k, n_vis).
    """
    s = np.asarray(scores_row, dtype=np.float64)[:n_vis]
    if np.any(np.isnan(s)):
        raise ValueError("NaN score")
    slots = np.arange(n_vis, dtype=np.int64)
    count = min(top_k, n_vis)
    chosen = np.sort(slots[_order_desc_slot_asc(s, slots)[:count]])
    out = np.full(top_k, -1, dtype=np.int64)
    out[:count] = chosen
    return out, count


def split_ranges(n: int, n_splits: int) -> list[tuple[int, int]]:
    """Contiguous equal chunks [j*c, min(n, (j+1)*c)) with c = ceil(n/n_splits);
    trailing chunks may be empty."""
    c = -(-n // n_splits) if n > 0 else 0
    return [(min(n, j * c), min(n, (j + 1) * c)) for j in range(n_splits)]


def topk_split_merge(scores_row, n_vis: int, top_k: int, n_splits: int) -> tuple[np.ndarray, int]:
    """Top-k by local selection per split followed by an exact merge.

    Subject page, "Indexer decode": every shard keeps its own top-k and the
    gathered candidates are merged into the exact global top-k.  Here the
    shards are ``n_splits`` contiguous slot ranges of one row.  Each split
    keeps its top-min(k, len) under (score desc, slot asc); the union is then
    cut to the top-k under the same order.  Output as :func:`topk_global`.
    """
    s = np.asarray(scores_row, dtype=np.float64)[:n_vis]
    cand_slots = []
    for lo, hi in split_ranges(n_vis, n_splits):
        if hi <= lo:
            continue
        slots = np.arange(lo, hi, dtype=np.int64)
        keep = _order_desc_slot_asc(s[lo:hi], slots)[: min(top_k, hi - lo)]
        cand_slots.append(slots[keep])
    if not cand_slots:
        return np.full(top_k, -1, dtype=np.int64), 0
    cs = np.concatenate(cand_slots)
    count = min(top_k, len(cs))
    chosen = np.sort(cs[_order_desc_slot_asc(s[cs], cs)[:count]])
    out = np.full(top_k, -1, dtype=np.int64)
    out[:count] = chosen
    return out, count


# ---------------------------------------------------------------------------
# Sparse absorbed-MLA attention, split along the selected list, and LSE merge
# ---------------------------------------------------------------------------

D_LATENT = 512
D_ROPE = 64
D_QK = D_LATENT + D_ROPE


def attend_split(q_row, x_rows, sm_scale: float) -> tuple[np.ndarray, np.ndarray]:
    """Softmax attention of H query heads over n gathered rows, returning the
    normalised partial output and its natural-log LSE.

    Subject page, "Sparse decode" and the split-K commit note: each split
    returns its output and the LSE of its logits, natural log.  Absorbed MLA
    reading: keys are the full 576-wide rows, values their first 512 entries.

    q_row float64 [H, 576]; x_rows float64 [n, 576].  Returns (o [H, 512],
    lse [H]); an empty split gives o = 0 and lse = -inf.
    """
    h = q_row.shape[0]
    if x_rows.shape[0] == 0:
        return np.zeros((h, D_LATENT)), np.full(h, -np.inf)
    logits = sm_scale * (q_row @ x_rows.T)            # [H, n]
    m = np.max(logits, axis=1, keepdims=True)
    p = np.exp(logits - m)
    z = np.sum(p, axis=1, keepdims=True)
    o = (p @ x_rows[:, :D_LATENT]) / z
    lse = (m + np.log(z))[:, 0]
    return o, lse


def lse_merge(part_o, part_lse) -> tuple[np.ndarray, np.ndarray]:
    """Merge split partials by their natural-log LSE.

    Subject page, split-K commit note (the reduce that can store the
    natural-log LSE): lse = log sum_s exp(lse_s); out = sum_s exp(lse_s - lse)
    * o_s.  Splits with lse_s = -inf carry no mass and are skipped; if every
    split is empty, out = 0 and lse = -inf.

    part_o [..., S, Dv]; part_lse [..., S].  Returns (out [..., Dv], lse [...]).
    """
    po = np.asarray(part_o, dtype=np.float64)
    pl = np.asarray(part_lse, dtype=np.float64)
    m = np.max(pl, axis=-1, keepdims=True)
    empty = ~np.isfinite(m)
    m_safe = np.where(empty, 0.0, m)
    wts = np.where(np.isfinite(pl), np.exp(pl - m_safe), 0.0)
    tot = np.sum(wts, axis=-1, keepdims=True)
    lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))[..., 0]
    out = np.sum(wts[..., None] * po, axis=-2) / np.where(empty, 1.0, tot)
    out = np.where(empty, 0.0, out)
    return out, lse


def project_v(out_latent, w_uv_bits) -> np.ndarray:
    """The value projection W_UV of absorbed MLA, applied to latent outputs.

    Page "[ROCm] Support decode context parallel (DCP) for GLM-5 /
    DeepSeek-V3.2", Future work: projecting V before the LSE merge (a
    follow-up that cut decode ITL).  Absorbed MLA keeps the attention output
    in the 512-wide latent space (R11); head h's value output is
    v[d] = sum_k latent[k] * W[h][d][k] for d < Dv.  The page gives no Dv or
    layout; reading: Dv = 128 and the weights bf16 [H, Dv, 512] (each output
    dimension's weights one contiguous row).

    out_latent [..., H, 512] float; w_uv_bits uint16 [H, Dv, 512] bf16.
    Returns float64 [..., H, Dv].
    """
    x = np.asarray(out_latent, dtype=np.float64)
    w = bf16_decode(w_uv_bits)
    return np.einsum("...hk,hdk->...hd", x, w)


def lse_merge_project(part_o, part_lse, w_uv_bits) -> tuple[np.ndarray, np.ndarray]:
    """The LSE merge followed by the value projection: since the projection
    is linear and the merge is a weighted sum with weights summing to one,
    this equals projecting each split before merging (the page's order),
    with the merge applied once instead of per split.

    part_o [R, H, S, 512]; part_lse [R, H, S]; w_uv_bits [H, Dv, 512].
    Returns (out [R, H, Dv] float64, lse [R, H]).
    """
    out, lse = lse_merge(part_o, part_lse)
    return project_v(out, w_uv_bits), lse


def gather_mla_rows(kv_code, kv_scale, page_table_row, slots, page_size: int) -> np.ndarray:
    """Dequantized 576-wide MLA rows of the given logical slots (one fp32 scale
    per token, read from the same physical row)."""
    kv_code = np.asarray(kv_code)
    n_pages = kv_code.shape[0]
    slots = np.asarray(slots, dtype=np.int64)
    pt = np.asarray(page_table_row, dtype=np.int64)
    pages = pt[slots // page_size]
    if np.any(pages < 0) or np.any(pages >= n_pages):
        raise ValueError("selected slot maps to an invalid page")
    phys = pages * page_size + slots % page_size
    codes = kv_code.reshape(-1, kv_code.shape[-1])[phys]
    scales = np.asarray(kv_scale, dtype=np.float64).reshape(-1)[phys]
    return fp8_e4m3fn_decode(codes) * scales[:, None]


def sparse_mla(q_bf16_bits, kv_code, kv_scale, page_table, row_req, topk_idx,
               topk_count, sm_scale: float, n_splits: int, page_size: int):
    """Split-K sparse absorbed-MLA attention over each row's selected slots.

    Subject page, "Sparse decode": each row attends only its selected slots;
    the selected list (the first ``topk_count[r]`` entries of ``topk_idx[r]``)
    is cut into ``n_splits`` contiguous equal chunks, each giving a partial
    (output, natural-log LSE).

    q_bf16_bits uint16 [R, H, 576]; kv_code uint8 [NP, P, 576];
    kv_scale [NP, P]; topk_idx int [R, k]; topk_count int [R].
    Returns (part_o float64 [R, H, S, 512], part_lse float64 [R, H, S]).
    """
    q = bf16_decode(q_bf16_bits)
    r_n, h = q.shape[0], q.shape[1]
    page_table = np.asarray(page_table)
    row_req = np.asarray(row_req, dtype=np.int64)
    part_o = np.zeros((r_n, h, n_splits, D_LATENT))
    part_lse = np.full((r_n, h, n_splits), -np.inf)
    for r in range(r_n):
        cnt = int(topk_count[r])
        sel = np.asarray(topk_idx[r][:cnt], dtype=np.int64)
        x = gather_mla_rows(kv_code, kv_scale, page_table[row_req[r]], sel, page_size)
        for s, (lo, hi) in enumerate(split_ranges(cnt, n_splits)):
            o, lse = attend_split(q[r], x[lo:hi], sm_scale)
            part_o[r, :, s] = o
            part_lse[r, :, s] = lse
    return part_o, part_lse


# ---------------------------------------------------------------------------
# The whole step
# ---------------------------------------------------------------------------


def decode_step(inp: dict, n_index_splits: int = 1, n_attn_splits: int = 1,
                rows=None) -> dict:
    """One DSA decode step: quantize the indexer query, score, select the
    top-k (per split, then merged), attend the selected rows per attention
    split, and merge by LSE.

    ``inp`` holds numpy arrays: q_idx (uint16 bf16 bits [R,64,128]), head_w,
    k_code, k_scale, kv_code, kv_scale, q_mla (uint16 [R,H,576]), page_table,
    kv_lens, row_req, row_vis, and the ints page_size, top_k and the float
    sm_scale.  ``rows`` optionally restricts the work to a subset of rows.
    Returns a dict of float64 / int64 arrays for those rows.
    """
    rows = np.arange(len(inp["row_req"])) if rows is None else np.asarray(rows)
    p = int(inp["page_size"])
    k = int(inp["top_k"])
    q_code, q_scale = quantize_q(inp["q_idx"][rows])
    row_req = np.asarray(inp["row_req"])[rows]
    row_vis = np.asarray(inp["row_vis"])[rows]
    score_len = max(1, int(np.max(row_vis)) if len(rows) else 1)
    scores = index_scores(q_code, q_scale, np.asarray(inp["head_w"])[rows],
                          inp["k_code"], inp["k_scale"], inp["page_table"],
                          inp["kv_lens"], row_req, row_vis, p, score_len)
    idx = np.full((len(rows), k), -1, dtype=np.int64)
    cnt = np.zeros(len(rows), dtype=np.int64)
    for i in range(len(rows)):
        idx[i], cnt[i] = topk_split_merge(scores[i], int(row_vis[i]), k, n_index_splits)
    part_o, part_lse = sparse_mla(inp["q_mla"][rows], inp["kv_code"], inp["kv_scale"],
                                  inp["page_table"], row_req, idx, cnt,
                                  float(inp["sm_scale"]), n_attn_splits, p)
    out, lse = lse_merge(part_o, part_lse)
    return {"q_code": q_code, "q_scale": q_scale, "scores": scores,
            "topk_idx": idx, "topk_count": cnt, "part_o": part_o,
            "part_lse": part_lse, "out": out, "lse": lse}


def decode_step_index_share(inp: dict, chain: int, n_index_splits: int = 1, n_attn_splits: int = 1) -> dict:
    """MTP IndexShare: one top-k list for a chain of draft rows.

    Subject page, Modifications, "MTP / EAGLE" and the chain-EAGLE commit
    note: the draft runs five steps with six draft tokens, and the option
    that shares the index across MTP iterations is named (it is switched off
    under DCP only because a rank there holds just its owned share of the
    top-k).  The page does not spell out what is shared; the reading taken
    here is the plainest one: the rows of one request's chain (``chain``
    consecutive rows, the chain's draft iterations in order, each seeing
    one more slot than the one before) run the indexer and the top-k once,
    for the chain's first row, and every row of the chain attends that one
    list with its own query.  The first row sees the fewest slots, so every
    entry of its list lies inside every later row's span.

    Returns the leads' scores and selection, the list each row attends
    (``row_list``, an index into the leads) and every row's merged output.
    """
    row_req = np.asarray(inp["row_req"], dtype=np.int64)
    row_vis = np.asarray(inp["row_vis"], dtype=np.int64)
    n_rows = len(row_req)
    if chain < 1 or n_rows % chain != 0:
        raise ValueError("the rows must form whole chains")
    lead = np.arange(0, n_rows, chain)
    row_list = np.arange(n_rows) // chain
    if np.any(row_req != row_req[lead][row_list]):
        raise ValueError("every row of a chain must belong to the chain's request")
    if np.any(row_vis < row_vis[lead][row_list]):
        raise ValueError("no row of a chain may see fewer slots than its first row")
    sel = decode_step(inp, n_index_splits, n_attn_splits, rows=lead)
    idx = sel["topk_idx"][row_list]
    cnt = sel["topk_count"][row_list]
    part_o, part_lse = sparse_mla(inp["q_mla"], inp["kv_code"], inp["kv_scale"], inp["page_table"], row_req,
                                  idx, cnt, float(inp["sm_scale"]), n_attn_splits, int(inp["page_size"]))
    out, lse = lse_merge(part_o, part_lse)
    return {"lead_rows": lead, "row_list": row_list, "q_code": sel["q_code"], "q_scale": sel["q_scale"],
            "scores": sel["scores"], "topk_idx": sel["topk_idx"], "topk_count": sel["topk_count"],
            "out": out, "lse": lse}


def sm_scale_default() -> float:
    """1/sqrt(576): unit-variance logits for unit-variance rows."""
    return 1.0 / math.sqrt(D_QK)
