"""Seeded synthetic inputs for the DSA sparse decode step.

This module only synthesises inputs: random numbers, fp8 encoding of the
synthetic caches (the cache writer's job, which precedes the step), page
tables and row geometry.  It holds none of the step's arithmetic and imports
neither the oracle nor the HIP binding, so both sides can consume what it
makes.

Shapes follow the workloads the subject page ("[ROCm] Support decode context
parallel (DCP) for GLM-5 / DeepSeek-V3.2", Modifications and Speed Tests)
describes: top-2048 selection, a 64-head x 128 fp8 indexer with one fp32
scale per token, absorbed MLA over 512 latent + 64 rope fp8 rows with one
fp32 scale per token, 256-token pages shuffled in a pool, decode rows,
six-token MTP verify rows and long-prefix prefill rows.

Layout of one page pool (NP pages of P tokens):
  k_code  uint8   [NP, P, 128]   indexer keys, E4M3FN codes
  k_scale float32 [NP, P]
  kv_cache uint8  [NP, P, 640]   MLA rows: bytes 0..575 the E4M3FN codes (512
                                 latent, then 64 rope), bytes 576..579 the
                                 row's fp32 scale, bytes 580..639 unused
                                 (filled with 0x7F, an E4M3FN NaN code)
  (kv_code and kv_scale are views of kv_cache's codes and scales)
Rows (query tokens) are request-major: row r belongs to request row_req[r]
and sees the first row_vis[r] slots of that request.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

IDX_HEADS = 64
IDX_DIM = 128
D_QK = 576
D_V = 512
TOP_K = 2048
POISON_SCALE = 1.0e6
KV_ROW_BYTES = 640      # 576 code bytes + 4 scale bytes, padded to five 128-byte lines
PAD_CODE = 0x7F


def kv_code_view(kv_cache: torch.Tensor) -> torch.Tensor:
    """uint8 [NP, P, 576] view of the codes of a packed MLA cache."""
    return kv_cache[..., :D_QK]


def kv_scale_view(kv_cache: torch.Tensor) -> torch.Tensor:
    """float32 [NP, P] view of the scales of a packed MLA cache."""
    return kv_cache[..., D_QK:D_QK + 4].view(torch.float32).squeeze(-1)


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    kv_lens: tuple | None = None          # fixed lengths, or None for uniform
    kv_range: tuple | None = None         # inclusive (lo, hi) for uniform lengths
    rows_per_req: int = 1
    causal: str = "decode"                # decode | mtp | prefill
    prefix: int = 0                       # prefill: cached prefix before the new rows
    page_size: int = 256
    mla_heads: int = 32
    top_k: int = TOP_K
    index_splits: int = 1
    attn_splits: int = 1
    pool_pages: int | None = None         # None: exactly the pages needed (+ spare)
    spare_pages: int = 3                  # unused, poison-filled pages in the pool
    planted: int = 0                      # boosted slots per request
    planted_factor: float = 8.0
    group_rows: int = 1                   # rows scored together against one key stream
    index_share: int = 0                  # MTP IndexShare: rows per chain sharing one top-k list
    index_topk: bool = False              # rows scored one at a time: scores and top-k in one call
    phys_rows: bool = False               # top-k emits physical rows; the attention gathers them directly


CONFIGS = {
    # Tiny decode step: request 0 is shorter than top-k (dense attention).
    "c0": Config("c0", batch=2, kv_lens=(1500, 5000), page_size=64, mla_heads=16,
                 pool_pages=256, index_splits=4, attn_splits=4),
    # Bulk decode, ragged lengths.
    "c1": Config("c1", batch=64, kv_range=(8192, 32768), mla_heads=32,
                 index_splits=1, attn_splits=4),
    # Bulk decode at the metric's point: every request 32768 tokens.
    "c1_l32k": Config("c1_l32k", batch=64, kv_lens=(32768,) * 64, mla_heads=32,
                      index_splits=1, attn_splits=4),
    # Long-context decode with planted high-score tokens.
    "c2": Config("c2", batch=8, kv_lens=(9600, 38000, 77000, 131072) * 2, mla_heads=32,
                 index_splits=16, attn_splits=32, planted=4),
    # MTP verify: 6 causal rows per request.
    "c3": Config("c3", batch=32, kv_range=(16384, 65536), rows_per_req=6, causal="mtp",
                 mla_heads=32, index_splits=4, attn_splits=1, group_rows=6),
    # MTP draft chains with IndexShare: the MTP-verify geometry (32 requests x
    # 6 causal rows), the indexer and top-k run on each chain's first row
    # only, and all six rows attend that row's list.
    "c3s": Config("c3s", batch=32, kv_range=(16384, 65536), rows_per_req=6, causal="mtp",
                  mla_heads=32, index_splits=4, attn_splits=1, index_share=6),
    # Long-prefix prefill on the owned top-k path: 4096 new rows after 65536.
    # Five index splits keep each split's list (69632 / 5 scores) within 16
    # keys a thread.
    "c4": Config("c4", batch=1, kv_lens=(65536 + 4096,), rows_per_req=4096,
                 causal="prefill", prefix=65536, mla_heads=32, index_splits=5,
                 attn_splits=1, group_rows=8),
}


@dataclass
class Inputs:
    cfg: Config
    seed: int
    q_idx: torch.Tensor       # bf16 [R, 64, 128]
    head_w: torch.Tensor      # f32 [R, 64]
    q_mla: torch.Tensor       # bf16 [R, H, 576]
    k_code: torch.Tensor      # u8 [NP, P, 128]
    k_scale: torch.Tensor     # f32 [NP, P]
    kv_cache: torch.Tensor    # u8 [NP, P, 640]: codes, fp32 scale, pad
    page_table: torch.Tensor  # i32 [B, max_pages], -1 past each span
    kv_lens: torch.Tensor     # i32 [B]
    row_req: torch.Tensor     # i32 [R]
    row_vis: torch.Tensor     # i32 [R]
    sm_scale: float = field(default=1.0 / math.sqrt(D_QK))
    planted_slots: torch.Tensor | None = None  # i64 [B, planted]

    @property
    def kv_code(self) -> torch.Tensor:
        return kv_code_view(self.kv_cache)

    @property
    def kv_scale(self) -> torch.Tensor:
        return kv_scale_view(self.kv_cache)

    @property
    def n_rows(self) -> int:
        return int(self.row_req.shape[0])

    @property
    def n_pages(self) -> int:
        return int(self.k_code.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def page_size(self) -> int:
        return int(self.k_code.shape[1])

    @property
    def mla_heads(self) -> int:
        return int(self.q_mla.shape[1])

    @property
    def top_k(self) -> int:
        return self.cfg.top_k

    def max_vis(self) -> int:
        return int(self.row_vis.max().item()) if self.n_rows else 0


def _encode_fp8_rows(x: torch.Tensor) -> tuple[torch.Tensor, torch.Tensor]:
    """Encode rows of synthetic values as E4M3FN codes with one fp32 scale per
    row (max|x| / 448), as a cache writer would; torch's cast rounds to
    nearest even."""
    amax = x.abs().amax(dim=-1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    y = (x / scale.unsqueeze(-1)).clamp_(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8), scale.float()


def _normal(shape, gen, device, std=1.0):
    return torch.randn(shape, generator=gen, device=device, dtype=torch.float32) * std


def make(name_or_cfg, seed: int | None = None, device="cpu", poison: bool = True,
         chunk_pages: int = 512) -> Inputs:
    """Build the seeded inputs of one configuration on ``device``.

    The same (config, seed, device type) always gives the same tensors.  Slots
    that no row may read (the tail of each request's last page and the spare
    pages) hold poison: codes of N(0,1) data with a scale of 1e6, so any leak
    shows up in scores and outputs.
    """
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    if seed is None:
        seed = sum(map(ord, cfg.name))
    device = torch.device(device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    b = cfg.batch
    p = cfg.page_size
    if cfg.kv_lens is not None:
        kv = torch.tensor(cfg.kv_lens, dtype=torch.int64)
    else:
        lo, hi = cfg.kv_range
        kv = torch.randint(lo, hi + 1, (b,), generator=gen, device=device).cpu()
    pages_per_req = [(-(-int(v) // p)) for v in kv.tolist()]
    need = sum(pages_per_req)
    n_pool = cfg.pool_pages if cfg.pool_pages is not None else need + cfg.spare_pages
    if n_pool < need:
        raise ValueError("pool smaller than the pages the requests need")
    perm = torch.randperm(n_pool, generator=gen, device=device).cpu()
    max_pages = max(pages_per_req)
    page_table = torch.full((b, max_pages), -1, dtype=torch.int32)
    used = torch.zeros(n_pool, dtype=torch.bool)
    off = 0
    for i, n in enumerate(pages_per_req):
        page_table[i, :n] = perm[off:off + n].to(torch.int32)
        used[perm[off:off + n]] = True
        off += n

    # Caches, page by page in chunks to bound temporary memory.
    k_code = torch.empty((n_pool, p, IDX_DIM), dtype=torch.uint8, device=device)
    k_scale = torch.empty((n_pool, p), dtype=torch.float32, device=device)
    kv_cache = torch.full((n_pool, p, KV_ROW_BYTES), PAD_CODE, dtype=torch.uint8, device=device)
    kv_code = kv_code_view(kv_cache)
    kv_scale = kv_scale_view(kv_cache)
    for s in range(0, n_pool, chunk_pages):
        e = min(n_pool, s + chunk_pages)
        c, sc = _encode_fp8_rows(_normal((e - s, p, IDX_DIM), gen, device))
        k_code[s:e] = c
        k_scale[s:e] = sc
        c, sc = _encode_fp8_rows(_normal((e - s, p, D_QK), gen, device))
        kv_code[s:e] = c
        kv_scale[s:e] = sc

    if poison:
        valid = torch.zeros((n_pool, p), dtype=torch.bool)
        for i, n in enumerate(pages_per_req):
            if n == 0:
                continue
            pages = page_table[i, :n].long()
            valid[pages] = True
            tail = int(kv[i]) - (n - 1) * p
            valid[pages[-1], tail:] = False
        bad = (~valid).to(device)
        k_scale.masked_fill_(bad, POISON_SCALE)
        kv_scale.masked_fill_(bad, POISON_SCALE)

    # Rows.
    rows_req, rows_vis = [], []
    for i in range(b):
        for j in range(cfg.rows_per_req):
            rows_req.append(i)
            if cfg.causal == "decode":
                rows_vis.append(int(kv[i]))
            elif cfg.causal == "mtp":
                rows_vis.append(int(kv[i]) - cfg.rows_per_req + j + 1)
            elif cfg.causal == "prefill":
                rows_vis.append(cfg.prefix + j + 1)
            else:
                raise ValueError(cfg.causal)
    n_rows = len(rows_req)
    q_idx = _normal((n_rows, IDX_HEADS, IDX_DIM), gen, device).to(torch.bfloat16)
    head_w = _normal((n_rows, IDX_HEADS), gen, device, std=1.0 / 8.0)
    q_mla = _normal((n_rows, cfg.mla_heads, D_QK), gen, device).to(torch.bfloat16)

    planted_slots = None
    if cfg.planted:
        planted_slots = torch.empty((b, cfg.planted), dtype=torch.int64)
        for i in range(b):
            sl = torch.randperm(int(kv[i]), generator=gen, device=device)[: cfg.planted].cpu()
            planted_slots[i] = sl
            pages = page_table[i, (sl // p)].long().to(device)
            offs = (sl % p).to(device)
            k_scale[pages, offs] *= cfg.planted_factor
            kv_scale[pages, offs] *= cfg.planted_factor

    return Inputs(cfg=cfg, seed=seed, q_idx=q_idx, head_w=head_w, q_mla=q_mla,
                  k_code=k_code, k_scale=k_scale, kv_cache=kv_cache,
                  page_table=page_table.to(device), kv_lens=kv.to(torch.int32).to(device),
                  row_req=torch.tensor(rows_req, dtype=torch.int32, device=device),
                  row_vis=torch.tensor(rows_vis, dtype=torch.int32, device=device),
                  planted_slots=planted_slots)


def to(inp: Inputs, device) -> Inputs:
    """Copy every tensor of ``inp`` to ``device``."""
    kw = {}
    for f in ("q_idx", "head_w", "q_mla", "k_code", "k_scale", "kv_cache",
              "page_table", "kv_lens", "row_req", "row_vis"):
        kw[f] = getattr(inp, f).to(device)
    return replace(inp, **kw)


def subset(inp: Inputs, rows) -> Inputs:
    """A smaller, self-contained copy holding only ``rows``, their requests and
    those requests' pages (on the CPU).  Page contents are copied bit for bit
    and the block tables are renumbered; nothing is computed."""
    rows = torch.as_tensor(rows, dtype=torch.int64).cpu()
    row_req = inp.row_req.cpu()[rows].long()
    reqs = torch.unique(row_req)
    pt = inp.page_table.cpu()
    new_req = {int(r): i for i, r in enumerate(reqs.tolist())}
    old_pages = []
    new_pt = torch.full((len(reqs), pt.shape[1]), -1, dtype=torch.int32)
    for i, r in enumerate(reqs.tolist()):
        row = pt[r]
        n = int((row >= 0).sum())
        new_pt[i, :n] = torch.arange(len(old_pages), len(old_pages) + n, dtype=torch.int32)
        old_pages.extend(row[:n].tolist())
    op = torch.tensor(old_pages, dtype=torch.int64, device=inp.k_code.device)
    return replace(
        inp,
        q_idx=inp.q_idx[rows.to(inp.q_idx.device)].cpu(),
        head_w=inp.head_w[rows.to(inp.head_w.device)].cpu(),
        q_mla=inp.q_mla[rows.to(inp.q_mla.device)].cpu(),
        k_code=inp.k_code[op].cpu(), k_scale=inp.k_scale[op].cpu(),
        kv_cache=inp.kv_cache[op].cpu(),
        page_table=new_pt, kv_lens=inp.kv_lens.cpu()[reqs],
        row_req=torch.tensor([new_req[int(r)] for r in row_req.tolist()], dtype=torch.int32),
        row_vis=inp.row_vis.cpu()[rows],
        planted_slots=None if inp.planted_slots is None else inp.planted_slots[reqs],
    )


def as_numpy(inp: Inputs) -> dict:
    """The inputs as numpy arrays (bf16 as uint16 bit patterns, fp8 as uint8
    codes), in the dict form the CPU oracle takes."""
    def u16(t):
        return t.cpu().contiguous().view(torch.int16).numpy().view("uint16")
    return {
        "q_idx": u16(inp.q_idx), "head_w": inp.head_w.cpu().numpy(),
        "q_mla": u16(inp.q_mla),
        "k_code": inp.k_code.cpu().numpy(), "k_scale": inp.k_scale.cpu().numpy(),
        "kv_code": inp.kv_code.cpu().contiguous().numpy(),
        "kv_scale": inp.kv_scale.cpu().contiguous().numpy(),
        "page_table": inp.page_table.cpu().numpy(), "kv_lens": inp.kv_lens.cpu().numpy(),
        "row_req": inp.row_req.cpu().numpy(), "row_vis": inp.row_vis.cpu().numpy(),
        "page_size": inp.page_size, "top_k": inp.top_k, "sm_scale": inp.sm_scale,
    }


# --------------------------------------------------------------------------
# New tokens for the cache write (the step before the decode path)
# --------------------------------------------------------------------------

ROPE_BASE = 10000.0


@dataclass
class NewTokens:
    latent: torch.Tensor      # bf16 [n, 512]
    rope: torch.Tensor        # bf16 [n, 64], before rotation
    index_k: torch.Tensor     # bf16 [n, 128]
    tok_req: torch.Tensor     # i32 [n]
    tok_slot: torch.Tensor    # i32 [n]
    rope_cos: torch.Tensor    # f32 [max_pos, 32]
    rope_sin: torch.Tensor    # f32 [max_pos, 32]


def rope_tables(max_pos: int, base: float = ROPE_BASE, device="cpu"):
    """cos / sin f32 [max_pos, 32] of the angles pos * base^(-j / 32): an
    input of the cache write, tabulated the usual way."""
    j = torch.arange(32, dtype=torch.float64)
    theta = torch.arange(max_pos, dtype=torch.float64)[:, None] * base ** (-j / 32.0)[None, :]
    return theta.cos().float().to(device), theta.sin().float().to(device)


def make_new_tokens(inp: Inputs, tok_req, tok_slot, seed: int = 0, device=None) -> NewTokens:
    """Seeded bf16 rows for tokens (tok_req[i], tok_slot[i]): latent, rope and
    index entries N(0, 1) times a per-token magnitude in [1e-3, 1e2], with an
    all-zero token and a token holding -0.0 entries when there are enough
    tokens; rotation tables cover every slot of the block table."""
    device = device or inp.k_code.device
    g = torch.Generator().manual_seed(seed)
    tok_req = torch.as_tensor(tok_req, dtype=torch.int32)
    tok_slot = torch.as_tensor(tok_slot, dtype=torch.int32)
    n = int(tok_req.shape[0])
    mag = torch.exp(torch.empty(n, 1).uniform_(math.log(1e-3), math.log(1e2), generator=g))
    latent = torch.randn(n, 512, generator=g) * mag
    rope = torch.randn(n, 64, generator=g) * mag
    index_k = torch.randn(n, 128, generator=g) * mag
    if n >= 3:
        latent[1] = 0.0
        rope[1] = 0.0
        index_k[1] = 0.0
        latent[2, ::7] = -0.0
        index_k[2, ::5] = -0.0
    cos, sin = rope_tables(inp.max_pages * inp.page_size)
    return NewTokens(latent=latent.to(torch.bfloat16).to(device), rope=rope.to(torch.bfloat16).to(device),
                     index_k=index_k.to(torch.bfloat16).to(device), tok_req=tok_req.to(device),
                     tok_slot=tok_slot.to(device), rope_cos=cos.to(device), rope_sin=sin.to(device))



# --------------------------------------------------------------------------
# Value projection (the step after the decode path)
# --------------------------------------------------------------------------

D_V = 128


def make_w_uv(n_heads: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """Seeded W_UV of one head shard: bf16 [H, 128, 512], entries
    N(0, 1/512), so a unit-scale latent projects to unit-scale values."""
    g = torch.Generator().manual_seed(seed)
    w = torch.randn(n_heads, D_V, 512, generator=g) / math.sqrt(512.0)
    return w.to(torch.bfloat16).to(device)


def make_partials(n_rows: int, n_heads: int, n_splits: int, seed: int = 0, device="cpu"):
    """Seeded split partials for the merge: part_o N(0, 1) bf16 [R, H, S, 512],
    part_lse N(0, 9) f32 [R, H, S], with an empty split (lse -inf, o 0) and,
    for R >= 3, a row whose splits are all empty."""
    g = torch.Generator().manual_seed(seed)
    po = torch.randn(n_rows, n_heads, n_splits, 512, generator=g)
    pl = torch.randn(n_rows, n_heads, n_splits, generator=g) * 3.0
    if n_splits > 1 and n_rows > 0:
        pl[0, 0, n_splits - 1] = -math.inf
        po[0, 0, n_splits - 1] = 0.0
    if n_rows >= 3:
        pl[2, :, :] = -math.inf
        po[2, :, :, :] = 0.0
    return po.to(torch.bfloat16).to(device), pl.to(device)
