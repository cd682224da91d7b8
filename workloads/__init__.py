"""Seeded synthetic inputs for striped paged-attention workloads.

This module only draws numbers: context lengths, query-token counts, logical page ids for each row's block table,
and the Q / K / V values of every row. It holds none of the method's arithmetic (no slot mapping, no striping, no
attention), so that both the float64 oracle and the HIP path can take their inputs from here.

Shapes follow the workloads on the pages: Llama-style GQA decode, a long-context GQA decode, a DeepSeek-style MLA
decode with one latent head, a mixed decode/extend step with own-token attention in a padded bucket, and a tiny fp32
case the oracle finishes instantly.

Conventions (one place, used by every consumer):

* Integers come from ``numpy.random.default_rng(seed)``: lengths first, then the page-id permutation.
* Page id 0 is the sink page and is never handed to a row. The free ids ``1..num_pages-1`` are randomly permuted and
  handed out in row order; a few spare ids at the end of the permutation stay unused, so unused pages exist in the
  pool. Block-table entries past a row's last page are 0 (the sink).
* Values are drawn per row from a ``torch.Generator`` seeded ``seed * 2**20 + row`` on the requested device, in the
  order q, k_ctx, v_ctx, k_new, v_new (MLA: q, latent_ctx, latent_new), as float32 normals times ``std`` and then
  rounded once to the workload dtype. A consumer on another device gets its copy with ``.cpu()``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

__all__ = ["Workload", "RowValues", "make", "CONFIG_NAMES", "row_values", "describe"]


CONFIG_NAMES = ("tiny", "llama8b", "longctx", "mla", "mixed")


@dataclass
class Workload:
    """One seeded workload: shapes, lengths, block tables. Values come from :func:`row_values`."""

    name: str
    kind: str                 # "gqa" or "mla"
    dtype: str                # "f32" or "bf16": the dtype of q, k, v in HBM
    num_q_heads: int
    num_kv_heads: int
    head_dim: int             # qk head dim (576 for MLA: 512 latent + 64 rope)
    head_dim_v: int           # value dim (512 for MLA: the latent part of the row)
    page_size: int            # logical page size (tokens a logical page)
    partners: int             # P: number of stripes
    scale: float
    std: float
    seed: int
    ctx_len: np.ndarray       # int32 [B]: tokens of each row already in the pool
    new_len: np.ndarray       # int32 [B]: query tokens of each row in this step
    own_token: bool           # in-step tokens attend each other causally (own-token partial)
    bucket: int               # padded number of query tokens (>= sum(new_len))
    block_table: np.ndarray   # int32 [B, max_pages]: logical page ids, 0 = sink
    num_pages: int            # pages in each stripe's pool (page ids are logical: same range for every stripe)
    pad_rows: int = 0         # extra padding rows (zero tokens, zero context) appended after the real rows
    interleave: int = 1       # KV-cache interleave size I of the pool (runs of I slots per partner)
    kv_dtype: str = "same"    # "same" (pools in dtype) or "fp8" (pools hold E4M3 codes with per-tensor descales)
    k_descale: float = 1.0    # fp8 pools: a key element is its code's value times k_descale
    v_descale: float = 1.0
    notes: list = field(default_factory=list)

    @property
    def batch(self) -> int:
        return int(self.ctx_len.shape[0])

    @property
    def num_tokens(self) -> int:
        return int(self.new_len.sum())

    @property
    def q_row_start(self) -> np.ndarray:
        out = np.zeros(self.batch + 1, dtype=np.int32)
        np.cumsum(self.new_len, out=out[1:])
        return out

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def max_pages(self) -> int:
        return int(self.block_table.shape[1])

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes of the context attention: every context token's K and V once."""
        el = 1 if self.kv_dtype == "fp8" else 4 if self.dtype == "f32" else 2
        total = int(self.ctx_len.astype(np.int64).sum())
        if self.kind == "mla":
            return total * self.head_dim * el
        return total * self.num_kv_heads * (self.head_dim + self.head_dim_v) * el


@dataclass
class RowValues:
    q: torch.Tensor                    # [n, Hq, D]
    k_ctx: torch.Tensor                # [c, Hkv, D]   (MLA: [c, 1, 576] latent rows)
    v_ctx: torch.Tensor                # [c, Hkv, Dv]  (MLA: a view of the first 512 latent columns)
    k_new: torch.Tensor | None         # [n, Hkv, D] own-token keys, or None
    v_new: torch.Tensor | None


def _uniform_int(rng, lo, hi, n):
    return rng.integers(lo, hi + 1, size=n).astype(np.int64)


def _log_uniform_int(rng, lo, hi, n):
    u = rng.uniform(math.log(lo), math.log(hi + 1), size=n)
    return np.clip(np.floor(np.exp(u)), lo, hi).astype(np.int64)


def _block_tables(rng, tokens_per_row, page_size, spare_frac=0.02, min_spare=2, width=None):
    """Hand out a random permutation of page ids 1..N-1 in row order; page 0 is the sink."""
    pages = [(int(t) + page_size - 1) // page_size for t in tokens_per_row]
    used = int(sum(pages))
    spare = max(min_spare, int(math.ceil(used * spare_frac)))
    num_pages = 1 + used + spare
    perm = rng.permutation(np.arange(1, num_pages, dtype=np.int64))
    w = max(1, max(pages) if pages else 1)
    if width is not None:
        w = max(w, int(width))
    bt = np.zeros((len(pages), w), dtype=np.int32)
    pos = 0
    for b, n in enumerate(pages):
        bt[b, :n] = perm[pos:pos + n]
        pos += n
    return bt, num_pages


def make(name: str, seed: int | None = None, *, batch: int | None = None, ctx_range=None,
         ctx_lengths=None, new_lengths=None, partners: int | None = None, page_size: int | None = None,
         bucket: int | None = None, pad_rows: int = 0, bt_width: int | None = None, interleave: int = 1,
         kv_dtype: str = "same", num_q_heads: int | None = None) -> Workload:
    """Build workload ``name`` (one of :data:`CONFIG_NAMES`), optionally shrunk for parity tests.

    ``seed`` defaults to ``1000 + k`` for the k-th config (1-based). ``batch``/``ctx_range``/``ctx_lengths``/
    ``new_lengths`` override the row count and the length distribution while keeping head shapes, dtype, page size
    and P; ``partners``/``page_size`` override P and the logical page size; ``interleave`` sets the pool's KV-cache
    interleave size (1 = the plain slot rule); ``kv_dtype="fp8"`` (bf16 workloads) stores the context K/V as E4M3
    codes: each value is divided by its tensor's descale (GQA: 0.0173 for K, 0.0291 for V, fixed, unequal, not powers
    of two; MLA: 0.0091 for the latent rows, which serve as keys and, by their first 512 columns, as values), clipped to
    +-448 and rounded by torch's float8_e4m3fn conversion. ``num_q_heads`` (MLA only) sets the query heads
    sharing the latent head: 128 is the whole model, 64, 32 and 16 are its share on 2, 4 and 8 tensor-parallel ranks.
    """
    if name not in CONFIG_NAMES:
        raise ValueError(f"unknown workload {name!r}; expected one of {CONFIG_NAMES}")
    k = CONFIG_NAMES.index(name) + 1
    seed = 1000 + k if seed is None else int(seed)
    rng = np.random.default_rng(seed)
    notes = []

    if name == "tiny":
        base = dict(kind="gqa", dtype="f32", num_q_heads=4, num_kv_heads=1, head_dim=64, head_dim_v=64,
                    page_size=16, partners=2, scale=1.0 / math.sqrt(64), std=1.0, own_token=False)
        ctx = np.array([1, 17, 100, 200], dtype=np.int64) if ctx_lengths is None else np.asarray(ctx_lengths)
        new = np.ones_like(ctx)
    elif name in ("llama8b", "longctx"):
        base = dict(kind="gqa", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, head_dim_v=128,
                    page_size=16, partners=4 if name == "llama8b" else 8, scale=1.0 / math.sqrt(128), std=1.0,
                    own_token=False)
        B = batch if batch is not None else (64 if name == "llama8b" else 256)
        if ctx_lengths is not None:
            ctx = np.asarray(ctx_lengths, dtype=np.int64)
        elif name == "llama8b":
            lo, hi = ctx_range if ctx_range is not None else (1024, 8192)
            ctx = _uniform_int(rng, lo, hi, B)
        else:
            lo, hi = ctx_range if ctx_range is not None else (4096, 32768)
            ctx = _log_uniform_int(rng, lo, hi, B)
        new = np.ones_like(ctx)
    elif name == "mla":
        base = dict(kind="mla", dtype="bf16", num_q_heads=128, num_kv_heads=1, head_dim=576, head_dim_v=512,
                    page_size=64, partners=4, scale=1.0 / math.sqrt(192), std=0.5, own_token=False)
        B = batch if batch is not None else 128
        if ctx_lengths is not None:
            ctx = np.asarray(ctx_lengths, dtype=np.int64)
        else:
            lo, hi = ctx_range if ctx_range is not None else (2048, 16384)
            ctx = _uniform_int(rng, lo, hi, B)
        new = np.ones_like(ctx)
    else:  # mixed
        base = dict(kind="gqa", dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, head_dim_v=128,
                    page_size=16, partners=4, scale=1.0 / math.sqrt(128), std=1.0, own_token=True)
        B = batch if batch is not None else 32
        half = B // 2
        if new_lengths is not None:
            new = np.asarray(new_lengths, dtype=np.int64)
        else:
            new = np.concatenate([np.ones(half, dtype=np.int64), _uniform_int(rng, 1, 512, B - half)])
        if ctx_lengths is not None:
            ctx = np.asarray(ctx_lengths, dtype=np.int64)
        else:
            lo, hi = ctx_range if ctx_range is not None else (0, 16384)
            ctx = _uniform_int(rng, lo, hi, B)
        if bucket is None:
            bucket = 8192 if batch is None else int(new.sum()) + 8
        if int(new.sum()) > bucket:
            raise ValueError(f"in-step tokens {int(new.sum())} exceed the bucket {bucket}")

    if num_q_heads is not None:
        if base["kind"] != "mla":
            raise ValueError("num_q_heads is only set for the MLA workload")
        base["num_q_heads"] = int(num_q_heads)
    if partners is not None:
        base["partners"] = int(partners)
    if page_size is not None:
        base["page_size"] = int(page_size)
    if new_lengths is not None and name != "mixed":
        new = np.asarray(new_lengths, dtype=np.int64)
    if bucket is None:
        bucket = int(new.sum())

    # Pages cover the prior context plus the in-step tokens (they are written to the pool after this step).
    tokens = ctx + (new if base["own_token"] else 0)
    bt, num_pages = _block_tables(rng, tokens, base["page_size"], width=bt_width)
    if pad_rows:
        ctx = np.concatenate([ctx, np.zeros(pad_rows, dtype=np.int64)])
        new = np.concatenate([new, np.zeros(pad_rows, dtype=np.int64)])
        bt = np.concatenate([bt, np.zeros((pad_rows, bt.shape[1]), dtype=np.int32)])
        notes.append(f"{pad_rows} padding rows (no tokens, no context, block table on the sink)")
    fp8 = {}
    if kv_dtype == "fp8":
        if base["dtype"] != "bf16":
            raise ValueError("fp8 pools are built for bf16 workloads")
        # GQA: separate K and V descales; MLA: the latent rows (keys, and values as their first columns) share one.
        fp8 = dict(kv_dtype="fp8", k_descale=0.0173, v_descale=0.0291) if base["kind"] == "gqa" else \
            dict(kv_dtype="fp8", k_descale=0.0091, v_descale=0.0091)
    return Workload(name=name, seed=seed, ctx_len=ctx.astype(np.int32), new_len=new.astype(np.int32),
                    bucket=int(bucket), block_table=bt, num_pages=int(num_pages), pad_rows=int(pad_rows),
                    interleave=int(interleave), notes=notes, **fp8, **base)


def row_values(wl: Workload, row: int, device="cpu") -> RowValues:
    """Draw row ``row``'s values on ``device`` (same seed and draw order on every call)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(wl.seed * (1 << 20) + int(row))
    n = int(wl.new_len[row])
    c = int(wl.ctx_len[row])
    dt = wl.torch_dtype

    def draw(*shape, descale=None):
        x = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
        if wl.std != 1.0:
            x = x * wl.std
        if descale is not None:     # fp8 pool contents: E4M3 codes of x / descale
            return (x / descale).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
        return x.to(dt)

    q = draw(n, wl.num_q_heads, wl.head_dim)
    if wl.kind == "mla":
        lat = draw(c, 1, wl.head_dim, descale=wl.k_descale if wl.kv_dtype == "fp8" else None)
        lat_new = draw(n, 1, wl.head_dim) if wl.own_token else None
        return RowValues(q=q, k_ctx=lat, v_ctx=lat[..., :wl.head_dim_v],
                         k_new=lat_new, v_new=None if lat_new is None else lat_new[..., :wl.head_dim_v])
    fp8 = wl.kv_dtype == "fp8"
    k_ctx = draw(c, wl.num_kv_heads, wl.head_dim, descale=wl.k_descale if fp8 else None)
    v_ctx = draw(c, wl.num_kv_heads, wl.head_dim_v, descale=wl.v_descale if fp8 else None)
    if wl.own_token:
        k_new = draw(n, wl.num_kv_heads, wl.head_dim)
        v_new = draw(n, wl.num_kv_heads, wl.head_dim_v)
    else:
        k_new = v_new = None
    return RowValues(q=q, k_ctx=k_ctx, v_ctx=v_ctx, k_new=k_new, v_new=v_new)


def describe(wl: Workload) -> dict:
    """A JSON-friendly summary of the workload recipe."""
    return {
        "workload": wl.name, "kind": wl.kind, "dtype": wl.dtype, "batch": wl.batch,
        "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads, "head_dim": wl.head_dim,
        "head_dim_v": wl.head_dim_v, "page_size": wl.page_size, "partners": wl.partners,
        "ctx_tokens": int(wl.ctx_len.astype(np.int64).sum()), "query_tokens": wl.num_tokens,
        "bucket": wl.bucket, "seed": wl.seed, "std": wl.std,
    }


def shrink(wl: Workload, **kw) -> Workload:
    return replace(wl, **kw)
