"""Resident stripe pools for a batch: allocate the P pools and write every row's context through ``kv_write``.

A paged KV manager names each context token by its logical slot, page_id * page_size + offset, with the page id from
the row's block table; the library's write path (slot map fused with the copy) places it in its partner's pool. All P
pools live on one device, as one tensor with a leading stripe axis.

Storage layouts:
* GQA "hnd": [P, num_pages, Hkv, pp, D] (a page's slots of one head are contiguous), passed to the kernels as the
  [stripe, page, slot, head, dim] view ``storage.transpose(2, 3)``.
* GQA "hnd_kv": [P, num_pages, Hkv, 2, pp, D]: the K block and the V block of one (page, kv head) are adjacent, so a
  head's share of a page is one contiguous run (K and V views share their strides).
* GQA "nhd": [P, num_pages, pp, Hkv, D].
* MLA: [P, num_pages, pp, 576] latent rows.
Slots that hold no token (the sink page 0, unused pages, tail slots) keep ``fill``: NaN for parity runs, so that any
read of them shows, zero for timing runs.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from . import api


@dataclass
class Batch:
    wl: object
    q: torch.Tensor                 # [bucket, Hq, D]
    q_row_start: torch.Tensor       # int32 [B + 1]
    ctx_len: torch.Tensor           # int32 [B]
    block_table: torch.Tensor       # int32 [B, max_pages]
    k_store: torch.Tensor
    v_store: torch.Tensor | None
    k_pool: torch.Tensor            # [P, pages, pp, Hkv, D] view (MLA: [P, pages, pp, 576])
    v_pool: torch.Tensor
    k_new: torch.Tensor | None      # [bucket, Hkv, D] in-step keys (own-token rows)
    v_new: torch.Tensor | None
    cu_seqlens: torch.Tensor        # int32 [B + 1] (same as q_row_start)
    max_ctx_len: int
    max_row_tokens: int

    @property
    def kind(self):
        return self.wl.kind


def logical_slots(block_table_row: torch.Tensor, ntok: int, page_size: int) -> torch.Tensor:
    """Logical slot of positions 0..ntok-1 of one row: page id from the block table times page_size plus offset."""
    t = torch.arange(ntok, device=block_table_row.device, dtype=torch.int64)
    return block_table_row.to(torch.int64)[t // page_size] * page_size + t % page_size


def build_batch(wl, device="cuda", *, fill=float("nan"), layout="hnd", rows=None, q_fill=None) -> Batch:
    """Allocate the stripe pools for ``wl``, draw every row's values on ``device`` and write them in.

    ``q_fill`` fills padding query tokens and padding in-step K/V (defaults to ``fill``).
    """
    import workloads

    P, ps = wl.partners, wl.page_size
    pp = ps // P
    dt = wl.torch_dtype
    dev = torch.device(device)
    q_fill = fill if q_fill is None else q_fill
    pdt = torch.float8_e4m3fn if getattr(wl, "kv_dtype", "same") == "fp8" else dt   # pool element type
    if wl.kind == "mla":
        k_store = torch.full((P, wl.num_pages, pp, wl.head_dim), fill, dtype=pdt, device=dev)
        v_store = None
        k_pool = v_pool = k_store
    elif layout == "hnd":
        k_store = torch.full((P, wl.num_pages, wl.num_kv_heads, pp, wl.head_dim), fill, dtype=pdt, device=dev)
        v_store = torch.full((P, wl.num_pages, wl.num_kv_heads, pp, wl.head_dim_v), fill, dtype=pdt, device=dev)
        k_pool, v_pool = k_store.transpose(2, 3), v_store.transpose(2, 3)
    elif layout == "hnd_kv":
        # K and V blocks of one (page, kv head) side by side: [P, num_pages, Hkv, 2, pp, D]
        if wl.head_dim != wl.head_dim_v:
            raise ValueError("the paired layout needs head_dim == head_dim_v")
        kv = torch.full((P, wl.num_pages, wl.num_kv_heads, 2, pp, wl.head_dim), fill, dtype=pdt, device=dev)
        k_store, v_store = kv, None
        k_pool, v_pool = kv[:, :, :, 0].transpose(2, 3), kv[:, :, :, 1].transpose(2, 3)
    elif layout == "nhd":
        k_store = torch.full((P, wl.num_pages, pp, wl.num_kv_heads, wl.head_dim), fill, dtype=pdt, device=dev)
        v_store = torch.full((P, wl.num_pages, pp, wl.num_kv_heads, wl.head_dim_v), fill, dtype=pdt, device=dev)
        k_pool, v_pool = k_store, v_store
    else:
        raise ValueError(f"unknown layout {layout!r}")

    T = wl.bucket
    q = torch.full((T, wl.num_q_heads, wl.head_dim), q_fill, dtype=dt, device=dev)
    k_new = v_new = None
    if wl.own_token:
        hkv = 1 if wl.kind == "mla" else wl.num_kv_heads
        k_new = torch.full((T, hkv, wl.head_dim), q_fill, dtype=dt, device=dev)
        v_new = torch.full((T, hkv, wl.head_dim_v), q_fill, dtype=dt, device=dev)
    bt = torch.from_numpy(np.ascontiguousarray(wl.block_table)).to(dev)
    qrs = wl.q_row_start
    for b in range(wl.batch) if rows is None else rows:
        c, n = int(wl.ctx_len[b]), int(wl.new_len[b])
        if c == 0 and n == 0:
            continue
        rv = workloads.row_values(wl, b, dev)
        t0 = int(qrs[b])
        q[t0:t0 + n] = rv.q
        if wl.own_token:
            k_new[t0:t0 + n] = rv.k_new
            v_new[t0:t0 + n] = rv.v_new
        if c:
            s = logical_slots(bt[b], c, ps)
            if wl.kind == "mla":
                api.kv_write(s, rv.k_ctx.reshape(c, 1, -1), None, k_pool, None, ps, P, kind="mla",
                             interleave=wl.interleave)
            else:
                api.kv_write(s, rv.k_ctx, rv.v_ctx, k_pool, v_pool, ps, P, interleave=wl.interleave)
        del rv
    ctx = torch.from_numpy(wl.ctx_len.astype(np.int32)).to(dev)
    qrs_t = torch.from_numpy(qrs.astype(np.int32)).to(dev)
    return Batch(wl=wl, q=q, q_row_start=qrs_t, ctx_len=ctx, block_table=bt, k_store=k_store, v_store=v_store,
                 k_pool=k_pool, v_pool=v_pool, k_new=k_new, v_new=v_new, cu_seqlens=qrs_t,
                 max_ctx_len=int(wl.ctx_len.max()) if wl.batch else 0,
                 max_row_tokens=int(wl.new_len.max()) if wl.batch else 0)


def run_step(batch: Batch, *, out=None, lse=None, merged=None, merged_lse=None, own_out=None, own_lse=None,
             out_dtype=torch.float32, workspace=None, stream=None, fixed_splits=False):
    """One pass of the hot path: every stripe's partial (plus the own-token partial), then the exact merge.

    Returns (merged_out [T, Hq, Dv], merged_lse [T, Hq], partial_out [P, T, Hq, Dv], partial_lse [P, T, Hq],
    own (out, lse) or None).
    """
    wl = batch.wl
    out, lse = api.paged_attn_partial(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len,
                                      batch.block_table, page_size=wl.page_size, partners=wl.partners,
                                      scale=wl.scale, kind=wl.kind, max_ctx_len=batch.max_ctx_len,
                                      max_row_tokens=batch.max_row_tokens, out=out, lse=lse, workspace=workspace,
                                      stream=stream, fixed_splits=fixed_splits, interleave=wl.interleave,
                                      k_descale=wl.k_descale, v_descale=wl.v_descale)
    outs = [out[s] for s in range(out.shape[0])]
    lses = [lse[s] for s in range(lse.shape[0])]
    own = None
    if wl.own_token:
        own = api.own_token_attn(batch.q, batch.k_new, batch.v_new, batch.cu_seqlens, scale=wl.scale,
                                 num_rows=wl.batch, max_row_tokens=batch.max_row_tokens, out=own_out, lse=own_lse,
                                 stream=stream)
        outs.append(own[0])
        lses.append(own[1])
    mo, ml = api.lse_merge(outs, lses, out_dtype=out_dtype, out=merged, lse_out=merged_lse, stream=stream)
    return mo, ml, out, lse, own


class StepPlan:
    """A prepared hot-path step for one batch: argument structs are built once, each run() is 1-3 C calls.

    Outputs (partials, own-token partial, merged result) are allocated once and overwritten by every run. With
    ``pad_lse_only`` (the default, CPATTN_FLAG_PAD_LSE_ONLY) the partials of padding tokens get their -inf lse only;
    the merge, told the real token count, writes the padding tokens' merged output as (0, -inf) without reading them.
    """

    def __init__(self, batch: Batch, out_dtype=torch.float32, stream=None, fixed_splits=False, fused=True,
                 pad_lse_only=True):
        import ctypes as C
        from . import _lib

        self.batch = batch
        wl = batch.wl
        self.lib = _lib.load()
        self.C = C
        dev = batch.q.device
        T, Hq = batch.q.shape[0], batch.q.shape[1]
        Dv = 512 if wl.kind == "mla" else batch.v_pool.shape[4]
        P = wl.partners
        self.out = torch.empty((P, T, Hq, Dv), dtype=torch.float32, device=dev)
        self.lse = torch.empty((P, T, Hq), dtype=torch.float32, device=dev)
        self.merged = torch.empty((T, Hq, Dv), dtype=out_dtype, device=dev)
        self.merged_lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
        self.paged = api._paged_args(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len,
                                     batch.block_table, page_size=wl.page_size, partners=P, scale=wl.scale,
                                     kind=wl.kind, stripe_begin=0, stripe_count=P, max_ctx_len=batch.max_ctx_len,
                                     max_row_tokens=batch.max_row_tokens, out=self.out, lse=self.lse, num_tokens=T,
                                     fixed_splits=fixed_splits, interleave=wl.interleave, k_descale=wl.k_descale,
                                     v_descale=wl.v_descale, pad_lse_only=pad_lse_only)
        n = C.c_int64(0)
        _lib.check(self.lib.cp_paged_attn_workspace_size(C.byref(self.paged), C.byref(n)))
        self.workspace_bytes = int(n.value)
        self.workspace = torch.zeros(max(1, self.workspace_bytes), dtype=torch.uint8, device=dev)
        if self.workspace_bytes:
            self.paged.workspace = self.workspace.data_ptr()
            self.paged.workspace_bytes = self.workspace_bytes
        outs = [self.out[s] for s in range(P)]
        lses = [self.lse[s] for s in range(P)]
        self.own = None
        if wl.own_token:
            self.own_out = torch.empty((T, Hq, batch.k_new.shape[2]), dtype=torch.float32, device=dev)
            self.own_lse = torch.empty((T, Hq), dtype=torch.float32, device=dev)
            a = api.OwnArgs()
            a.dtype = api._dtype_code(batch.q.dtype)
            a.num_rows, a.bucket_tokens = wl.batch, T
            a.num_q_heads, a.num_kv_heads, a.head_dim = Hq, batch.k_new.shape[1], batch.k_new.shape[2]
            a.scale, a.max_row_tokens = float(wl.scale), batch.max_row_tokens
            a.flags = _lib.CPATTN_FLAG_PAD_LSE_ONLY if pad_lse_only else 0
            a.cu_seqlens, a.q = batch.cu_seqlens.data_ptr(), batch.q.data_ptr()
            a.q_stride_token, a.q_stride_head = batch.q.stride(0), batch.q.stride(1)
            a.k, a.v = batch.k_new.data_ptr(), batch.v_new.data_ptr()
            a.kv_stride_token, a.kv_stride_head = batch.k_new.stride(0), batch.k_new.stride(1)
            a.out, a.out_stride_token, a.out_stride_head = self.own_out.data_ptr(), self.own_out.stride(0), \
                self.own_out.stride(1)
            a.lse, a.lse_stride_token = self.own_lse.data_ptr(), self.own_lse.stride(0)
            self.own = a
            outs.append(self.own_out)
            lses.append(self.own_lse)
        m = api.MergeArgs()
        m.num_partials, m.num_tokens, m.num_heads, m.head_dim_v = len(outs), T, Hq, Dv
        m.out_dtype = api._dtype_code(out_dtype)
        for i, (o, l) in enumerate(zip(outs, lses)):
            m.part_out[i], m.part_lse[i] = o.data_ptr(), l.data_ptr()
            m.part_out_stride_token[i], m.part_out_stride_head[i] = o.stride(0), o.stride(1)
            m.part_lse_stride_token[i], m.part_lse_stride_head[i] = l.stride(0), l.stride(1)
        m.out, m.out_stride_token, m.out_stride_head = self.merged.data_ptr(), self.merged.stride(0), \
            self.merged.stride(1)
        m.lse_out, m.lse_out_stride_token = self.merged_lse.data_ptr(), self.merged_lse.stride(0)
        # The bucket's real token count (last entry of q_row_start): padding tokens are written as (0, -inf) without
        # reading their partials.
        self._token_count = batch.q_row_start[-1:]
        m.token_count = self._token_count.data_ptr()
        self.merge = m
        self._check = _lib.check
        self.stream = stream
        # Without an own-token partial every merged partial is a stripe's: one cp_paged_attn_merged call computes them
        # and merges them (the same bits as the partial call followed by the merge call).
        self.fused = bool(fused) and self.own is None
        self.merged_out = api._merge_out(self.merged, self.merged_lse)

    def _s(self):
        s = torch.cuda.current_stream() if self.stream is None else self.stream
        return self.C.c_void_p(s.cuda_stream)

    def partial(self):
        """The partial call (with the fused plan: the merged call, which also writes the merged output)."""
        if self.fused:
            self._check(self.lib.cp_paged_attn_merged(self.C.byref(self.paged), self.C.byref(self.merged_out),
                                                      self._s()))
        else:
            self._check(self.lib.cp_paged_attn_partial(self.C.byref(self.paged), self._s()))

    def own_token(self):
        if self.own is not None:
            self._check(self.lib.cp_own_token_attn(self.C.byref(self.own), self._s()))

    def combine(self):
        """The merge call (nothing with the fused plan: the merged call did it)."""
        if not self.fused:
            self._check(self.lib.cp_lse_merge(self.C.byref(self.merge), self._s()))

    def run(self):
        self.partial()
        self.own_token()
        self.combine()
        return self.merged, self.merged_lse
