"""PyTorch-facing binding of libcpattn: shape/dtype checks and argument marshalling only.

Every computation runs in the HIP library; torch provides device memory and the current stream. Tensors must live on
the GPU. Layouts follow include/cpattn.h:

* GQA pools are 5-D tensors indexed [stripe, page, slot, kv_head, dim] (any strides, dim contiguous). The usual
  storage is head-major inside a page, [P, num_pages, Hkv, pp, D], passed as ``pool.transpose(2, 3)``.
* MLA pools are 4-D [stripe, page, slot, 576].
* Partials are [S, T, Hq, Dv] fp32 with lse [S, T, Hq] fp32 (natural log).
"""
from __future__ import annotations

import ctypes as C

import torch

from . import _lib
from ._lib import CPATTN_BF16, CPATTN_F32, CPATTN_GQA, CPATTN_MLA, MAX_PARTIALS, PagedArgs, OwnArgs, MergeArgs, MergeOut

__all__ = ["slot_map", "slot_map_rank", "kv_write", "paged_attn_partial", "paged_attn_workspace_size",
           "own_token_attn", "lse_merge", "stripe_length", "debug_gather_stripe", "version",
           "paged_attn_partial_noalloc", "noalloc_scratch_bytes", "paged_attn_merged"]


def _lib_handle():
    return _lib.load()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return C.c_void_p(s.cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else C.c_void_p(0)


def _dtype_code(dt):
    if dt == torch.float32:
        return CPATTN_F32
    if dt == torch.bfloat16:
        return CPATTN_BF16
    if dt == torch.float8_e4m3fn:
        return _lib.CPATTN_FP8_E4M3
    raise TypeError(f"unsupported dtype {dt}; expected float32, bfloat16 or float8_e4m3fn (pools and rows only)")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("cpattn tensors must live on the GPU")


def version():
    return _lib_handle().cpattn_version().decode()


def slot_map(logical_slot: torch.Tensor, page_size: int, partners: int, stream=None, *, interleave: int = 1):
    """(partner int32, physical slot int64) for each logical slot (int64; < 0 = padding -> -1, -1)."""
    lib = _lib_handle()
    _need_cuda(logical_slot)
    s = logical_slot.to(torch.int64).contiguous()
    partner = torch.empty(s.shape, dtype=torch.int32, device=s.device)
    phys = torch.empty(s.shape, dtype=torch.int64, device=s.device)
    _lib.check(lib.cp_slot_map(_ptr(s), s.numel(), int(page_size), int(partners), int(interleave), _ptr(partner),
                               _ptr(phys), _stream(stream)))
    return partner, phys


def slot_map_rank(logical_slot: torch.Tensor, page_size: int, partners: int, rank: int, sink_slot: int, stream=None,
                  *, interleave: int = 1):
    """Per-rank write slot: physical slot if `rank` owns the token, else `sink_slot`; -1 for padding."""
    lib = _lib_handle()
    _need_cuda(logical_slot)
    s = logical_slot.to(torch.int64).contiguous()
    out = torch.empty(s.shape, dtype=torch.int64, device=s.device)
    _lib.check(lib.cp_slot_map_rank(_ptr(s), s.numel(), int(page_size), int(partners), int(interleave), int(rank),
                                    int(sink_slot), _ptr(out), _stream(stream)))
    return out


def _pool_strides(pool, kind):
    if kind == "mla":
        if pool.dim() != 4 or pool.stride(3) != 1:
            raise ValueError("MLA pool must be [stripe, page, slot, 576] with a contiguous last dim")
        return pool.stride(0), pool.stride(1), pool.stride(2), 0
    if pool.dim() != 5 or pool.stride(4) != 1:
        raise ValueError("GQA pool must be [stripe, page, slot, kv_head, dim] with a contiguous last dim")
    return pool.stride(0), pool.stride(1), pool.stride(2), pool.stride(3)


def _need(cond, msg, exc=ValueError):
    if not cond:
        raise exc(msg)


def kv_write(logical_slot, k_src, v_src, k_pool, v_pool, page_size: int, partners: int, *, kind="gqa",
             stripe_begin=0, stripe_count=None, sink_slot=-1, stream=None, interleave: int = 1):
    """Write rows k_src [n, Hkv, D] (v_src [n, Hkv, Dv] or None) into the stripe pools through the slot map.

    Pools hold all P stripes (leading axis P). Rows must have the pools' element type and head shape; MLA rows are
    [n, 576] or [n, 1, 576]."""
    lib = _lib_handle()
    if kind == "mla":
        k_src = k_src.reshape(k_src.shape[0], 1, -1)
    P = int(partners)
    _need(logical_slot.dim() == 1 and not logical_slot.dtype.is_floating_point,
          "logical_slot must be a 1-D integer tensor")
    _need(k_src.dim() == 3, "k_src must be [n, Hkv, D]")
    _need(k_src.shape[0] == logical_slot.numel(), f"k_src has {k_src.shape[0]} rows for {logical_slot.numel()} slots")
    _need(k_src.dtype == k_pool.dtype, f"k_src dtype {k_src.dtype} differs from the pool's {k_pool.dtype}", TypeError)
    _need(k_pool.shape[0] == P, f"pools must hold all {P} stripes on their leading axis (got {k_pool.shape[0]})")
    if kind == "mla":
        _need(k_pool.dim() == 4 and k_src.shape[1] == 1 and k_src.shape[2] == k_pool.shape[3],
              f"MLA rows {tuple(k_src.shape)} do not fit latent pool rows of {k_pool.shape[-1]}")
        _need(v_src is None, "MLA writes latent rows only (v_src must be None)")
    else:
        _need(k_pool.dim() == 5 and tuple(k_src.shape[1:]) == (k_pool.shape[3], k_pool.shape[4]),
              f"k_src heads/dims {tuple(k_src.shape[1:])} differ from the pool's {tuple(k_pool.shape[3:])}")
        if v_src is not None:
            _need(v_pool is not None, "v_src given without v_pool")
            _need(v_src.dtype == v_pool.dtype == k_pool.dtype, "v_src and the pools must share the dtype", TypeError)
            _need(v_src.dim() == 3 and v_src.shape[0] == k_src.shape[0] and
                  tuple(v_src.shape[1:]) == (v_pool.shape[3], v_pool.shape[4]),
                  f"v_src {tuple(v_src.shape)} does not fit the value pool {tuple(v_pool.shape)}")
            _need(tuple(v_pool.shape[:4]) == tuple(k_pool.shape[:4]), "K and V pools differ in shape")
    _need_cuda(logical_slot, k_src, v_src, k_pool, v_pool)
    s = logical_slot.to(torch.int64).contiguous()
    if k_src.stride(-1) != 1 or (v_src is not None and v_src.stride(-1) != 1):
        raise ValueError("source rows must have a contiguous last dim")
    if v_src is not None and (v_src.stride(0) != k_src.stride(0) or v_src.stride(1) != k_src.stride(1)):
        v_src = v_src.contiguous()
        k_src = k_src.contiguous()
    ss, sp, sl, sh = _pool_strides(k_pool, kind)
    if v_pool is not None and _pool_strides(v_pool, kind) != (ss, sp, sl, sh):
        raise ValueError("K and V pools must share strides")
    sc = P - stripe_begin if stripe_count is None else int(stripe_count)
    hkv = k_src.shape[1]
    _lib.check(lib.cp_kv_write(_ptr(s), s.numel(), _ptr(k_src), _ptr(v_src), k_src.stride(0), k_src.stride(1),
                               _dtype_code(k_src.dtype), hkv, k_src.shape[2],
                               0 if v_src is None else v_src.shape[2], _ptr(k_pool),
                               _ptr(v_pool if v_pool is not None else k_pool), ss, sp, sl, sh, int(page_size), P,
                               int(interleave), k_pool.shape[1], int(stripe_begin), sc, int(sink_slot),
                               _stream(stream)))


def _paged_args(q, k_pool, v_pool, q_row_start, ctx_len, block_table, *, page_size, partners, scale, kind,
                stripe_begin, stripe_count, max_ctx_len, max_row_tokens, out, lse, num_tokens, fixed_splits=False,
                interleave=1, k_descale=1.0, v_descale=1.0, pad_lse_only=False):
    a = PagedArgs()
    a.flags = (_lib.CPATTN_FLAG_FIXED_SPLITS if fixed_splits else 0) | (_lib.CPATTN_FLAG_PAD_LSE_ONLY if pad_lse_only else 0)
    a.interleave = int(interleave)
    a.kind = CPATTN_MLA if kind == "mla" else CPATTN_GQA
    a.dtype = _dtype_code(q.dtype)
    if k_pool.dtype == torch.float8_e4m3fn:
        # fp8 pools: codes dequantized with the per-tensor descales
        a.kv_format = _lib.CPATTN_KV_FP8_E4M3
        a.k_descale, a.v_descale = float(k_descale), float(v_descale)
    elif k_pool.dtype != q.dtype:
        raise TypeError("q and the pools must share a dtype (or the pools hold float8_e4m3fn codes)")
    a.num_rows = ctx_len.numel()
    a.num_tokens = num_tokens
    a.num_partners = int(partners)
    a.stripe_begin = int(stripe_begin)
    a.stripe_count = int(stripe_count)
    a.page_size = int(page_size)
    a.num_pages = k_pool.shape[1]
    a.num_q_heads = q.shape[1]
    if kind == "mla":
        a.num_kv_heads = 1
        a.head_dim = k_pool.shape[3]
        a.head_dim_v = 512
    else:
        a.num_kv_heads = k_pool.shape[3]
        a.head_dim = k_pool.shape[4]
        a.head_dim_v = v_pool.shape[4]
    a.scale = float(scale)
    a.max_ctx_len = int(max_ctx_len)
    a.max_row_tokens = int(max_row_tokens)
    a.max_pages = block_table.shape[1]
    a.q_row_start = q_row_start.data_ptr()
    a.ctx_len = ctx_len.data_ptr()
    a.block_table = block_table.data_ptr()
    a.bt_stride = block_table.stride(0)
    a.q = q.data_ptr()
    a.q_stride_token, a.q_stride_head = q.stride(0), q.stride(1)
    a.k_pool = k_pool.data_ptr()
    a.v_pool = v_pool.data_ptr()
    a.kv_stride_stripe, a.kv_stride_page, a.kv_stride_slot, a.kv_stride_head = _pool_strides(k_pool, kind)
    if out is not None:
        a.out = out.data_ptr()
        a.out_stride_stripe, a.out_stride_token, a.out_stride_head = out.stride(0), out.stride(1), out.stride(2)
        a.lse = lse.data_ptr()
        a.lse_stride_stripe, a.lse_stride_token = lse.stride(0), lse.stride(1)
    return a


class _Workspace:
    """Per-device zero-initialised scratch for split chunks; grown on demand, kept for reuse."""

    def __init__(self):
        self.buf = {}

    def get(self, device, nbytes):
        if nbytes <= 0:
            return None
        cur = self.buf.get(device)
        if cur is None or cur.numel() < nbytes:
            cur = torch.zeros(int(nbytes), dtype=torch.uint8, device=device)
            self.buf[device] = cur
        return cur


_WS = _Workspace()


def _check_int32_dev(*ts):
    for t in ts:
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise TypeError("row offsets, lengths and block tables must be contiguous int32 tensors")


def _validate_paged(q, k_pool, v_pool, q_row_start, ctx_len, block_table, kind, P, S, out, lse):
    """Shape and dtype checks of a partial call, made before anything reaches the library."""
    _need(q.dim() == 3 and q.stride(2) == 1, "q must be [T, Hq, D] with a contiguous last dim")
    if kind == "mla":
        _need(k_pool.dim() == 4, "MLA pool must be [stripe, page, slot, 576]")
        _need(v_pool is k_pool or v_pool.data_ptr() == k_pool.data_ptr(), "MLA values are the latent rows: "
              "v_pool must be k_pool")
        _need(q.shape[2] == k_pool.shape[3], f"q head dim {q.shape[2]} differs from the latent rows' {k_pool.shape[3]}")
        Dv = 512
    else:
        _need(k_pool.dim() == 5 and v_pool is not None and v_pool.dim() == 5,
              "GQA pools must be [stripe, page, slot, kv_head, dim]")
        _need(tuple(v_pool.shape[:4]) == tuple(k_pool.shape[:4]), "K and V pools differ in shape")
        _need(q.shape[2] == k_pool.shape[4], f"q head dim {q.shape[2]} differs from the pool's {k_pool.shape[4]}")
        _need(q.shape[1] % k_pool.shape[3] == 0, f"{q.shape[1]} query heads over {k_pool.shape[3]} kv heads")
        _need(v_pool.dtype == k_pool.dtype, "K and V pools must share a dtype", TypeError)
        Dv = v_pool.shape[4]
    _need(k_pool.shape[0] == P, f"pools must hold all {P} stripes on their leading axis (got {k_pool.shape[0]})")
    if k_pool.dtype == torch.float8_e4m3fn:
        _need(q.dtype == torch.bfloat16, "fp8 pools are read with bf16 queries", TypeError)
    else:
        _need(k_pool.dtype == q.dtype, "q and the pools must share a dtype (or the pools hold float8_e4m3fn codes)",
              TypeError)
    _check_int32_dev(q_row_start, ctx_len, block_table)
    B = ctx_len.numel()
    _need(ctx_len.dim() == 1, "ctx_len must be 1-D [B]")
    _need(q_row_start.dim() == 1 and q_row_start.numel() == B + 1,
          f"q_row_start must have B + 1 = {B + 1} entries (got {q_row_start.numel()})")
    _need(block_table.dim() == 2 and block_table.shape[0] >= B,
          f"block_table must be [>= {B}, max_pages] (got {tuple(block_table.shape)})")
    T, Hq = q.shape[0], q.shape[1]
    if out is not None:
        _need(out.dtype == torch.float32 and tuple(out.shape) == (S, T, Hq, Dv) and out.stride(3) == 1,
              f"out must be fp32 [{S}, {T}, {Hq}, {Dv}] with a contiguous last dim (got {out.dtype} "
              f"{tuple(out.shape)})")
    if lse is not None:
        _need(lse.dtype == torch.float32 and tuple(lse.shape) == (S, T, Hq) and lse.stride(2) == 1,
              f"lse must be fp32 [{S}, {T}, {Hq}] with a contiguous last dim (got {lse.dtype} {tuple(lse.shape)})")
    _need((out is None) == (lse is None), "give both out and lse, or neither")


def paged_attn_workspace_size(q, k_pool, v_pool, q_row_start, ctx_len, block_table, *, page_size, partners, scale,
                              kind="gqa", stripe_begin=0, stripe_count=None, max_ctx_len, max_row_tokens,
                              fixed_splits=False, interleave=1, k_descale=1.0, v_descale=1.0):
    lib = _lib_handle()
    sc = int(partners) - stripe_begin if stripe_count is None else stripe_count
    a = _paged_args(q, k_pool, v_pool, q_row_start, ctx_len, block_table, page_size=page_size, partners=partners,
                    scale=scale, kind=kind, stripe_begin=stripe_begin, stripe_count=sc, max_ctx_len=max_ctx_len,
                    max_row_tokens=max_row_tokens, out=None, lse=None, num_tokens=q.shape[0],
                    fixed_splits=fixed_splits, interleave=interleave, k_descale=k_descale, v_descale=v_descale)
    n = C.c_int64(0)
    _lib.check(lib.cp_paged_attn_workspace_size(C.byref(a), C.byref(n)))
    return int(n.value)


def paged_attn_partial(q, k_pool, v_pool, q_row_start, ctx_len, block_table, *, page_size, partners, scale,
                       kind="gqa", stripe_begin=0, stripe_count=None, max_ctx_len=None, max_row_tokens=None,
                       out=None, lse=None, workspace=None, stream=None, fixed_splits=False, interleave=1,
                       k_descale=1.0, v_descale=1.0):
    """Per-stripe partials (out [S, T, Hq, Dv] fp32, lse [S, T, Hq] fp32) of attention over the striped pool.

    q [T, Hq, D]; q_row_start int32 [B + 1]; ctx_len int32 [B]; block_table int32 [B, max_pages]. ``max_ctx_len``
    and ``max_row_tokens`` are host upper bounds (read from the device with a sync when omitted). ``fixed_splits``
    makes each row's result independent, to the bit, of the rest of the call (CPATTN_FLAG_FIXED_SPLITS).
    ``interleave`` is the KV-cache interleave size the pool was written with (runs of that many slots per partner).
    float8_e4m3fn pools hold fp8 codes; ``k_descale``/``v_descale`` are their per-tensor descales.
    """
    lib = _lib_handle()
    if kind == "mla" and v_pool is None:
        v_pool = k_pool
    sc = int(partners) - stripe_begin if stripe_count is None else int(stripe_count)
    _validate_paged(q, k_pool, v_pool, q_row_start, ctx_len, block_table, kind, int(partners), sc, out, lse)
    _need_cuda(q, k_pool, v_pool, q_row_start, ctx_len, block_table, out, lse)
    T, Hq = q.shape[0], q.shape[1]
    Dv = 512 if kind == "mla" else v_pool.shape[4]
    if max_ctx_len is None:
        max_ctx_len = int(ctx_len.max().item()) if ctx_len.numel() else 0
    if max_row_tokens is None:
        max_row_tokens = int((q_row_start[1:] - q_row_start[:-1]).max().item()) if ctx_len.numel() else 0
    if out is None:
        out = torch.empty((sc, T, Hq, Dv), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((sc, T, Hq), dtype=torch.float32, device=q.device)
    a = _paged_args(q, k_pool, v_pool, q_row_start, ctx_len, block_table, page_size=page_size, partners=partners,
                    scale=scale, kind=kind, stripe_begin=stripe_begin, stripe_count=sc, max_ctx_len=max_ctx_len,
                    max_row_tokens=max_row_tokens, out=out, lse=lse, num_tokens=T, fixed_splits=fixed_splits,
                    interleave=interleave, k_descale=k_descale, v_descale=v_descale)
    n = C.c_int64(0)
    _lib.check(lib.cp_paged_attn_workspace_size(C.byref(a), C.byref(n)))
    if n.value > 0:
        ws = workspace if workspace is not None else _WS.get(q.device, n.value)
        if ws.numel() * ws.element_size() < n.value:
            raise ValueError(f"workspace too small: {n.value} bytes needed")
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel() * ws.element_size()
    _lib.check(lib.cp_paged_attn_partial(C.byref(a), _stream(stream)))
    return out, lse


def paged_attn_merged(q, k_pool, v_pool, q_row_start, ctx_len, block_table, *, page_size, partners, scale,
                      kind="gqa", max_ctx_len=None, max_row_tokens=None, out=None, lse=None, merged=None,
                      merged_lse=None, out_dtype=torch.float32, workspace=None, stream=None, fixed_splits=False,
                      interleave=1, k_descale=1.0, v_descale=1.0):
    """cp_paged_attn_merged: every stripe's partial (into ``out``/``lse``) and their exact merge (into ``merged`` [T,
    Hq, Dv] of ``out_dtype`` and ``merged_lse`` [T, Hq]) in one call; all P stripes are attended. The same bits as
    :func:`paged_attn_partial` followed by :func:`lse_merge` with the real token count.

    Returns (merged, merged_lse, out, lse)."""
    lib = _lib_handle()
    if kind == "mla" and v_pool is None:
        v_pool = k_pool
    P = int(partners)
    _validate_paged(q, k_pool, v_pool, q_row_start, ctx_len, block_table, kind, P, P, out, lse)
    T, Hq = q.shape[0], q.shape[1]
    Dv = 512 if kind == "mla" else v_pool.shape[4]
    if merged is not None:
        _need(merged.dtype in (torch.float32, torch.bfloat16) and tuple(merged.shape) == (T, Hq, Dv) and
              merged.stride(2) == 1, f"merged must be fp32 or bf16 [{T}, {Hq}, {Dv}] with a contiguous last dim")
    if merged_lse is not None:
        _need(merged_lse.dtype == torch.float32 and tuple(merged_lse.shape) == (T, Hq) and merged_lse.stride(1) == 1,
              f"merged_lse must be fp32 [{T}, {Hq}] with a contiguous last dim")
    _need_cuda(q, k_pool, v_pool, q_row_start, ctx_len, block_table, out, lse, merged, merged_lse)
    if max_ctx_len is None:
        max_ctx_len = int(ctx_len.max().item()) if ctx_len.numel() else 0
    if max_row_tokens is None:
        max_row_tokens = int((q_row_start[1:] - q_row_start[:-1]).max().item()) if ctx_len.numel() else 0
    if out is None:
        out = torch.empty((P, T, Hq, Dv), dtype=torch.float32, device=q.device)
        lse = torch.empty((P, T, Hq), dtype=torch.float32, device=q.device)
    if merged is None:
        merged = torch.empty((T, Hq, Dv), dtype=out_dtype, device=q.device)
    if merged_lse is None:
        merged_lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    a = _paged_args(q, k_pool, v_pool, q_row_start, ctx_len, block_table, page_size=page_size, partners=P,
                    scale=scale, kind=kind, stripe_begin=0, stripe_count=P, max_ctx_len=max_ctx_len,
                    max_row_tokens=max_row_tokens, out=out, lse=lse, num_tokens=T, fixed_splits=fixed_splits,
                    interleave=interleave, k_descale=k_descale, v_descale=v_descale)
    n = C.c_int64(0)
    _lib.check(lib.cp_paged_attn_workspace_size(C.byref(a), C.byref(n)))
    if n.value > 0:
        ws = workspace if workspace is not None else _WS.get(q.device, n.value)
        if ws.numel() * ws.element_size() < n.value:
            raise ValueError(f"workspace too small: {n.value} bytes needed")
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel() * ws.element_size()
    m = _merge_out(merged, merged_lse)
    _lib.check(lib.cp_paged_attn_merged(C.byref(a), C.byref(m), _stream(stream)))
    return merged, merged_lse, out, lse


def _merge_out(merged, merged_lse):
    m = MergeOut()
    m.out_dtype = _dtype_code(merged.dtype)
    m.out = merged.data_ptr()
    m.out_stride_token, m.out_stride_head = merged.stride(0), merged.stride(1)
    if merged_lse is not None:
        m.lse = merged_lse.data_ptr()
        m.lse_stride_token = merged_lse.stride(0)
    return m


def paged_attn_partial_noalloc(q, k_pool, v_pool, q_row_start, ctx_len, block_table, *, page_size, partners, scale,
                               kind="gqa", stripe_begin=0, stripe_count=None, max_ctx_len, max_row_tokens, out, lse,
                               stream=None, fixed_splits=False, interleave=1, k_descale=1.0, v_descale=1.0):
    """cp_paged_attn_partial_noalloc: the partial call with the library's static device scratch as its workspace.

    Allocates nothing: the caller passes ``out`` [S, T, Hq, Dv] and ``lse`` [S, T, Hq] (fp32) and the host bounds
    ``max_ctx_len`` and ``max_row_tokens`` (no device read)."""
    lib = _lib_handle()
    if kind == "mla" and v_pool is None:
        v_pool = k_pool
    sc = int(partners) - stripe_begin if stripe_count is None else int(stripe_count)
    _need(out is not None and lse is not None, "the no-allocation call writes into caller-provided out and lse")
    _validate_paged(q, k_pool, v_pool, q_row_start, ctx_len, block_table, kind, int(partners), sc, out, lse)
    _need_cuda(q, k_pool, v_pool, q_row_start, ctx_len, block_table, out, lse)
    a = _paged_args(q, k_pool, v_pool, q_row_start, ctx_len, block_table, page_size=page_size, partners=partners,
                    scale=scale, kind=kind, stripe_begin=stripe_begin, stripe_count=sc, max_ctx_len=max_ctx_len,
                    max_row_tokens=max_row_tokens, out=out, lse=lse, num_tokens=q.shape[0],
                    fixed_splits=fixed_splits, interleave=interleave, k_descale=k_descale, v_descale=v_descale)
    _lib.check(lib.cp_paged_attn_partial_noalloc(C.byref(a), _stream(stream)))
    return out, lse


def noalloc_scratch_bytes() -> int:
    return int(_lib_handle().cp_paged_attn_noalloc_scratch_bytes())


def own_token_attn(q, k, v, cu_seqlens, *, scale, num_rows=None, max_row_tokens=None, out=None, lse=None,
                   stream=None):
    """Causal attention of each row's in-step queries over its in-step K/V: out [T, Hq, D] fp32, lse [T, Hq]."""
    lib = _lib_handle()
    _need(q.dim() == 3 and k.dim() == 3 and v.dim() == 3, "q, k, v must be [T, H, D]")
    T, Hq, D = q.shape
    _need(q.dtype == k.dtype == v.dtype, "q, k and v must share a dtype", TypeError)
    _need(k.shape[0] == T and tuple(v.shape) == tuple(k.shape) and k.shape[2] == D,
          f"k {tuple(k.shape)} and v {tuple(v.shape)} must be [{T}, Hkv, {D}]")
    _need(Hq % k.shape[1] == 0, f"{Hq} query heads over {k.shape[1]} kv heads")
    _check_int32_dev(cu_seqlens)
    B = cu_seqlens.numel() - 1 if num_rows is None else int(num_rows)
    _need(cu_seqlens.dim() == 1 and 0 <= B <= cu_seqlens.numel() - 1,
          f"cu_seqlens must hold num_rows + 1 = {B + 1} entries (got {cu_seqlens.numel()})")
    if out is not None:
        _need(out.dtype == torch.float32 and tuple(out.shape) == (T, Hq, D) and out.stride(2) == 1,
              f"out must be fp32 [{T}, {Hq}, {D}] with a contiguous last dim")
    if lse is not None:
        _need(lse.dtype == torch.float32 and tuple(lse.shape) == (T, Hq) and lse.stride(1) == 1,
              f"lse must be fp32 [{T}, {Hq}] with a contiguous last dim")
    _need_cuda(q, k, v, cu_seqlens, out, lse)
    if q.stride(2) != 1 or k.stride(2) != 1 or v.stride(2) != 1 or k.stride() != v.stride():
        raise ValueError("q/k/v need contiguous last dims and k, v the same strides")
    if max_row_tokens is None:
        max_row_tokens = int((cu_seqlens[1:B + 1] - cu_seqlens[:B]).max().item()) if B > 0 else 0
    if out is None:
        out = torch.empty((T, Hq, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((T, Hq), dtype=torch.float32, device=q.device)
    a = OwnArgs()
    a.dtype = _dtype_code(q.dtype)
    a.num_rows = B
    a.bucket_tokens = T
    a.num_q_heads = Hq
    a.num_kv_heads = k.shape[1]
    a.head_dim = D
    a.scale = float(scale)
    a.max_row_tokens = int(max_row_tokens)
    a.cu_seqlens = cu_seqlens.data_ptr()
    a.q = q.data_ptr()
    a.q_stride_token, a.q_stride_head = q.stride(0), q.stride(1)
    a.k, a.v = k.data_ptr(), v.data_ptr()
    a.kv_stride_token, a.kv_stride_head = k.stride(0), k.stride(1)
    a.out = out.data_ptr()
    a.out_stride_token, a.out_stride_head = out.stride(0), out.stride(1)
    a.lse = lse.data_ptr()
    a.lse_stride_token = lse.stride(0)
    _lib.check(lib.cp_own_token_attn(C.byref(a), _stream(stream)))
    return out, lse


def lse_merge(outs, lses, *, out_dtype=torch.float32, out=None, lse_out=None, token_count=None, stream=None):
    """Exact LSE merge of N partials: outs is a list of [T, H, Dv] fp32, lses a list of [T, H] fp32."""
    lib = _lib_handle()
    n = len(outs)
    if n != len(lses) or not 1 <= n <= MAX_PARTIALS:
        raise ValueError(f"need 1..{MAX_PARTIALS} partials with matching lses")
    _need(outs[0].dim() == 3, "partials must be [T, H, Dv]")
    T, H, Dv = outs[0].shape
    for o, l in zip(outs, lses):
        _need(o.dtype == torch.float32 and l.dtype == torch.float32, "partials and lses must be fp32", TypeError)
        _need(tuple(o.shape) == (T, H, Dv) and o.stride(2) == 1,
              "partials must be fp32 [T, H, Dv] with a contiguous last dim")
        _need(tuple(l.shape) == (T, H), f"partial lses must be [{T}, {H}] (got {tuple(l.shape)})")
    if out is not None:
        _need(out.dtype in (torch.float32, torch.bfloat16) and tuple(out.shape) == (T, H, Dv) and out.stride(2) == 1,
              f"out must be fp32 or bf16 [{T}, {H}, {Dv}] with a contiguous last dim")
    if lse_out is not None:
        _need(lse_out.dtype == torch.float32 and tuple(lse_out.shape) == (T, H) and lse_out.stride(1) == 1,
              f"lse_out must be fp32 [{T}, {H}] with a contiguous last dim")
    if token_count is not None:
        _need(token_count.dtype == torch.int32 and token_count.numel() >= 1, "token_count must be int32 [1]",
              TypeError)
    _need_cuda(*outs, *lses, out, lse_out, token_count)
    if out is None:
        out = torch.empty((T, H, Dv), dtype=out_dtype, device=outs[0].device)
    if lse_out is None:
        lse_out = torch.empty((T, H), dtype=torch.float32, device=outs[0].device)
    a = MergeArgs()
    a.num_partials, a.num_tokens, a.num_heads, a.head_dim_v = n, T, H, Dv
    a.out_dtype = _dtype_code(out.dtype)
    a.token_count = token_count.data_ptr() if token_count is not None else None
    for i, (o, l) in enumerate(zip(outs, lses)):
        a.part_out[i] = o.data_ptr()
        a.part_lse[i] = l.data_ptr()
        a.part_out_stride_token[i], a.part_out_stride_head[i] = o.stride(0), o.stride(1)
        a.part_lse_stride_token[i], a.part_lse_stride_head[i] = l.stride(0), l.stride(1)
    a.out = out.data_ptr()
    a.out_stride_token, a.out_stride_head = out.stride(0), out.stride(1)
    a.lse_out = lse_out.data_ptr()
    a.lse_out_stride_token = lse_out.stride(0)
    _lib.check(lib.cp_lse_merge(C.byref(a), _stream(stream)))
    return out, lse_out


def stripe_length(ctx_len: int, page_size: int, partners: int, r: int, *, interleave: int = 1) -> int:
    """Context tokens of a row that stripe r holds, by the library's own rule (cp_stripe_length)."""
    lib = _lib_handle()
    n = C.c_int32(-1)
    _lib.check(lib.cp_stripe_length(int(ctx_len), int(page_size), int(partners), int(interleave), int(r),
                                    C.byref(n)))
    return int(n.value)


def debug_gather_stripe(k_pool, block_table_row, ctx_len: int, page_size: int, partners: int, r: int, *,
                        kind="gqa", stream=None, interleave: int = 1):
    """Stripe r's keys of one row in local order, read with the kernels' own addressing: [Lr, Hkv, D].

    The row count comes from the library (cp_stripe_length) and the gather reports how many rows it wrote; the two
    must agree."""
    lib = _lib_handle()
    _need_cuda(k_pool, block_table_row)
    _check_int32_dev(block_table_row)
    ss, sp, sl, sh = _pool_strides(k_pool, kind)
    hkv = 1 if kind == "mla" else k_pool.shape[3]
    D = k_pool.shape[-1]
    P, I = int(partners), int(interleave)
    Lr = stripe_length(ctx_len, page_size, P, r, interleave=I)
    dst = torch.empty((Lr, hkv, D), dtype=k_pool.dtype, device=k_pool.device)
    rows = C.c_int32(-1)
    _lib.check(lib.cp_debug_gather_stripe(_ptr(k_pool), _dtype_code(k_pool.dtype), ss, sp, sl, sh, k_pool.shape[1],
                                          _ptr(block_table_row), int(ctx_len), int(page_size), P, I, int(r), hkv,
                                          D, _ptr(dst), Lr, C.byref(rows), _stream(stream)))
    if rows.value != Lr:
        raise RuntimeError(f"cp_debug_gather_stripe wrote {rows.value} rows, cp_stripe_length said {Lr}")
    return dst


def debug_stream_read(buf, *, sink=None, stream=None):
    """Read the bytes of the contiguous device tensor ``buf`` once (the streaming-read reference kernel).

    Returns the int32 sink: one XOR word per workgroup (2048 by default, or ``sink.numel()`` words)."""
    lib = _lib_handle()
    _need_cuda(buf)
    if not buf.is_contiguous():
        raise ValueError("debug_stream_read: buf must be contiguous")
    if sink is None:
        sink = torch.empty(2048, dtype=torch.int32, device=buf.device)
    _lib.check(lib.cp_debug_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink), sink.numel(),
                                        _stream(stream)))
    return sink
