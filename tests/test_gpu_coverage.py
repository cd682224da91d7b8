"""GPU parity of paths the workload-shaped tests do not reach: padded decode and MLA buckets, one rank's write view
with the sink slot, and the generic kernels (fp32 pools and queries, head dim 64) of the partial and own-token calls.
Everything goes through the C ABI and is compared with the float64 oracle."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from cp_slot_map_amd import api, pool
from tests.gpu_helpers import check_padding, compare_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.view({torch.bfloat16: torch.int16, torch.float8_e4m3fn: torch.uint8, torch.float32: torch.int32}[t.dtype])


# -------------------------------------------------------------------------------------- padded buckets
# Padding rows (no tokens, no context, block table on the sink) and padding tokens past the real ones, in decode and
# MLA batches: the review thread on the padding test of mstar PR #1124 asks for a bucket larger than its real rows.
PADDED = [
    ("tiny", dict(pad_rows=2, bucket=4 + 3)),
    ("llama8b", dict(batch=4, ctx_lengths=[3, 17, 300, 2100], pad_rows=2, bucket=4 + 7)),
    ("llama8b-fp8", dict(batch=4, ctx_lengths=[3, 17, 300, 2100], pad_rows=2, bucket=4 + 7, kv_dtype="fp8")),
    ("longctx", dict(batch=3, ctx_lengths=[5, 100, 5000], pad_rows=3, bucket=3 + 9)),
    ("mla", dict(batch=3, ctx_lengths=[7, 130, 2000], pad_rows=2, bucket=3 + 5)),
    ("mla-16h", dict(batch=3, ctx_lengths=[1, 64, 700], pad_rows=2, bucket=3 + 4, num_q_heads=16)),
]


def _make(name, kw):
    return workloads.make(name.split("-")[0], **kw)


@pytest.mark.parametrize("fixed_splits", [False, True], ids=["balanced", "fixed"])
@pytest.mark.parametrize("name,kw", PADDED, ids=[p[0] for p in PADDED])
def test_padded_bucket_parity(name, kw, fixed_splits):
    """Real rows match the oracle; padding tokens come out as (0, -inf) in every partial and in the merge."""
    wl = _make(name, kw)
    say(f"padded bucket {name} fixed_splits={fixed_splits} rows={wl.batch} tokens={wl.num_tokens} bucket={wl.bucket}")
    assert wl.bucket > wl.num_tokens and wl.pad_rows >= 2
    batch = pool.build_batch(wl, DEV)                      # NaN in every padding query and unused slot
    res = pool.run_step(batch, fixed_splits=fixed_splits)
    torch.cuda.synchronize()
    w = compare_rows(wl, batch, res, range(wl.batch), DEV)
    check_padding(wl, res)
    say(f"  worst errors {w}")


@pytest.mark.parametrize("name,kw", PADDED, ids=[p[0] for p in PADDED])
def test_padded_bucket_nan_poison_is_bit_identical(name, kw):
    """NaN in padding queries, padding rows' block tables (the sink page) and unused slots changes no bit of the real
    rows, and padding outputs are (0, -inf) either way."""
    wl = _make(name, kw)
    say(f"padded bucket poison {name}")
    a = pool.run_step(pool.build_batch(wl, DEV, fill=float("nan")))
    b = pool.run_step(pool.build_batch(wl, DEV, fill=0.0))
    t = wl.num_tokens
    assert torch.equal(a[0][:t], b[0][:t]) and torch.equal(a[1][:t], b[1][:t])
    assert torch.equal(a[2][:, :t], b[2][:, :t]) and torch.equal(a[3][:, :t], b[3][:, :t])
    check_padding(wl, a)
    check_padding(wl, b)


# ------------------------------------------------------------------------------ one rank's write view
SINK = [
    ("llama8b", dict(batch=3, ctx_lengths=[1, 37, 301]), 1),
    ("llama8b", dict(batch=3, ctx_lengths=[5, 64, 333]), 2),
    ("longctx", dict(batch=2, ctx_lengths=[3, 211]), 1),
    ("mla", dict(batch=2, ctx_lengths=[5, 200]), 1),
    ("mla", dict(batch=2, ctx_lengths=[70, 333]), 4),
]


@pytest.mark.parametrize("name,kw,I", SINK, ids=[f"{n}-i{i}" for n, _, i in SINK])
def test_rank_write_view_with_sink(name, kw, I):
    """cp_kv_write for one rank's stripe (stripe_count = 1) with a sink slot: every token the rank owns lands at its
    physical slot, bit for bit as the oracle's per-rank view places it; every other token goes to the sink slot (which
    therefore holds one of them); the other stripes' pools are not touched."""
    wl = workloads.make(name, interleave=I, **kw)
    P, ps = wl.partners, wl.page_size
    pp = ps // P
    sink = 1                                               # slot 1 of the sink page 0
    for rank in range(P):
        say(f"rank write view {name} I={I} rank={rank}")
        batch = pool.build_batch(wl, DEV, rows=[])           # NaN pools, nothing written yet
        rows = []
        for b in range(wl.batch):
            rv = workloads.row_values(wl, b, DEV)
            c = int(wl.ctx_len[b])
            s = pool.logical_slots(batch.block_table[b], c, ps)
            if wl.kind == "mla":
                api.kv_write(s, rv.k_ctx.reshape(c, 1, -1), None, batch.k_pool, None, ps, P, kind="mla",
                             stripe_begin=rank, stripe_count=1, sink_slot=sink, interleave=I)
            else:
                api.kv_write(s, rv.k_ctx, rv.v_ctx, batch.k_pool, batch.v_pool, ps, P, stripe_begin=rank,
                             stripe_count=1, sink_slot=sink, interleave=I)
            rows.append((s.cpu().numpy(), rv.k_ctx.reshape(c, -1).cpu()))
        torch.cuda.synchronize()
        got = batch.k_pool[rank].reshape(wl.num_pages * pp, -1).cpu()
        want = torch.full_like(got, float("nan"))
        sunk = []
        for s, k in rows:
            wslot = oracle.slot_map_rank(s, ps, P, rank, sink, I)
            for t, ws in enumerate(wslot.tolist()):
                if ws == sink:
                    sunk.append(k[t])
                elif ws >= 0:
                    want[ws] = k[t]
        keep = torch.ones(got.shape[0], dtype=torch.bool)
        keep[sink] = False
        assert torch.equal(_bits(got[keep]), _bits(want[keep])), f"rank {rank}: owned slots differ"
        if sunk:
            # tokens sharing the sink race (each wave copies its row in 16-byte pieces), so every element of the sink
            # row must come from one of the non-owned tokens
            cand = _bits(torch.stack(sunk))
            assert (cand == _bits(got[sink])[None]).any(0).all(), f"rank {rank}: sink holds a value of no token"
        else:
            assert torch.isnan(got[sink].float()).all()
        for other in range(P):                             # other stripes untouched
            if other != rank:
                assert torch.isnan(batch.k_pool[other].float()).all(), f"rank {rank} wrote stripe {other}"


# ------------------------------------------------------------------------------------- generic kernels
# Shapes the specialised kernels do not take: fp32 pools and queries (paged_generic_kernel, own_token_generic_kernel)
# and head dim 64 in bf16 (both generic kernels). The oracle sees the same rounded inputs.
_MIX = dict(batch=5, new_lengths=[1, 3, 40, 1, 130], ctx_lengths=[0, 19, 300, 1000, 2], pad_rows=2)
_D64 = dict(head_dim=64, head_dim_v=64, scale=1.0 / 8.0)
GENERIC = [
    ("paged-bf16-d64", "llama8b", dict(batch=4, ctx_lengths=[1, 17, 300, 2100]), _D64),
    ("paged-f32-d128", "llama8b", dict(batch=4, ctx_lengths=[1, 17, 300, 2100]), dict(dtype="f32")),
    ("own-f32-d128", "mixed", _MIX, dict(dtype="f32")),
    ("own-bf16-d64", "mixed", _MIX, _D64),
    ("own-f32-d64", "mixed", _MIX, dict(dtype="f32", **_D64)),
]


@pytest.mark.parametrize("case,name,kw,over", GENERIC, ids=[g[0] for g in GENERIC])
def test_generic_kernels_parity(case, name, kw, over):
    wl = dataclasses.replace(workloads.make(name, **kw), **over)
    say(f"generic {case}: dtype={wl.dtype} D={wl.head_dim} ctx={list(wl.ctx_len)} new={list(wl.new_len)}")
    batch = pool.build_batch(wl, DEV)
    res = pool.run_step(batch)
    torch.cuda.synchronize()
    w = compare_rows(wl, batch, res, range(wl.batch), DEV)
    check_padding(wl, res)
    say(f"  worst errors {w}")
    z = pool.run_step(pool.build_batch(wl, DEV, fill=0.0))  # NaN poison changes no bit
    t = wl.num_tokens
    assert torch.equal(res[0][:t], z[0][:t]) and torch.equal(res[1][:t], z[1][:t])


# ------------------------------------------------------------------------- MLA: short, peaked stripes
@pytest.mark.parametrize("heads", [16, 128])
def test_mla_short_peaked_stripes(heads):
    """Stripes of 0-3 latent rows with one row aligned to head 0's query at several strengths (peaked softmax over a
    few keys): the bf16-rounded probabilities that weight the values must be normalised by their own sum, so that
    the fp32 partials stay within 2e-3 absolute (a constant value row is reproduced exactly)."""
    wl = workloads.make("mla", batch=5, ctx_lengths=[1, 2, 3, 6, 11], num_q_heads=heads)
    say(f"mla short peaked stripes heads={heads}")
    batch = pool.build_batch(wl, DEV)
    P, ps = wl.partners, wl.page_size
    lat_rows = []
    for b, amp in enumerate([0.1, 0.2, 0.3, 0.5, 1.0]):
        rv = workloads.row_values(wl, b, DEV)
        c = int(wl.ctx_len[b])
        lat = rv.k_ctx.clone()
        lat[c - 1, 0] = (amp * torch.sign(rv.q[0, 0].float())).to(lat.dtype)
        s = pool.logical_slots(batch.block_table[b], c, ps)
        api.kv_write(s, lat, None, batch.k_pool, None, ps, P, kind="mla")
        lat_rows.append((rv.q.cpu(), lat.cpu()))
    res = pool.run_step(batch)
    torch.cuda.synchronize()
    from tests.gpu_helpers import check_lse, check_out
    for b, (q, lat) in enumerate(lat_rows):
        parts, merged = oracle.row_partials(q, lat, lat[..., :wl.head_dim_v], P, wl.scale)
        t0 = int(wl.q_row_start[b])
        for r in range(P):
            check_out(res[2][r, t0:t0 + 1], parts[r][0], f"row {b} stripe {r} out")
            check_lse(res[3][r, t0:t0 + 1], parts[r][1], f"row {b} stripe {r} lse")
        check_out(res[0][t0:t0 + 1], merged[0], f"row {b} merged out")
        check_lse(res[1][t0:t0 + 1], merged[1], f"row {b} merged lse")


# ---------------------------------------------------------------------- padding tokens: lse-only flag
PAD_FLAG = [
    ("llama8b", dict(batch=4, ctx_lengths=[3, 17, 300, 2100], pad_rows=2, bucket=4 + 7), {}, False),
    ("llama8b", dict(batch=4, ctx_lengths=[3, 17, 300, 2100], pad_rows=2, bucket=4 + 7), {}, True),
    ("mla", dict(batch=3, ctx_lengths=[7, 130, 2000], pad_rows=2, bucket=3 + 5), {}, False),
    ("tiny", dict(pad_rows=2, bucket=4 + 3), {}, False),
    ("mixed", dict(batch=5, new_lengths=[1, 3, 40, 1, 130], ctx_lengths=[0, 19, 300, 1000, 2], pad_rows=2), {}, False),
    ("mixed", dict(batch=5, new_lengths=[1, 3, 40, 1, 130], ctx_lengths=[0, 19, 300, 1000, 2], pad_rows=2),
     dict(dtype="f32"), False),
]


@pytest.mark.parametrize("name,kw,over,fixed", PAD_FLAG,
                         ids=["decode", "decode-fixed", "mla", "generic", "extend-own", "generic-own-f32"])
def test_pad_lse_only_flag(name, kw, over, fixed):
    """CPATTN_FLAG_PAD_LSE_ONLY: padding tokens get lse = -inf and their out rows are left untouched, in every kernel's
    padding role (partial and own-token calls); real tokens' results are the same bits as without the flag."""
    from cp_slot_map_amd import _lib
    wl = dataclasses.replace(workloads.make(name, **kw), **over)
    say(f"pad lse only {name} {over} fixed={fixed}")
    batch = pool.build_batch(wl, DEV)
    t = wl.num_tokens
    T, Hq = wl.bucket, wl.num_q_heads
    common = dict(page_size=wl.page_size, partners=wl.partners, scale=wl.scale, kind=wl.kind,
                  max_ctx_len=batch.max_ctx_len, max_row_tokens=batch.max_row_tokens, fixed_splits=fixed,
                  interleave=wl.interleave)
    ref_o, ref_l = api.paged_attn_partial(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len,
                                          batch.block_table, **common)
    o = torch.full_like(ref_o, 7.0)
    l = torch.full_like(ref_l, 7.0)
    a = api._paged_args(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len, batch.block_table,
                        page_size=wl.page_size, partners=wl.partners, scale=wl.scale, kind=wl.kind, stripe_begin=0,
                        stripe_count=wl.partners, max_ctx_len=batch.max_ctx_len, max_row_tokens=batch.max_row_tokens,
                        out=o, lse=l, num_tokens=T, fixed_splits=fixed, interleave=wl.interleave, pad_lse_only=True)
    import ctypes as C
    lib = _lib.load()
    n = C.c_int64(0)
    _lib.check(lib.cp_paged_attn_workspace_size(C.byref(a), C.byref(n)))
    ws = torch.zeros(max(1, n.value), dtype=torch.uint8, device=DEV)
    a.workspace, a.workspace_bytes = ws.data_ptr(), ws.numel()
    _lib.check(lib.cp_paged_attn_partial(C.byref(a), C.c_void_p(torch.cuda.current_stream().cuda_stream)))
    torch.cuda.synchronize()
    assert torch.equal(o[:, :t], ref_o[:, :t]) and torch.equal(l[:, :t], ref_l[:, :t])
    assert torch.all(torch.isneginf(l[:, t:])) and torch.all(o[:, t:] == 7.0)
    if wl.own_token:
        ro, rl = api.own_token_attn(batch.q, batch.k_new, batch.v_new, batch.cu_seqlens, scale=wl.scale,
                                    num_rows=wl.batch, max_row_tokens=batch.max_row_tokens)
        oo = torch.full_like(ro, 7.0)
        ol = torch.full_like(rl, 7.0)
        b = api.OwnArgs()
        b.dtype = api._dtype_code(batch.q.dtype)
        b.num_rows, b.bucket_tokens, b.num_q_heads = wl.batch, T, Hq
        b.num_kv_heads, b.head_dim = batch.k_new.shape[1], batch.k_new.shape[2]
        b.scale, b.max_row_tokens, b.flags = float(wl.scale), batch.max_row_tokens, _lib.CPATTN_FLAG_PAD_LSE_ONLY
        b.cu_seqlens, b.q = batch.cu_seqlens.data_ptr(), batch.q.data_ptr()
        b.q_stride_token, b.q_stride_head = batch.q.stride(0), batch.q.stride(1)
        b.k, b.v = batch.k_new.data_ptr(), batch.v_new.data_ptr()
        b.kv_stride_token, b.kv_stride_head = batch.k_new.stride(0), batch.k_new.stride(1)
        b.out, b.out_stride_token, b.out_stride_head = oo.data_ptr(), oo.stride(0), oo.stride(1)
        b.lse, b.lse_stride_token = ol.data_ptr(), ol.stride(0)
        _lib.check(lib.cp_own_token_attn(C.byref(b), C.c_void_p(torch.cuda.current_stream().cuda_stream)))
        torch.cuda.synchronize()
        assert torch.equal(oo[:t], ro[:t]) and torch.equal(ol[:t], rl[:t])
        assert torch.all(torch.isneginf(ol[t:])) and torch.all(oo[t:] == 7.0)
