"""Parity of the HIP path (through the C ABI) with the float64 oracle, on the GPU."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from cp_slot_map_amd import api, pool
from tests.gpu_helpers import check_lse, check_out, check_padding, compare_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


# ------------------------------------------------------------------------------------------- integer paths
@pytest.mark.parametrize("page_size,P", [(16, 1), (16, 2), (16, 4), (16, 8), (16, 16), (64, 4), (48, 4), (6, 3)])
def test_slot_map_bit_exact(page_size, P):
    say(f"slot_map page_size={page_size} P={P}")
    rng = np.random.default_rng(page_size * 31 + P)
    s = np.concatenate([rng.integers(-5, 1 << 40, size=5000), np.arange(-3, 300), [0, (1 << 62) + 7]])
    partner, phys = api.slot_map(torch.from_numpy(s).to(DEV), page_size, P)
    rp, rq = oracle.slot_map(s, page_size, P)
    assert np.array_equal(partner.cpu().numpy().astype(np.int64), rp)
    assert np.array_equal(phys.cpu().numpy(), rq)
    for rank in range(P):
        w = api.slot_map_rank(torch.from_numpy(s).to(DEV), page_size, P, rank, 3)
        assert np.array_equal(w.cpu().numpy(), oracle.slot_map_rank(s, page_size, P, rank, 3))


@pytest.mark.parametrize("page_size,P,I", [(16, 4, 2), (16, 4, 4), (16, 2, 8), (64, 4, 16), (12, 3, 2), (16, 1, 16)])
def test_interleaved_slot_map_bit_exact(page_size, P, I):
    say(f"slot_map page_size={page_size} P={P} interleave={I}")
    rng = np.random.default_rng(page_size * 37 + P * 5 + I)
    s = np.concatenate([rng.integers(-5, 1 << 40, size=5000), np.arange(-3, 300), [0, (1 << 62) + 7]])
    partner, phys = api.slot_map(torch.from_numpy(s).to(DEV), page_size, P, interleave=I)
    rp, rq = oracle.slot_map(s, page_size, P, I)
    assert np.array_equal(partner.cpu().numpy().astype(np.int64), rp)
    assert np.array_equal(phys.cpu().numpy(), rq)
    for rank in range(P):
        w = api.slot_map_rank(torch.from_numpy(s).to(DEV), page_size, P, rank, 3, interleave=I)
        assert np.array_equal(w.cpu().numpy(), oracle.slot_map_rank(s, page_size, P, rank, 3, I))


@pytest.mark.parametrize("name,kw", [
    ("tiny", dict(interleave=4)),
    ("llama8b", dict(batch=3, ctx_lengths=[1, 37, 301], interleave=2)),
    ("llama8b", dict(batch=3, ctx_lengths=[5, 64, 333], interleave=4)),
    ("mla", dict(batch=2, ctx_lengths=[5, 200], interleave=8)),
], ids=["tiny-i4", "llama8b-i2", "llama8b-i4", "mla-i8"])
def test_interleaved_write_path_and_page_addressing_bit_exact(name, kw):
    """With interleave I, kv_write places every token by the interleaved rule and the kernels' addressing reads
    stripe r back as the positions t with floor(t / I) mod P == r, in order."""
    wl = workloads.make(name, **kw)
    I = wl.interleave
    say(f"interleaved write path {name} I={I}")
    batch = pool.build_batch(wl, DEV)
    P, ps = wl.partners, wl.page_size
    for b in range(wl.batch):
        rv = workloads.row_values(wl, b, DEV)
        c = int(wl.ctx_len[b])
        for r in range(P):
            got = api.debug_gather_stripe(batch.k_pool, batch.block_table[b], c, ps, P, r, kind=wl.kind,
                                          interleave=I)
            idx = torch.from_numpy(oracle.stripe_positions(c, P, r, I)).to(DEV)
            want = rv.k_ctx[idx]
            assert got.shape == want.shape
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32))
    rows = [workloads.row_values(wl, b, DEV).k_ctx.cpu().double().numpy().reshape(int(wl.ctx_len[b]), -1)
            for b in range(wl.batch)]
    ref = oracle.place_logical_rows(rows, wl.block_table, wl.ctx_len, ps, P, wl.num_pages, interleave=I)
    pp = ps // P
    kp = batch.k_pool.double().cpu().numpy()
    for r in range(P):
        got = kp[r].reshape(wl.num_pages * pp, -1)
        assert np.array_equal(np.isnan(got), np.isnan(ref[r]))
        fin = ~np.isnan(ref[r])
        assert np.array_equal(got[fin], ref[r][fin])


INTERLEAVED = [
    ("tiny", dict(interleave=8)),
    ("llama8b", dict(batch=5, ctx_lengths=[1, 9, 255, 1031, 4100], interleave=2)),
    ("llama8b", dict(batch=4, ctx_lengths=[3, 17, 517, 2049], interleave=4)),
    ("longctx", dict(batch=3, ctx_lengths=[5, 100, 3001], interleave=2)),
    ("mla", dict(batch=3, ctx_lengths=[7, 130, 2000], interleave=16)),
    ("mixed", dict(batch=6, new_lengths=[1, 1, 5, 33, 1, 70], ctx_lengths=[0, 19, 0, 300, 1000, 2100], pad_rows=2,
                   interleave=4)),
]


@pytest.mark.parametrize("fixed_splits", [False, True], ids=["balanced", "fixed"])
@pytest.mark.parametrize("name,kw", INTERLEAVED, ids=[f"{n}-i{k['interleave']}" for n, k in INTERLEAVED])
def test_interleaved_step_parity(name, kw, fixed_splits):
    """Partials, own-token partial and merge of pools written with a KV-cache interleave size, against the oracle."""
    wl = workloads.make(name, **kw)
    say(f"interleaved step {name} I={wl.interleave} fixed_splits={fixed_splits} ctx={list(wl.ctx_len)}")
    batch = pool.build_batch(wl, DEV)
    res = pool.run_step(batch, fixed_splits=fixed_splits)
    torch.cuda.synchronize()
    w = compare_rows(wl, batch, res, range(wl.batch), DEV)
    check_padding(wl, res)
    say(f"  worst errors {w}")


def _bits(t):
    return t.view({torch.bfloat16: torch.int16, torch.float8_e4m3fn: torch.uint8, torch.float32: torch.int32}[t.dtype])


FP8 = [
    ("llama8b", dict(batch=5, ctx_lengths=[1, 9, 255, 1031, 4100], kv_dtype="fp8")),
    ("longctx", dict(batch=3, ctx_lengths=[5, 100, 3001], kv_dtype="fp8")),
    ("llama8b", dict(batch=3, ctx_lengths=[17, 300, 2222], kv_dtype="fp8", interleave=4)),
    ("mixed", dict(batch=6, new_lengths=[1, 1, 5, 33, 1, 70], ctx_lengths=[0, 19, 0, 300, 1000, 2100], pad_rows=2,
                   kv_dtype="fp8")),
    ("mixed", dict(batch=4, new_lengths=[17, 2, 130, 64], ctx_lengths=[5000, 33, 1, 2999], pad_rows=1,
                   kv_dtype="fp8", interleave=2)),
    ("mla", dict(batch=4, ctx_lengths=[1, 3, 70, 700], kv_dtype="fp8")),
    ("mla", dict(batch=2, ctx_lengths=[65, 1500], kv_dtype="fp8", num_q_heads=16, interleave=2)),
    ("mla", dict(batch=3, ctx_lengths=[7, 130, 2000], kv_dtype="fp8", num_q_heads=64)),
    ("mla", dict(batch=3, ctx_lengths=[2, 31, 900], kv_dtype="fp8", num_q_heads=32, interleave=4)),
]


@pytest.mark.parametrize("name", ["llama8b", "mla"])
def test_fp8_write_path_bit_exact(name):
    """fp8 pools: kv_write copies the E4M3 codes by the slot rule and the kernels' addressing reads them back."""
    wl = workloads.make(name, batch=3, ctx_lengths=[1, 37, 301], kv_dtype="fp8", interleave=2)
    batch = pool.build_batch(wl, DEV)
    assert batch.k_pool.dtype == torch.float8_e4m3fn
    P, ps = wl.partners, wl.page_size
    for b in range(wl.batch):
        rv = workloads.row_values(wl, b, DEV)
        c = int(wl.ctx_len[b])
        for r in range(P):
            got = api.debug_gather_stripe(batch.k_pool, batch.block_table[b], c, ps, P, r, kind=wl.kind, interleave=2)
            idx = torch.from_numpy(oracle.stripe_positions(c, P, r, 2)).to(DEV)
            assert torch.equal(_bits(got), _bits(rv.k_ctx[idx]))
            if wl.kind == "mla":        # values are the latent rows' first head_dim_v columns, in the same pool
                assert torch.equal(_bits(got[..., :wl.head_dim_v].contiguous()), _bits(rv.v_ctx[idx].contiguous()))
                continue
            got = api.debug_gather_stripe(batch.v_pool, batch.block_table[b], c, ps, P, r, interleave=2)
            assert torch.equal(_bits(got), _bits(rv.v_ctx[idx]))


@pytest.mark.parametrize("fixed_splits", [False, True], ids=["balanced", "fixed"])
@pytest.mark.parametrize("name,kw", FP8, ids=[f"{n}-fp8{'-i' + str(k['interleave']) if 'interleave' in k else ''}"
                                             for n, k in FP8])
def test_fp8_step_parity(name, kw, fixed_splits):
    """bf16 queries over fp8 pools (E4M3 codes, per-tensor descales): partials and merge against the oracle, which
    decodes the codes itself."""
    wl = workloads.make(name, **kw)
    say(f"fp8 step {name} fixed_splits={fixed_splits} ctx={list(wl.ctx_len)}")
    batch = pool.build_batch(wl, DEV)
    res = pool.run_step(batch, fixed_splits=fixed_splits)
    torch.cuda.synchronize()
    w = compare_rows(wl, batch, res, range(wl.batch), DEV)
    check_padding(wl, res)
    say(f"  worst errors {w}")


def test_slot_map_empty_and_errors():
    p, q = api.slot_map(torch.empty(0, dtype=torch.int64, device=DEV), 16, 4)
    assert p.numel() == 0 and q.numel() == 0
    with pytest.raises(RuntimeError):
        api.slot_map(torch.zeros(4, dtype=torch.int64, device=DEV), 16, 3)


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("llama8b", dict(batch=3, ctx_lengths=[1, 37, 301])),
    ("longctx", dict(batch=3, ctx_lengths=[3, 50, 129])),
    ("mla", dict(batch=2, ctx_lengths=[5, 200])),
])
@pytest.mark.parametrize("layout", ["hnd", "nhd"])
def test_write_path_and_page_addressing_bit_exact(name, kw, layout):
    """kv_write places every token by the slot rule; the kernels' addressing reads stripe r back as positions r::P."""
    wl = workloads.make(name, **kw)
    if wl.kind == "mla" and layout == "nhd":
        pytest.skip("MLA pools have one layout")
    say(f"write path {name} {layout}")
    batch = pool.build_batch(wl, DEV, layout=layout)
    P, ps = wl.partners, wl.page_size
    for b in range(wl.batch):
        rv = workloads.row_values(wl, b, DEV)
        c = int(wl.ctx_len[b])
        for r in range(P):
            got = api.debug_gather_stripe(batch.k_pool, batch.block_table[b], c, ps, P, r, kind=wl.kind)
            want = rv.k_ctx[r::P]
            assert got.shape == want.shape
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32))
    # the whole pool, NaN where the oracle's placement leaves a slot untouched
    rows = [workloads.row_values(wl, b, DEV).k_ctx.cpu().double().numpy().reshape(int(wl.ctx_len[b]), -1)
            for b in range(wl.batch)]
    ref = oracle.place_logical_rows(rows, wl.block_table, wl.ctx_len, ps, P, wl.num_pages)
    pp = ps // P
    kp = batch.k_pool.double().cpu().numpy()
    for r in range(P):
        got = kp[r].reshape(wl.num_pages * pp, -1)
        assert np.array_equal(np.isnan(got), np.isnan(ref[r]))
        fin = ~np.isnan(ref[r])
        assert np.array_equal(got[fin], ref[r][fin])


# ----------------------------------------------------------------------------------------------- merge
@pytest.mark.parametrize("N,Dv", [(5, 128), (9, 128), (17, 128), (3, 68), (7, 8), (4, 512)])
def test_merge_edge_cases(N, Dv):
    """Every width path of the merge (16, 8 or 4 dims a thread; arrays for 5, 9 or 17 partials)."""
    say(f"merge edge cases N={N} Dv={Dv}")
    g = torch.Generator(device=DEV).manual_seed(5 + N + Dv)
    T, H = 37, 6
    outs = [torch.randn(T, H, Dv, generator=g, device=DEV) for _ in range(N)]
    lses = [torch.randn(T, H, generator=g, device=DEV) * 3 for _ in range(N)]
    lses[1][:5] = -float("inf")
    outs[1][:5] = float("nan")                 # an empty partial's row is never read
    for i in range(N):
        lses[i][7] = -float("inf")             # token 7: every partial empty
    mo, ml = api.lse_merge(outs, lses)
    ro, rl = oracle.merge([o.cpu() for o in outs[:1]] + [torch.where(torch.isnan(outs[1]), 0, outs[1]).cpu()]
                          + [o.cpu() for o in outs[2:]], [l.cpu() for l in lses])
    check_out(mo, ro, "merge out")
    check_lse(ml, rl, "merge lse")
    assert torch.all(mo[7] == 0) and torch.all(torch.isneginf(ml[7]))
    # bf16 output is the round-to-nearest-even of the fp32 merge
    mb, _ = api.lse_merge(outs, lses, out_dtype=torch.bfloat16)
    assert torch.equal(mb, mo.to(torch.bfloat16))
    # padding tokens given by a device count are written as (0, -inf) without reading
    cnt = torch.tensor([20], dtype=torch.int32, device=DEV)
    po, pl = api.lse_merge(outs, lses, token_count=cnt)
    assert torch.equal(po[:20], mo[:20]) and torch.all(po[20:] == 0) and torch.all(torch.isneginf(pl[20:]))
    # one partial is the identity; an empty partial changes nothing
    io, il = api.lse_merge(outs[:1], lses[:1])
    live = torch.isfinite(lses[0])
    assert torch.equal(io[live], outs[0][live]) and torch.equal(il[live], lses[0][live])
    assert torch.all(io[~live] == 0) and torch.all(torch.isneginf(il[~live]))


# ------------------------------------------------------------------------------------ attention parity
SMALL = [
    ("tiny", {}),
    ("llama8b", dict(batch=7, ctx_lengths=[1, 3, 4, 17, 255, 1031, 4100])),
    ("longctx", dict(batch=4, ctx_lengths=[5, 100, 4097, 9001])),
    ("mla", dict(batch=3, ctx_lengths=[7, 130, 2000])),
    ("mixed", dict(batch=6, new_lengths=[1, 1, 5, 33, 1, 70], ctx_lengths=[0, 19, 0, 300, 1000, 2100], pad_rows=2)),
]


EXTEND_PAGES = [
    # the extend kernel addresses keys a 4-token group at a time when pages hold 4 or more slots, else lane by lane
    ("pp2", dict(batch=4, new_lengths=[1, 40, 7, 100], ctx_lengths=[500, 3000, 40, 9], partners=8, pad_rows=1)),
    ("pp1", dict(batch=3, new_lengths=[33, 5, 64], ctx_lengths=[1000, 77, 2], partners=8, page_size=8)),
    ("pp8-fp8", dict(batch=3, new_lengths=[70, 1, 20], ctx_lengths=[2000, 300, 31], partners=2, kv_dtype="fp8")),
    ("pp16-i2", dict(batch=3, new_lengths=[9, 130, 2], ctx_lengths=[700, 2500, 65], partners=2, page_size=32,
                     interleave=2)),
]


@pytest.mark.parametrize("case,kw", EXTEND_PAGES, ids=[c[0] for c in EXTEND_PAGES])
def test_extend_page_geometries(case, kw):
    """Multi-token rows over pools whose pages hold 1, 2, 8 or 16 slots (P = 8 or 2, pages of 8 to 32): the extend
    kernel's lane-by-lane and grouped key addressing, against the oracle."""
    wl = workloads.make("mixed", **kw)
    say(f"extend page geometry {case}: P={wl.partners} page={wl.page_size} ctx={list(wl.ctx_len)}")
    batch = pool.build_batch(wl, DEV)
    res = pool.run_step(batch)
    torch.cuda.synchronize()
    w = compare_rows(wl, batch, res, range(wl.batch), DEV)
    check_padding(wl, res)
    say(f"  worst errors {w}")


@pytest.mark.parametrize("fixed_splits", [False, True], ids=["balanced", "fixed"])
@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_step_parity_small(name, kw, fixed_splits):
    wl = workloads.make(name, **kw)
    say(f"step parity {name} fixed_splits={fixed_splits} B={wl.batch} ctx={list(wl.ctx_len)} new={list(wl.new_len)}")
    batch = pool.build_batch(wl, DEV)                      # NaN in every slot that holds no token
    res = pool.run_step(batch, fixed_splits=fixed_splits)
    torch.cuda.synchronize()
    w = compare_rows(wl, batch, res, range(wl.batch), DEV)
    check_padding(wl, res)
    say(f"  worst errors {w}")


@pytest.mark.parametrize("name,kw", SMALL, ids=[s[0] for s in SMALL])
def test_nan_poison_is_bit_identical_to_zero_fill(name, kw):
    """Slots, pages, queries and in-step K/V that hold no real token are never read: NaN there changes no bit."""
    wl = workloads.make(name, **kw)
    say(f"poison {name}")
    a = pool.run_step(pool.build_batch(wl, DEV, fill=float("nan")))
    b = pool.run_step(pool.build_batch(wl, DEV, fill=0.0))
    t = wl.num_tokens
    assert torch.equal(a[0][:t], b[0][:t]) and torch.equal(a[1][:t], b[1][:t])
    assert torch.equal(a[2][:, :t], b[2][:, :t]) and torch.equal(a[3][:, :t], b[3][:, :t])
    check_padding(wl, a)


@pytest.mark.parametrize("fixed_splits", [False, True], ids=["balanced", "fixed"])
def test_stripe_subset_matches_all_stripes(fixed_splits):
    """One rank's share (stripe_begin, stripe_count = 1) equals the same stripe of the all-stripes call: to the bit
    with fixed splits, within the parity tolerance with the balanced schedule (its split points follow the call's
    total work, so only the rounding may differ)."""
    wl = workloads.make("llama8b", batch=5, ctx_lengths=[9, 400, 1100, 3000, 64])
    say(f"stripe subset fixed_splits={fixed_splits}")
    batch = pool.build_batch(wl, DEV)
    _, _, po, pl, _ = pool.run_step(batch, fixed_splits=fixed_splits)
    for r in range(wl.partners):
        o, l = api.paged_attn_partial(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len,
                                      batch.block_table, page_size=wl.page_size, partners=wl.partners,
                                      scale=wl.scale, stripe_begin=r, stripe_count=1,
                                      max_ctx_len=batch.max_ctx_len, max_row_tokens=1, fixed_splits=fixed_splits)
        if fixed_splits:
            assert torch.equal(o[0], po[r]) and torch.equal(l[0], pl[r])
        else:
            t = wl.num_tokens
            check_out(o[0, :t], po[r, :t].double().cpu().numpy(), f"stripe {r} subset out")
            check_lse(l[0, :t], pl[r, :t].double().cpu().numpy(), f"stripe {r} subset lse")
    # the two schedules agree within the parity tolerance
    if not fixed_splits:
        _, _, fo, fl, _ = pool.run_step(batch, fixed_splits=True)
        t = wl.num_tokens
        check_out(po[:, :t], fo[:, :t].double().cpu().numpy(), "balanced vs fixed out")
        check_lse(pl[:, :t], fl[:, :t].double().cpu().numpy(), "balanced vs fixed lse")


@pytest.mark.parametrize("heads", [16, 32, 64])
def test_mla_query_head_counts(heads):
    """The MLA kernel runs Hq / 16 waves per workgroup and splits the value dims over them (512, 256, 128 dims a wave
    for 16, 32, 64 heads); contexts of one token, a ragged tail and several chunks per stripe."""
    wl = workloads.make("mla", batch=3, ctx_lengths=[7, 130, 2000], num_q_heads=heads)
    say(f"mla heads={heads} ctx={list(wl.ctx_len)}")
    batch = pool.build_batch(wl, DEV)
    res = pool.run_step(batch)
    torch.cuda.synchronize()
    w = compare_rows(wl, batch, res, range(wl.batch), DEV)
    check_padding(wl, res)
    say(f"  worst errors {w}")


@pytest.mark.parametrize("target", ["lane0", "lane10"])
@pytest.mark.parametrize("heads", [16, 32, 64, 128])
def test_mla_late_score_jump(heads, target):
    """A late latent row aligned with one query head scores far above everything in the stripe's first tile. The MLA
    kernel takes its softmax reference from a unit's first tile, so this case makes it repeat the unit with the exact
    maximum; the partials must still match the oracle. The aligned head is the first of a wave's 16 or one held by
    another lane (the workgroup's vote must see every lane)."""
    wl = workloads.make("mla", batch=2, ctx_lengths=[300, 1000], num_q_heads=heads)
    h = 0 if target == "lane0" else heads - 6
    say(f"mla late score jump heads={heads} head={h}")
    batch = pool.build_batch(wl, DEV)
    b, c = 1, 1000
    rv = workloads.row_values(wl, b, DEV)
    lat = rv.k_ctx.clone()
    lat[c - 3, 0] = (6.0 * torch.sign(rv.q[0, h].float())).to(lat.dtype)   # about +100 in log2 units for head h
    slots = pool.logical_slots(batch.block_table[b], c, wl.page_size)
    api.kv_write(slots, lat, None, batch.k_pool, None, wl.page_size, wl.partners, kind="mla")
    res = pool.run_step(batch)
    torch.cuda.synchronize()
    parts, _ = oracle.row_partials(rv.q.cpu(), lat.cpu(), lat[..., :wl.head_dim_v].cpu(), wl.partners, wl.scale)
    full = oracle.row_attention(rv.q.cpu(), lat.cpu(), lat[..., :wl.head_dim_v].cpu(), wl.scale)
    t0 = int(wl.q_row_start[b])
    for r in range(wl.partners):
        check_out(res[2][r, t0:t0 + 1], parts[r][0], f"stripe {r} out")
        check_lse(res[3][r, t0:t0 + 1], parts[r][1], f"stripe {r} lse")
    check_out(res[0][t0:t0 + 1], full[0], "merged out")
    check_lse(res[1][t0:t0 + 1], full[1], "merged lse")
    compare_rows(wl, batch, res, [0], DEV)                # the other row is untouched


@pytest.mark.parametrize("kv_dtype", ["same", "fp8"])
def test_extend_late_score_jump(kv_dtype):
    """A late key aligned with one query head scores far above every key of its tile-0 (over 200 log2 units in bf16,
    about 100 over fp8 pools, whose largest code is 448 times the key descale), once among a row's context keys and
    once among its in-step keys. The extend kernel takes its softmax reference from a unit's first tile, so p
    overflows here and the unit repeats with the exact maxima; partials, the own-token part and the merge must still
    match the oracle."""
    wl = workloads.make("mixed", batch=2, new_lengths=[40, 3], ctx_lengths=[3000, 500], kv_dtype=kv_dtype)
    say(f"extend late score jump {kv_dtype}")
    batch = pool.build_batch(wl, DEV)
    b, c, n, h = 0, 3000, 40, 5
    g = h // (wl.num_q_heads // wl.num_kv_heads)
    rv = workloads.row_values(wl, b, DEV)
    k_ctx = rv.k_ctx.clone()
    big = 448.0 if kv_dtype == "fp8" else 16.0       # fp8: the largest E4M3 code, stored as the code itself
    k_ctx[c - 3, g] = (big * torch.sign(rv.q[0, h].float())).to(k_ctx.dtype)     # context key 2997 (stripe 1)
    slots = pool.logical_slots(batch.block_table[b], c, wl.page_size)
    api.kv_write(slots, k_ctx, rv.v_ctx, batch.k_pool, batch.v_pool, wl.page_size, wl.partners)
    k_new = rv.k_new.clone()
    k_new[n - 2, g] = (16.0 * torch.sign(rv.q[n - 1, h].float())).to(k_new.dtype)  # in-step key 38, second tile
    t0 = int(wl.q_row_start[b])
    batch.k_new[t0:t0 + n] = k_new
    res = pool.run_step(batch)
    torch.cuda.synchronize()
    kc, vc = k_ctx.cpu(), rv.v_ctx.cpu()
    if kv_dtype == "fp8":               # what the codes stand for, by the oracle's own decoding
        kc = oracle.dequantize_e4m3(kc.view(torch.uint8), wl.k_descale)
        vc = oracle.dequantize_e4m3(vc.view(torch.uint8), wl.v_descale)
    parts, merged = oracle.row_partials(rv.q.cpu(), kc, vc, wl.partners, wl.scale, k_new.cpu(), rv.v_new.cpu())
    for r in range(wl.partners):
        check_out(res[2][r, t0:t0 + n], parts[r][0], f"stripe {r} out")
        check_lse(res[3][r, t0:t0 + n], parts[r][1], f"stripe {r} lse")
    check_out(res[4][0][t0:t0 + n], parts[-1][0], "own out")
    check_lse(res[4][1][t0:t0 + n], parts[-1][1], "own lse")
    check_out(res[0][t0:t0 + n], merged[0], "merged out")
    check_lse(res[1][t0:t0 + n], merged[1], "merged lse")
    compare_rows(wl, batch, res, [1], DEV)                # the other row is untouched


@pytest.mark.parametrize("fixed_splits", [False, True], ids=["balanced", "fixed"])
def test_repeat_calls_are_deterministic(fixed_splits):
    """Split items merged from their records give the same bits on every call, with the workspace reused."""
    wl = workloads.make("llama8b", batch=4, ctx_lengths=[8192, 5000, 2000, 7777])
    say(f"repeat determinism fixed_splits={fixed_splits}")
    batch = pool.build_batch(wl, DEV)
    first = pool.run_step(batch, fixed_splits=fixed_splits)
    for _ in range(3):
        again = pool.run_step(batch, fixed_splits=fixed_splits)
        assert torch.equal(first[0], again[0]) and torch.equal(first[1], again[1])


WORKSPACE_CASES = [
    ("llama8b", dict(batch=6, ctx_lengths=[8192, 5000, 2000, 7777, 31, 12000])),
    ("mixed", dict(batch=5, new_lengths=[1, 200, 37, 3, 90], ctx_lengths=[5000, 2100, 0, 777, 64], pad_rows=1)),
]


@pytest.mark.parametrize("kv_dtype", ["same", "fp8"])
@pytest.mark.parametrize("name,kw", WORKSPACE_CASES, ids=[c[0] for c in WORKSPACE_CASES])
def test_workspace_needs_no_initial_contents(name, kw, kv_dtype):
    """The calls give the same bits whatever the workspace held before: zeros, all-ones bytes, random bytes, a NaN
    fill, or what the previous call left. It holds the decode kernel's row offsets and split-item records and the
    extend kernel's plan (the units' order); every entry is written before it is read."""
    wl = workloads.make(name, kv_dtype=kv_dtype, **kw)
    say(f"workspace contents {name} {kv_dtype}")
    batch = pool.build_batch(wl, DEV)
    args = (batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len, batch.block_table)
    kw = dict(page_size=wl.page_size, partners=wl.partners, scale=wl.scale, kind=wl.kind,
              max_ctx_len=batch.max_ctx_len, max_row_tokens=batch.max_row_tokens, interleave=wl.interleave,
              k_descale=wl.k_descale, v_descale=wl.v_descale)
    n = api.paged_attn_workspace_size(*args, **kw)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ref_o, ref_l = api.paged_attn_partial(*args, workspace=ws, **kw)
    g = torch.Generator(device=DEV).manual_seed(5)
    fills = {"ones": lambda: ws.fill_(255), "random": lambda: ws.copy_(torch.randint(0, 256, (n,), generator=g,
             device=DEV, dtype=torch.uint8)), "nan": lambda: ws[: n // 4 * 4].view(torch.float32).fill_(float("nan")),
             "leftover": lambda: None, "zeros": lambda: ws.zero_()}
    for what, fill in fills.items():
        fill()
        o, l = api.paged_attn_partial(*args, workspace=ws, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(l, ref_l), what
    mo = torch.empty(batch.q.shape[0], wl.num_q_heads, wl.head_dim_v, dtype=torch.float32, device=DEV)
    ml = torch.empty(batch.q.shape[0], wl.num_q_heads, dtype=torch.float32, device=DEV)
    api.paged_attn_merged(*args, merged=mo, merged_lse=ml, workspace=ws, **kw)
    ref_mo, ref_ml = mo.clone(), ml.clone()
    for what, fill in fills.items():
        fill()
        api.paged_attn_merged(*args, merged=mo, merged_lse=ml, workspace=ws, **kw)
        torch.cuda.synchronize()
        assert torch.equal(mo, ref_mo) and torch.equal(ml, ref_ml), f"merged {what}"


def test_extend_plan_and_grid_order_give_the_same_bits():
    """The context part runs its units longest stripe first when the launch has at most 8192 (row, stripe, query
    block) triples (a plan kernel ranks them), in grid order beyond that. 70 rows with one of 1000 tokens make 8960
    triples over four stripes (grid order) and 2240 for one stripe (planned): each stripe's share equals the same
    stripe of the all-stripes call to the bit, and sampled rows match the oracle."""
    rng = np.random.default_rng(11)
    new = [int(x) for x in rng.integers(1, 4, size=70)]
    new[17] = 1000
    ctx = [int(x) for x in rng.integers(0, 200, size=70)]
    wl = workloads.make("mixed", batch=70, new_lengths=new, ctx_lengths=ctx)
    say(f"extend plan vs grid order: {sum(new)} tokens")
    batch = pool.build_batch(wl, DEV)
    res = pool.run_step(batch)
    _, _, po, pl, _ = res
    t = int(sum(new))
    for r in range(wl.partners):
        o, l = api.paged_attn_partial(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len,
                                      batch.block_table, page_size=wl.page_size, partners=wl.partners,
                                      scale=wl.scale, stripe_begin=r, stripe_count=1, max_ctx_len=batch.max_ctx_len,
                                      max_row_tokens=batch.max_row_tokens)
        torch.cuda.synchronize()
        assert torch.equal(o[0, :t], po[r, :t]) and torch.equal(l[0, :t], pl[r, :t]), f"stripe {r}"
    w = compare_rows(wl, batch, res, [0, 17, 40, 69], DEV, check_partials=True)
    say(f"  worst errors {w}")


def test_mla_plan_and_grid_order_give_the_same_bits():
    """The MLA kernel runs its units longest first when a launch has at most 1024 of them (a plan kernel ranks them),
    in grid order beyond that. 260 rows over four stripes make 1040 units (grid order), one stripe 260 (planned): each
    stripe's share equals the same stripe of the all-stripes call to the bit, and sampled rows match the oracle."""
    rng = np.random.default_rng(12)
    ctx = [int(x) for x in rng.integers(0, 96, size=260)]
    ctx[100] = 760                              # stripes of at most 190 tokens: one chunk in both calls
    wl = workloads.make("mla", batch=260, ctx_lengths=ctx)
    say(f"mla plan vs grid order: {sum(ctx)} context tokens")
    batch = pool.build_batch(wl, DEV)
    res = pool.run_step(batch)
    _, _, po, pl, _ = res
    t = wl.num_tokens
    for r in range(wl.partners):
        o, l = api.paged_attn_partial(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len,
                                      batch.block_table, page_size=wl.page_size, partners=wl.partners,
                                      scale=wl.scale, kind="mla", stripe_begin=r, stripe_count=1,
                                      max_ctx_len=batch.max_ctx_len, max_row_tokens=batch.max_row_tokens)
        torch.cuda.synchronize()
        assert torch.equal(o[0, :t], po[r, :t]) and torch.equal(l[0, :t], pl[r, :t]), f"stripe {r}"
    w = compare_rows(wl, batch, res, [0, 100, 259], DEV, check_partials=True)
    say(f"  worst errors {w}")


@pytest.mark.parametrize("ctx_lengths", [[32768, 30001, 20000], [32769, 64, 5000]], ids=["at_limit", "past_limit"])
def test_extend_rows_at_page_staging_limit(ctx_lengths):
    """Multi-token rows whose stripes hold 2048 pages (the most the bf16 extend kernel stages in LDS), and a batch one
    token past that (served by the generic kernel)."""
    wl = workloads.make("mixed", batch=3, new_lengths=[3, 40, 150], ctx_lengths=ctx_lengths, pad_rows=1)
    say(f"extend at page limit: ctx={list(wl.ctx_len)} new={list(wl.new_len)}")
    batch = pool.build_batch(wl, DEV)
    res = pool.run_step(batch)
    torch.cuda.synchronize()
    w = compare_rows(wl, batch, res, range(wl.batch), DEV, check_partials=True)
    check_padding(wl, res)
    say(f"  worst errors {w}")


@pytest.mark.parametrize("name,kw", [SMALL[1], SMALL[4]], ids=["llama8b", "mixed"])
def test_step_plan_matches_run_step(name, kw):
    """The prepared step the benchmark times (argument structs built once, the merge told the real token count) gives
    the same bits as the plain calls, padding tokens included."""
    wl = workloads.make(name, **kw)
    batch = pool.build_batch(wl, DEV)
    mo, ml, po, pl, own = pool.run_step(batch)
    t = wl.num_tokens
    for pad_lse_only in (False, True):
        plan = pool.StepPlan(batch, pad_lse_only=pad_lse_only)
        for rep in range(3):    # repeated steps into poisoned buffers: every output is rewritten every time
            plan.out.fill_(7.0)
            plan.lse.fill_(7.0)
            plan.merged.fill_(7.0)
            if own is not None:
                plan.own_out.fill_(float("nan"))
                plan.own_lse.fill_(7.0)
            pm, pml = plan.run()
            torch.cuda.synchronize()
            assert torch.equal(pm, mo) and torch.equal(pml, ml)
            assert torch.equal(plan.lse, pl)
            if pad_lse_only:    # padding tokens' partial rows are not written (they keep the poison)
                assert torch.equal(plan.out[:, :t], po[:, :t]) and torch.all(plan.out[:, t:] == 7.0)
            else:
                assert torch.equal(plan.out, po)
            if own is not None:
                assert torch.equal(plan.own_lse, own[1])
                assert torch.equal(plan.own_out[:t], own[0][:t])
                if not pad_lse_only:
                    assert torch.equal(plan.own_out, own[0])


def test_empty_batch_and_empty_context():
    wl = workloads.make("llama8b", batch=3, ctx_lengths=[0, 0, 2])
    batch = pool.build_batch(wl, DEV)
    mo, ml, po, pl, _ = pool.run_step(batch)
    assert torch.all(mo[:2] == 0) and torch.all(torch.isneginf(ml[:2]))
    assert torch.all(torch.isneginf(pl[2:, 2]))          # stripes 2, 3 of a 2-token row are empty
    compare_rows(wl, batch, (mo, ml, po, pl, None), [2], DEV)


# ----------------------------------------------------------------------------------------------- full sizes
# Every row's merged output and LSE is compared with the oracle; the per-stripe (and own-token) partials on sampled
# rows (shortest, longest and random ones).
FULL = [("tiny", None), ("llama8b", 6), ("longctx", 6), ("mla", 6), ("mixed", 6)]


def _sample_rows(wl, nsample, seed):
    if nsample is None:
        return list(range(wl.batch))
    order = np.argsort(wl.ctx_len + wl.new_len)
    rng = np.random.default_rng(seed)
    return sorted(set([int(order[0]), int(order[-1])] +
                      [int(x) for x in rng.choice(wl.batch, size=nsample - 2, replace=False)]))


@pytest.mark.parametrize("name,nsample", [("mixed", 6), ("llama8b", 4)])
def test_full_size_fp8(name, nsample):
    """Full-size workloads over fp8 pools (the extend kernel for mixed, the decode kernel for llama8b), as the
    benchmark times them with --kv-dtype fp8: every row's merged result and sampled rows' partials against the
    oracle."""
    wl = workloads.make(name, kv_dtype="fp8")
    say(f"full size fp8 {name}: B={wl.batch}")
    batch = pool.build_batch(wl, DEV, fill=0.0)
    plan = pool.StepPlan(batch, out_dtype=torch.bfloat16)
    plan.run()
    torch.cuda.synchronize()
    own = (plan.own_out, plan.own_lse) if plan.own is not None else None
    res = (plan.merged, plan.merged_lse, plan.out, plan.lse, own)
    part_rows = _sample_rows(wl, nsample, 13)
    w = compare_rows(wl, batch, res, range(wl.batch), DEV, check_partials=part_rows)
    check_padding(wl, res, partial_rows_written=False)
    say(f"  partial rows {part_rows} worst {w}")
    del plan, batch, res
    torch.cuda.empty_cache()


def test_full_size_interleaved_llama8b():
    """The llama8b workload written with interleave 4 (runs of 4 slots, one physical page per run at page 16, P 4):
    every row's merged result and sampled rows' partials against the oracle at full size."""
    wl = workloads.make("llama8b", interleave=4)
    batch = pool.build_batch(wl, DEV, fill=0.0)
    res = pool.run_step(batch)
    torch.cuda.synchronize()
    part_rows = _sample_rows(wl, 4, 3)
    w = compare_rows(wl, batch, res, range(wl.batch), DEV, check_partials=part_rows)
    say(f"  partial rows {part_rows} worst {w}")
    del batch, res
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,nsample", FULL, ids=[f[0] for f in FULL])
def test_full_size_all_rows(name, nsample):
    wl = workloads.make(name)
    say(f"full size {name}: B={wl.batch} ctx tokens={int(wl.ctx_len.sum())}")
    batch = pool.build_batch(wl, DEV, fill=0.0)
    res = pool.run_step(batch)
    torch.cuda.synchronize()
    part_rows = _sample_rows(wl, nsample, 7)
    w = compare_rows(wl, batch, res, range(wl.batch), DEV, check_partials=part_rows)
    check_padding(wl, res)
    say(f"  partial rows {part_rows} worst {w}")
    del batch, res
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,nsample", [("llama8b", 6), ("longctx", 4), ("mla", 4), ("mixed", 6)])
def test_full_size_bench_configuration(name, nsample):
    """The step exactly as the benchmark times it (zero-filled pools, prepared StepPlan, bf16 merged output, the merge
    told the real token count), repeated: every row's merged result and sampled rows' partials against the oracle."""
    wl = workloads.make(name)
    say(f"bench configuration {name}: B={wl.batch}")
    batch = pool.build_batch(wl, DEV, fill=0.0)
    plan = pool.StepPlan(batch, out_dtype=torch.bfloat16)
    for _ in range(3):
        plan.run()
    torch.cuda.synchronize()
    own = (plan.own_out, plan.own_lse) if plan.own is not None else None
    res = (plan.merged, plan.merged_lse, plan.out, plan.lse, own)
    part_rows = _sample_rows(wl, nsample, 11)
    w = compare_rows(wl, batch, res, range(wl.batch), DEV, check_partials=part_rows)
    check_padding(wl, res, partial_rows_written=False)
    say(f"  partial rows {part_rows} worst {w}")
    del plan, batch, res
    torch.cuda.empty_cache()


CLAMP_CASES = [
    ("decode_balanced", "llama8b", dict(batch=5, ctx_lengths=[9, 400, 1100, 3000, 64]), 1000, False),
    ("decode_fixed", "llama8b", dict(batch=5, ctx_lengths=[9, 400, 1100, 3000, 64]), 1000, True),
    ("extend", "mixed", dict(batch=3, new_lengths=[1, 40, 7], ctx_lengths=[500, 3000, 40]), 1000, False),
    ("mla", "mla", dict(batch=3, ctx_lengths=[7, 130, 2000], num_q_heads=16), 500, False),
    ("generic", "tiny", dict(ctx_lengths=[1, 17, 100, 200]), 60, False),
]


@pytest.mark.parametrize("case,name,kw,cap,fixed_splits", CLAMP_CASES, ids=[c[0] for c in CLAMP_CASES])
def test_understated_max_ctx_len_clamps_rows(case, name, kw, cap, fixed_splits):
    """max_ctx_len sizes the launch and the workspace; a row whose device ctx_len exceeds it is taken as its first
    max_ctx_len tokens, in every kernel (fixed-split decode, balanced decode, extend, MLA, generic)."""
    wl = workloads.make(name, **kw)
    say(f"clamp {case}: ctx={list(wl.ctx_len)} max_ctx_len={cap}")
    batch = pool.build_batch(wl, DEV)
    o, l = api.paged_attn_partial(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len,
                                  batch.block_table, page_size=wl.page_size, partners=wl.partners, scale=wl.scale,
                                  kind=wl.kind, max_ctx_len=cap, max_row_tokens=batch.max_row_tokens,
                                  fixed_splits=fixed_splits, interleave=wl.interleave)
    torch.cuda.synchronize()
    qrs = wl.q_row_start
    for b in range(wl.batch):
        n = int(wl.new_len[b])
        if n == 0:
            continue
        c = min(int(wl.ctx_len[b]), cap)
        rv = workloads.row_values(wl, b, DEV)
        q, k, v = rv.q.cpu(), rv.k_ctx.cpu()[:c], rv.v_ctx.cpu()[:c]
        t0 = int(qrs[b])
        for r in range(wl.partners):
            ro, rl = oracle.stripe_partial(q, k, v, wl.partners, r, wl.scale, wl.interleave)
            check_out(o[r, t0:t0 + n], ro, f"row {b} stripe {r} out")
            check_lse(l[r, t0:t0 + n], rl, f"row {b} stripe {r} lse")


@pytest.mark.parametrize("nbytes,words", [(16, 2048), (4096 * 8 * 3 + 16 * 37, 2048), (64 << 20, 2048), (1 << 20, 3)])
def test_stream_read_reads_every_byte(nbytes, words):
    """The streaming-read reference kernel reads the whole buffer: the XOR of its per-workgroup words is the XOR of
    every 32-bit word of the buffer (ragged sizes and a sink smaller than the grid would be)."""
    say(f"stream read {nbytes} bytes, {words} sink words")
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g)
    sink = torch.zeros(words, dtype=torch.int32, device=DEV)
    api.debug_stream_read(host.to(DEV), sink=sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want
