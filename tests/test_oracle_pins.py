"""CPU pins of the float64 oracle (no GPU, no HIP library)."""
import math

import numpy as np
import pytest

import oracle
import workloads
from tests import oracle_pins as pins


def test_slot_map_golden_roundtrip_bijection():
    assert pins.check_slot_map(oracle.slot_map) == []


def test_slot_map_refuses_bad_geometry():
    with pytest.raises(ValueError):
        oracle.slot_map([1], 16, 3)          # P does not divide page_size
    with pytest.raises(ValueError):
        oracle.slot_map([1], 16, 0)
    with pytest.raises(ValueError):
        oracle.slot_map([1], 0, 1)


def test_slot_map_rank_view_with_sink():
    s = np.array([0, 1, 2, 3, 37, -1, 1000])
    P, sink = 4, 0
    for r in range(P):
        w = oracle.slot_map_rank(s, 16, P, r, sink)
        for si, wi in zip(s.tolist(), w.tolist()):
            if si < 0:
                assert wi == -1
            elif si % P == r:
                assert wi == si // P
            else:
                assert wi == sink
    with pytest.raises(ValueError):
        oracle.slot_map_rank(s, 16, P, P, sink)


def test_stripes_golden_and_length_formula():
    assert pins.check_stripes(oracle.stripe_positions) == []
    for L in range(0, 40):
        for P in (1, 2, 3, 4, 8):
            for r in range(P):
                assert oracle.stripe_len(L, P, r) == max(0, -(-(L - r) // P))


def test_stripe_is_a_paged_cache_of_page_size_over_P():
    """Every context position t of a row lands on partner t mod P at page bt[t // page_size], slot (t mod page_size) // P."""
    rng = np.random.default_rng(11)
    for page_size, P in ((16, 4), (16, 8), (16, 2), (64, 4), (8, 1)):
        pp = page_size // P
        L = int(rng.integers(1, 300))
        n = (L + page_size - 1) // page_size
        bt = rng.permutation(np.arange(1, n + 5))[:n]
        t = np.arange(L)
        s = bt[t // page_size] * page_size + t % page_size
        partner, phys = oracle.slot_map(s, page_size, P)
        assert np.array_equal(partner, t % P)
        assert np.array_equal(phys, bt[t // page_size] * pp + (t % page_size) // P)
        # local index j = t // P addresses page bt[j // pp], slot j % pp
        j = t // P
        assert np.array_equal(phys, bt[j // pp] * pp + j % pp)


def test_place_and_gather_round_trip_leaves_other_slots_untouched():
    rng = np.random.default_rng(12)
    page_size, P, L = 16, 4, 77
    n = (L + page_size - 1) // page_size
    num_pages = n + 3
    bt = np.concatenate([rng.permutation(np.arange(1, num_pages))[:n], [0, 0]])
    k = rng.standard_normal((L, 2, 3))
    pools = oracle.place_logical_rows([k], [bt], [L], page_size, P, num_pages)
    written = 0
    for r in range(P):
        got = oracle.gather_stripe(pools[r], bt, L, page_size, P, r)
        assert np.array_equal(got, k[r::P])
        written += np.isfinite(pools[r][:, 0, 0]).sum()
    assert written == L                       # nothing else was written: sink and spare slots stay NaN
    for r in range(P):
        assert np.all(np.isnan(pools[r][: page_size // P]))     # the sink page 0


def test_unplaced_write_addressing_is_caught():
    """Negative control (review thread on resident planning): writing at the logical page size, bypassing the placement,
    puts tokens at the wrong physical slots, so the stripe read back is not the row's positions r, r + P, ..."""
    rng = np.random.default_rng(13)
    page_size, P, L = 16, 4, 64
    pp = page_size // P
    n = L // page_size
    num_pages = n + 2
    bt = rng.permutation(np.arange(1, num_pages))[:n]
    k = rng.standard_normal((L, 1, 2))
    pools = [np.full((num_pages * pp, 1, 2), np.nan) for _ in range(P)]
    for t in range(L):                        # every rank writes every token at page * page_size + offset
        idx = bt[t // page_size] * page_size + t % page_size
        for r in range(P):
            if idx < pools[r].shape[0]:
                pools[r][idx] = k[t]
    bad = 0
    for r in range(P):
        got = oracle.gather_stripe(pools[r], bt, L, page_size, P, r)
        if got.shape != k[r::P].shape or not np.array_equal(got, k[r::P]):
            bad += 1
    assert bad == P


def test_attention_brute_force():
    assert pins.check_brute_force(oracle.attention) == []


def test_attention_matches_torch_sdpa_float64():
    assert pins.check_torch_sdpa(oracle.attention) == []


def test_attention_closed_forms_and_worked_example():
    assert pins.check_closed_forms(oracle.attention) == []


def test_merge_worked_example_and_empty_partials():
    assert pins.check_merge_golden(oracle.merge) == []
    assert pins.check_empty_partials(oracle.merge) == []


def test_merge_of_any_split_equals_unsplit():
    assert pins.check_partition_invariance(oracle.attention, oracle.merge) == []


def test_gqa_head_grouping():
    assert pins.check_gqa_grouping(oracle.gqa_attention) == []


def test_own_token_is_causal():
    assert pins.check_own_token_causal(oracle.own_token_partial) == []


def test_stripe_partial_attends_its_pool():
    assert pins.check_stripe_partial(oracle.stripe_partial, oracle.gather_stripe, oracle.place_logical_rows,
                                     oracle.gqa_attention) == []


def test_one_stripe_is_plain_attention_bit_identical():
    wl = workloads.make("tiny")
    for b in range(wl.batch):
        rv = workloads.row_values(wl, b)
        parts, (o, l) = oracle.row_partials(rv.q, rv.k_ctx, rv.v_ctx, 1, wl.scale)
        ro, rl = oracle.row_attention(rv.q, rv.k_ctx, rv.v_ctx, wl.scale)
        assert np.array_equal(o, ro) and np.array_equal(l, rl)


def test_striped_rows_equal_unstriped_rows_tiny():
    wl = workloads.make("tiny")
    for b in range(wl.batch):
        rv = workloads.row_values(wl, b)
        parts, (o, l) = oracle.row_partials(rv.q, rv.k_ctx, rv.v_ctx, wl.partners, wl.scale)
        ro, rl = oracle.row_attention(rv.q, rv.k_ctx, rv.v_ctx, wl.scale)
        assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(l - rl)) < 1e-12
        if wl.ctx_len[b] == 1:                 # L = 1 with P = 2: stripe 1 is empty
            assert np.all(parts[1][0] == 0) and np.all(np.isneginf(parts[1][1]))


def test_no_context_reduces_to_own_token_partial():
    wl = workloads.make("mixed", batch=4, ctx_lengths=[0, 0, 5, 0], new_lengths=[3, 1, 4, 7])
    for b in range(wl.batch):
        rv = workloads.row_values(wl, b)
        _, (o, l) = oracle.row_partials(rv.q, rv.k_ctx, rv.v_ctx, wl.partners, wl.scale, rv.k_new, rv.v_new)
        ro, rl = oracle.row_attention(rv.q, rv.k_ctx, rv.v_ctx, wl.scale, rv.k_new, rv.v_new)
        assert np.max(np.abs(o - ro)) < 1e-12 and np.max(np.abs(l - rl)) < 1e-12
        if wl.ctx_len[b] == 0:
            so, sl = oracle.own_token_partial(rv.q, rv.k_new, rv.v_new, wl.scale)
            assert np.array_equal(o, so) and np.array_equal(l, sl)


def test_mla_row_is_one_latent_head():
    """MLA: the key is the whole 576-wide latent row and the value its first 512 columns; brute force on one head."""
    wl = workloads.make("mla", batch=2, ctx_lengths=[5, 9])
    for b in range(wl.batch):
        rv = workloads.row_values(wl, b)
        o, l = oracle.row_attention(rv.q, rv.k_ctx, rv.v_ctx, wl.scale)
        assert o.shape == (1, 128, 512)
        k = rv.k_ctx[:, 0].double().numpy()
        for h in (0, 77):
            bo, bl = pins.brute_attention(rv.q[:, h].double().numpy().tolist(), k.tolist(), k[:, :512].tolist(),
                                          wl.scale)
            assert np.max(np.abs(o[:, h] - bo)) < 1e-12 and abs(l[0, h] - bl[0]) < 1e-12


def test_workload_recipes():
    """The seeded generators reproduce the configs' shapes and length ranges."""
    t = workloads.make("tiny")
    assert list(t.ctx_len) == [1, 17, 100, 200] and t.partners == 2 and t.page_size == 16
    a = workloads.make("llama8b")
    assert a.batch == 64 and a.ctx_len.min() >= 1024 and a.ctx_len.max() <= 8192 and a.partners == 4
    b = workloads.make("longctx")
    assert b.batch == 256 and b.ctx_len.min() >= 4096 and b.ctx_len.max() <= 32768 and b.partners == 8
    c = workloads.make("mla")
    assert c.batch == 128 and c.head_dim == 576 and c.head_dim_v == 512 and c.page_size == 64
    d = workloads.make("mixed")
    assert d.batch == 32 and d.bucket == 8192 and d.num_tokens <= 8192 and list(d.new_len[:16]) == [1] * 16
    for wl in (t, a, b, c, d):
        bt = wl.block_table
        used = np.concatenate([bt[i, : -(-int(wl.ctx_len[i] + (wl.new_len[i] if wl.own_token else 0))
                                      // wl.page_size)] for i in range(wl.batch)])
        assert len(np.unique(used)) == len(used) and used.min() >= 1 and used.max() < wl.num_pages
    # same seed, same values
    r1 = workloads.row_values(t, 2)
    r2 = workloads.row_values(t, 2)
    assert np.array_equal(r1.k_ctx.numpy(), r2.k_ctx.numpy())


def test_interleaved_placement_is_pinned():
    assert pins.check_interleave_slot_map(oracle.slot_map) == []
    assert pins.check_interleave_stripes(oracle.stripe_positions, oracle.stripe_len) == []
    assert pins.check_interleave_stripe_partial(oracle.stripe_partial, oracle.gather_stripe, oracle.place_logical_rows,
                                                oracle.gqa_attention) == []


def test_fp8_codes_are_pinned():
    assert pins.check_e4m3(oracle.e4m3_value, oracle.dequantize_e4m3) == []
