"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that the pins catch every one."""
import numpy as np

import oracle
from oracle import attn as A
from oracle import slots as S
from tests import oracle_pins as pins


def _attention_no_scale(q, k, v, scale, visible=None):
    return A.attention(q, k, v, 1.0, visible)


def _attention_lse_without_max(q, k, v, scale, visible=None):
    o, l = A.attention(q, k, v, scale, visible)
    q64, k64 = np.asarray(q, float), np.asarray(k, float)
    if k64.shape[0] == 0:
        return o, l
    s = scale * (q64 @ k64.T)
    return o, np.where(np.isfinite(l), l - s.max(axis=1), l)   # dropped the max term


def _attention_values_are_keys(q, k, v, scale, visible=None):
    return A.attention(q, k, np.asarray(k)[:, : np.asarray(v).shape[1]] if np.asarray(k).ndim == 2 and
                       np.asarray(k).shape[1] >= np.asarray(v).shape[1] else v, scale, visible)


def _attention_ignores_mask(q, k, v, scale, visible=None):
    return A.attention(q, k, v, scale, None)


def _attention_transposed_scores(q, k, v, scale, visible=None):
    o, l = A.attention(q, k, v, scale, visible)
    return o, l * 1.0000001 if np.all(np.isfinite(l)) else l


def _merge_unnormalised(outs, lses):
    o, l = A.merge(outs, lses)
    w = [np.exp(np.asarray(x)) for x in lses]
    out = sum(wi[..., None] * np.asarray(oi) for wi, oi in zip(w, outs))
    return out, l


def _merge_wrong_sign(outs, lses):
    L = np.stack([np.asarray(x, float) for x in lses])
    mx = np.where(np.isfinite(L.max(0)), L.max(0), 0.0)
    w = np.exp(mx - L)
    w = np.where(np.isfinite(w), w, 0.0)
    tot = w.sum(0)
    out = sum((w[i] / np.where(tot > 0, tot, 1))[..., None] * np.asarray(o) for i, o in enumerate(outs))
    return out, mx + np.log(np.where(tot > 0, tot, 1))


def _merge_plain_average(outs, lses):
    o = sum(np.asarray(x) for x in outs) / len(outs)
    return o, A.merge(outs, lses)[1]


def _gqa_modulo_grouping(q, k, v, scale, visible=None):
    q, k, v = A._f64(q), A._f64(k), A._f64(v)
    hq, hkv = q.shape[1], k.shape[1]
    out = np.zeros((q.shape[0], hq, v.shape[2]))
    lse = np.zeros((q.shape[0], hq))
    for h in range(hq):
        out[:, h], lse[:, h] = A.attention(q[:, h], k[:, h % hkv], v[:, h % hkv], scale, visible)
    return out, lse


def _own_token_not_causal(q, k, v, scale):
    return A.gqa_attention(q, k, v, scale)


def _own_token_strict(q, k, v, scale):
    n = A._f64(q).shape[0]
    return A.gqa_attention(q, k, v, scale, visible=np.tril(np.ones((n, n), dtype=bool), k=-1))


def _stripe_off_by_one(q, k_ctx, v_ctx, P, r, scale):
    return A.stripe_partial(q, k_ctx, v_ctx, P, (r + 1) % P, scale)


def _slot_map_swapped(s, ps, P):
    a, b = S.slot_map(s, ps, P)
    return b, a


def _slot_map_page_local(s, ps, P):
    s = np.asarray(s, dtype=np.int64)
    off = s % ps
    return np.where(s >= 0, off % P, -1), np.where(s >= 0, (s // ps) * (ps // P) + off // P + (off % P > 0), -1)


def _slot_map_logical_page_size(s, ps, P):
    s = np.asarray(s, dtype=np.int64)
    return np.where(s >= 0, s % P, -1), np.where(s >= 0, (s // ps) * ps + s % ps // P, -1)


def _stripes_from_one(L, P, r):
    return np.array([t for t in range(1, L + 1) if t % P == r], dtype=np.int64)


def test_scale_dropped_is_caught():
    assert pins.check_brute_force(_attention_no_scale) and pins.check_torch_sdpa(_attention_no_scale)


def test_lse_missing_max_is_caught():
    assert pins.check_brute_force(_attention_lse_without_max)
    assert pins.check_closed_forms(_attention_lse_without_max)


def test_values_swapped_for_keys_is_caught():
    assert pins.check_brute_force(_attention_values_are_keys) or pins.check_closed_forms(_attention_values_are_keys)


def test_mask_ignored_is_caught():
    assert pins.check_brute_force(_attention_ignores_mask)


def test_lse_perturbed_is_caught():
    assert pins.check_brute_force(_attention_transposed_scores)


def test_unnormalised_merge_is_caught():
    assert pins.check_partition_invariance(A.attention, _merge_unnormalised)
    assert pins.check_merge_golden(_merge_unnormalised)


def test_merge_sign_flip_is_caught():
    assert pins.check_partition_invariance(A.attention, _merge_wrong_sign)


def test_merge_plain_average_is_caught():
    assert pins.check_merge_golden(_merge_plain_average)


def test_modulo_head_grouping_is_caught():
    assert pins.check_gqa_grouping(_gqa_modulo_grouping)


def test_non_causal_own_token_is_caught():
    assert pins.check_own_token_causal(_own_token_not_causal)
    assert pins.check_own_token_causal(_own_token_strict)


def test_stripe_selection_off_by_one_is_caught():
    assert pins.check_stripe_partial(_stripe_off_by_one, oracle.gather_stripe, oracle.place_logical_rows,
                                     oracle.gqa_attention)


def test_slot_map_mistakes_are_caught():
    assert pins.check_slot_map(_slot_map_swapped)
    assert pins.check_slot_map(_slot_map_page_local)
    assert pins.check_slot_map(_slot_map_logical_page_size)


def test_stripe_membership_mistake_is_caught():
    assert pins.check_stripes(_stripes_from_one)


def _slot_map_interleave_dense_phys(s, ps, P, I=1):
    a, _ = S.slot_map(s, ps, P, I)                  # right partner, physical slot as if I were 1
    s = np.asarray(s, dtype=np.int64)
    return a, np.where(s >= 0, s // P, -1)


def _slot_map_interleave_ignored(s, ps, P, I=1):
    return S.slot_map(s, ps, P)


def _slot_map_interleave_runs_per_partner(s, ps, P, I=1):
    s = np.asarray(s, dtype=np.int64)              # runs of P slots to I "partners": the two sizes swapped
    return np.where(s >= 0, (s // P) % I if I > 1 else s % P, -1), np.where(s >= 0, (s // (I * P)) * I + s % I, -1)


def _stripes_interleave_ignored(L, P, r, I=1):
    return S.stripe_positions(L, P, r)


def _stripe_len_interleave_ignored(L, P, r, I=1):
    return S.stripe_len(L, P, r)


def _stripe_partial_interleave_ignored(q, k_ctx, v_ctx, P, r, scale, I=1):
    return A.stripe_partial(q, k_ctx, v_ctx, P, r, scale)


def test_interleave_mistakes_are_caught():
    assert pins.check_interleave_slot_map(_slot_map_interleave_dense_phys)
    assert pins.check_interleave_slot_map(_slot_map_interleave_ignored)
    assert pins.check_interleave_slot_map(_slot_map_interleave_runs_per_partner)
    assert pins.check_interleave_stripes(_stripes_interleave_ignored, S.stripe_len)
    assert pins.check_interleave_stripes(S.stripe_positions, _stripe_len_interleave_ignored)
    assert pins.check_interleave_stripe_partial(_stripe_partial_interleave_ignored, oracle.gather_stripe,
                                                oracle.place_logical_rows, oracle.gqa_attention)


def _e4m3_bias_8(code):
    v = oracle.e4m3_value(code)
    return v / 2.0 if np.isfinite(v) else v


def _e4m3_no_subnormals(code):
    return 0.0 if (code & 0x78) == 0 else oracle.e4m3_value(code)


def _e4m3_fnuz_nan(code):
    return float("nan") if code == 0x80 else oracle.e4m3_value(code) if code not in (0x7f, 0xff) else 480.0


def _dequant_inverse(codes, descale):
    from oracle import quant
    return quant.dequantize_e4m3(codes, 1.0) / descale


def test_fp8_mistakes_are_caught():
    from oracle import quant
    assert pins.check_e4m3(_e4m3_bias_8, quant.dequantize_e4m3)
    assert pins.check_e4m3(_e4m3_no_subnormals, quant.dequantize_e4m3)
    assert pins.check_e4m3(_e4m3_fnuz_nan, quant.dequantize_e4m3)
    assert pins.check_e4m3(oracle.e4m3_value, _dequant_inverse)
