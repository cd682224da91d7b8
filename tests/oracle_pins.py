"""Pins that tie the float64 oracle to something other than itself.

Each ``check_*`` takes the functions under test as arguments and returns a list of failure strings (empty = pinned),
so the same checks run against the real oracle (tests/test_oracle_pins.py) and against mistakes planted in copies of
it (tests/test_oracle_mutations.py), which must be caught.

What pins what:
* brute force: scalar Python loops with exactly rounded sums (math.fsum) on tiny inputs, no BLAS;
* a library routine: torch's float64 scaled_dot_product_attention and logsumexp on the CPU;
* closed forms and hand-worked values (tests/golden/*.txt, each citing its passage);
* invariants the pages state: merging the partials of any split of the keys gives the unsplit result; one stripe is
  plain attention; an empty partial changes nothing; with no context only the own-token partial remains; the slot
  rule is a bijection whose inverse is phys * P + partner;
* the interleaved placement against an independent dealing of each page's slots, run by run.
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


# ----------------------------------------------------------------------------------------------- brute force
def brute_attention(q, k, v, scale, visible=None, dv=None):
    """Scalar loops, exactly rounded sums: q [m][D], k [n][D], v [n][Dv] as nested lists."""
    m, n = len(q), len(k)
    if dv is None:
        dv = len(v[0]) if n else 0
    outs, lses = [], []
    for i in range(m):
        js = [j for j in range(n) if visible is None or visible[i][j]]
        if not js:
            outs.append([0.0] * dv)
            lses.append(-math.inf)
            continue
        s = [scale * math.fsum(q[i][d] * k[j][d] for d in range(len(q[i]))) for j in js]
        mx = max(s)
        w = [math.exp(x - mx) for x in s]
        tot = math.fsum(w)
        lses.append(mx + math.log(tot))
        outs.append([math.fsum(w[a] * v[js[a]][e] for a in range(len(js))) / tot for e in range(dv)])
    return np.array(outs, dtype=np.float64).reshape(m, dv), np.array(lses, dtype=np.float64)


def check_brute_force(attention, seed=0, trials=12):
    fails = []
    rng = np.random.default_rng(seed)
    for t in range(trials):
        m, n, d, dv = int(rng.integers(1, 4)), int(rng.integers(0, 40)), int(rng.integers(1, 9)), int(rng.integers(1, 7))
        q = rng.standard_normal((m, d)) * 1.5
        k = rng.standard_normal((n, d))
        v = rng.standard_normal((n, dv))
        scale = float(rng.uniform(0.2, 1.5))
        vis = None
        if t % 3 == 1:
            vis = rng.random((m, n)) < 0.6
        elif t % 3 == 2:
            vis = np.tril(np.ones((m, n), dtype=bool), k=n - m)
        o, l = attention(q, k, v, scale, vis)
        bo, bl = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, None if vis is None else vis.tolist(), dv)
        if not np.array_equal(np.isneginf(l), np.isneginf(bl)):
            fails.append(f"trial {t}: empty-set pattern differs")
            continue
        fin = np.isfinite(bl)
        if fin.any() and np.max(np.abs(l[fin] - bl[fin])) > 1e-12:
            fails.append(f"trial {t}: lse off by {np.max(np.abs(l[fin] - bl[fin])):.3e}")
        if o.shape != bo.shape or (o.size and np.max(np.abs(o - bo)) > 1e-12):
            fails.append(f"trial {t}: out differs")
    return fails


def check_torch_sdpa(attention, seed=1):
    """torch's float64 CPU scaled_dot_product_attention (and logsumexp for the lse) on single rows."""
    import torch
    fails = []
    rng = np.random.default_rng(seed)
    for t in range(6):
        m, n, d, dv = int(rng.integers(1, 5)), int(rng.integers(1, 70)), int(rng.integers(2, 65)), int(rng.integers(1, 65))
        q, k, v = rng.standard_normal((m, d)), rng.standard_normal((n, d)), rng.standard_normal((n, dv))
        scale = 1.0 / math.sqrt(d)
        causal = t % 2 == 1 and m <= n
        vis = np.tril(np.ones((m, n), dtype=bool), k=n - m) if causal else None
        tq, tk, tv = (torch.from_numpy(x)[None, None] for x in (q, k, v))
        mask = None if vis is None else torch.from_numpy(vis)[None, None]
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale)[0, 0].numpy()
        sc = (torch.from_numpy(q) @ torch.from_numpy(k).T) * scale
        if vis is not None:
            sc = sc.masked_fill(~torch.from_numpy(vis), float("-inf"))
        ref_lse = torch.logsumexp(sc, dim=1).numpy()
        o, l = attention(q, k, v, scale, vis)
        if np.max(np.abs(o - ref)) > 1e-12 or np.max(np.abs(l - ref_lse)) > 1e-12:
            fails.append(f"trial {t}: differs from torch sdpa by {np.max(np.abs(o - ref)):.3e}")
    return fails


# ------------------------------------------------------------------------------------ closed forms and golden
def check_closed_forms(attention, seed=2):
    fails = []
    rng = np.random.default_rng(seed)
    n, d, dv = 13, 8, 5
    k, v = rng.standard_normal((n, d)), rng.standard_normal((n, dv))
    # q = 0: every score is 0, so lse = ln n and out = mean of the values
    o, l = attention(np.zeros((1, d)), k, v, 0.7)
    if abs(l[0] - math.log(n)) > 1e-13 or np.max(np.abs(o[0] - v.mean(0))) > 1e-13:
        fails.append("q = 0 closed form")
    # one key: out = v0, lse = s0
    q = rng.standard_normal((1, d))
    o, l = attention(q, k[:1], v[:1], 0.3)
    if abs(l[0] - 0.3 * float(q[0] @ k[0])) > 1e-13 or np.max(np.abs(o[0] - v[0])) > 1e-13:
        fails.append("single key closed form")
    # identical keys: lse = s + ln n, out = mean v
    kk = np.repeat(k[:1], n, axis=0)
    o, l = attention(q, kk, v, 0.3)
    if abs(l[0] - (0.3 * float(q[0] @ k[0]) + math.log(n))) > 1e-12 or np.max(np.abs(o[0] - v.mean(0))) > 1e-12:
        fails.append("identical keys closed form")
    # one dominant key: out -> its value
    kd = k.copy()
    kd[4] = q[0] * 40.0
    o, l = attention(q, kd, v, 1.0)
    if np.max(np.abs(o[0] - v[4])) > 1e-12:
        fails.append("dominant key")
    # hand-worked example
    g = dict((r.split()[0], [float(x) for x in r.split()[1:]]) for r in read_golden("attention_worked.txt"))
    o, l = attention(np.array([[1.0, 0.0]]), np.array([[1.0, 0], [0, 1.0], [1.0, 1.0]]),
                     np.array([[1.0, 0], [0, 1.0], [2.0, 2.0]]), 1.0)
    if abs(l[0] - g["lse"][0]) > 1e-14 or np.max(np.abs(o[0] - np.array(g["out"]))) > 1e-14:
        fails.append("hand-worked attention example")
    # empty key set
    o, l = attention(rng.standard_normal((2, d)), np.zeros((0, d)), np.zeros((0, dv)), 1.0)
    if not (np.all(o == 0) and np.all(np.isneginf(l))):
        fails.append("empty key set is not (0, -inf)")
    return fails


def check_merge_golden(merge):
    g = dict((r.split()[0], [float(x) for x in r.split()[1:]]) for r in read_golden("attention_worked.txt"))
    o, l = merge([np.array([[1.0, 2.0]]), np.array([[4.0, 0.0]])], [np.array([math.log(3.0)]), np.array([0.0])])
    fails = []
    if abs(l[0] - g["merge_lse"][0]) > 1e-15 or np.max(np.abs(o[0] - np.array(g["merge_out"]))) > 1e-15:
        fails.append("hand-worked merge example")
    return fails


# ------------------------------------------------------------------------------------------------ invariants
def check_partition_invariance(attention, merge, seed=3):
    """Merging the partials of any split of the key set gives the unsplit result (the exactness the pages claim)."""
    fails = []
    rng = np.random.default_rng(seed)
    for t in range(16):
        m, n, d, dv = int(rng.integers(1, 4)), int(rng.integers(0, 60)), 6, 4
        q, k, v = rng.standard_normal((m, d)) * 2, rng.standard_normal((n, d)), rng.standard_normal((n, dv))
        full_o, full_l = attention(q, k, v, 0.9)
        parts = int(rng.integers(1, 9))
        if t % 2:
            label = np.arange(n) % parts                      # the striping itself
        else:
            label = rng.integers(0, parts, size=n)            # any split, some parts possibly empty
        order = rng.permutation(parts)
        po, pl = [], []
        for p in order:
            sel = label == p
            o, l = attention(q, k[sel], v[sel], 0.9)
            po.append(o)
            pl.append(l)
        mo, ml = merge(po, pl)
        if not np.array_equal(np.isneginf(ml), np.isneginf(full_l)):
            fails.append(f"trial {t}: empty pattern differs")
            continue
        fin = np.isfinite(full_l)
        if fin.any() and (np.max(np.abs(ml[fin] - full_l[fin])) > 1e-12 or np.max(np.abs(mo - full_o)) > 1e-12):
            fails.append(f"trial {t}: merged partials differ from the unsplit result")
    return fails


def check_empty_partials(merge, seed=4):
    fails = []
    rng = np.random.default_rng(seed)
    o, l = rng.standard_normal((3, 5)), rng.standard_normal(3)
    mo, ml = merge([o, np.zeros_like(o)], [l, np.full(3, -np.inf)])
    if not (np.array_equal(mo, o) and np.array_equal(ml, l)):
        fails.append("merging with an empty partial is not the identity")
    mo, ml = merge([np.zeros_like(o)] * 3, [np.full(3, -np.inf)] * 3)
    if not (np.all(mo == 0) and np.all(np.isneginf(ml))):
        fails.append("all-empty merge is not (0, -inf)")
    mo, ml = merge([o], [l])
    if not (np.array_equal(mo, o) and np.array_equal(ml, l)):
        fails.append("merge of one partial is not the identity")
    return fails


def check_gqa_grouping(gqa_attention):
    """Query head h reads kv head h // (Hq / Hkv): give each kv head a constant value equal to its index."""
    fails = []
    hq, hkv, d = 12, 3, 4
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, hq, d))
    k = rng.standard_normal((7, hkv, d))
    v = np.zeros((7, hkv, 3))
    for g in range(hkv):
        v[:, g, :] = g
    o, _ = gqa_attention(q, k, v, 0.5)
    for h in range(hq):
        if np.max(np.abs(o[:, h] - h // (hq // hkv))) > 1e-13:
            fails.append(f"head {h} did not read kv head {h // (hq // hkv)}")
    return fails


def check_own_token_causal(own_token_partial, seed=6):
    """Own-token attention is causal: in-step query i sees keys 0..i (pinned against brute force with that mask)."""
    fails = []
    rng = np.random.default_rng(seed)
    n, hq, hkv, d = 6, 4, 2, 5
    q, k, v = rng.standard_normal((n, hq, d)), rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d))
    o, l = own_token_partial(q, k, v, 0.8)
    for h in range(hq):
        g = h // (hq // hkv)
        vis = [[j <= i for j in range(n)] for i in range(n)]
        bo, bl = brute_attention(q[:, h].tolist(), k[:, g].tolist(), v[:, g].tolist(), 0.8, vis)
        if np.max(np.abs(o[:, h] - bo)) > 1e-12 or np.max(np.abs(l[:, h] - bl)) > 1e-12:
            fails.append(f"own-token head {h} is not causal attention")
    # first query sees only key 0
    if np.max(np.abs(o[0, 0] - v[0, 0])) > 1e-12:
        fails.append("own-token query 0 does not return v0")
    return fails


def check_stripe_partial(stripe_partial, gather_stripe, place_logical_rows, gqa_attention, seed=7):
    """Partner r's partial equals attention over the keys found in r's pool by physical addressing."""
    fails = []
    rng = np.random.default_rng(seed)
    page_size, P, hkv, hq, d = 8, 4, 2, 4, 3
    L = 29
    num_pages = 1 + (L + page_size - 1) // page_size + 2
    bt = np.concatenate([rng.permutation(np.arange(1, num_pages))[: (L + page_size - 1) // page_size], [0, 0]])
    k = rng.standard_normal((L, hkv, d))
    v = rng.standard_normal((L, hkv, d))
    q = rng.standard_normal((1, hq, d))
    kp = place_logical_rows([k], [bt], [L], page_size, P, num_pages)
    vp = place_logical_rows([v], [bt], [L], page_size, P, num_pages)
    for r in range(P):
        kr = gather_stripe(kp[r], bt, L, page_size, P, r)
        vr = gather_stripe(vp[r], bt, L, page_size, P, r)
        ref_o, ref_l = gqa_attention(q, kr, vr, 0.5)
        o, l = stripe_partial(q, k, v, P, r, 0.5)
        if np.max(np.abs(o - ref_o)) > 1e-13 or np.max(np.abs(l - ref_l)) > 1e-13:
            fails.append(f"stripe {r} partial does not attend the keys its pool holds")
    return fails


def check_slot_map(slot_map):
    fails = []
    for row in read_golden("slot_map.txt"):
        ps, P, s, partner, phys = (int(x) for x in row.split())
        a, b = slot_map([s], ps, P)
        if (int(a[0]), int(b[0])) != (partner, phys):
            fails.append(f"golden slot {s} (page_size {ps}, P {P}): got {(int(a[0]), int(b[0]))}")
    for row in read_golden("slot_map_pages.txt"):
        ps, P, page, off, partner, ppage, poff = (int(x) for x in row.split())
        a, b = slot_map([page * ps + off], ps, P)
        if (int(a[0]), int(b[0])) != (partner, ppage * (ps // P) + poff):
            fails.append(f"golden page {page} offset {off} (page_size {ps}, P {P})")
    # round trip and bijection over a full small pool
    for ps in (4, 16, 64):
        for P in (1, 2, 4):
            if ps % P:
                continue
            num_pages = 5
            s = np.arange(num_pages * ps)
            a, b = slot_map(s, ps, P)
            if not np.array_equal(b * P + a, s):
                fails.append(f"round trip fails (page_size {ps}, P {P})")
            pp = ps // P
            for r in range(P):
                got = np.sort(b[a == r])
                if not np.array_equal(got, np.arange(num_pages * pp)):
                    fails.append(f"partner {r} slots are not a bijection onto [0, {num_pages * pp})")
    return fails


def check_stripes(stripe_positions):
    fails = []
    for row in read_golden("stripes.txt"):
        head, _, tail = row.partition(":")
        L, P, r, cnt = (int(x) for x in head.split())
        pos = [int(x) for x in tail.split()]
        got = list(stripe_positions(L, P, r))
        if got != pos or len(got) != cnt:
            fails.append(f"stripe (L={L}, P={P}, r={r}) = {got}, expected {pos}")
    return fails


# ------------------------------------------------------------------------------------------------ interleave
def deal_page(page, page_size, P, I):
    """Independent construction of the interleaved placement of one page: walk its slots in order, hand each run of I
    slots to the next partner in turn, and let every partner fill its own physical slots of the page in arrival
    order. Returns {logical slot: (partner, phys)}."""
    pp = page_size // P
    filled = [0] * P
    out = {}
    for off in range(page_size):
        run = off // I
        partner = run - (run // P) * P                 # runs go to partners 0, 1, ..., P-1, 0, ...
        out[page * page_size + off] = (partner, page * pp + filled[partner])
        filled[partner] += 1
    return out


def check_interleave_slot_map(slot_map):
    """slot_map(s, page_size, P, I) against hand-dealt golden values and the dealing construction."""
    fails = []
    for row in read_golden("slot_map_interleave.txt"):
        ps, P, I, s, partner, phys = (int(x) for x in row.split())
        a, b = slot_map([s], ps, P, I)
        if (int(a[0]), int(b[0])) != (partner, phys):
            fails.append(f"golden slot {s} (page_size {ps}, P {P}, I {I}): got {(int(a[0]), int(b[0]))}")
    for ps, P, I in ((8, 2, 2), (16, 4, 2), (16, 2, 4), (32, 4, 4), (64, 4, 16), (16, 1, 4), (12, 3, 2)):
        for page in (0, 1, 5):
            dealt = deal_page(page, ps, P, I)
            slots = sorted(dealt)
            a, b = slot_map(slots, ps, P, I)
            got = {s: (int(x), int(y)) for s, x, y in zip(slots, a, b)}
            if got != dealt:
                fails.append(f"placement differs from the dealing (page_size {ps}, P {P}, I {I}, page {page})")
    return fails


def check_interleave_stripes(stripe_positions, stripe_len):
    """Membership against hand-worked lists, and the count against its closed form
    L_r = floor(L / (I P)) * I + min(max(L mod (I P) - r I, 0), I)."""
    fails = []
    for row in read_golden("stripes_interleave.txt"):
        head, _, tail = row.partition(":")
        L, P, I, r, cnt = (int(x) for x in head.split())
        pos = [int(x) for x in tail.split()]
        got = list(stripe_positions(L, P, r, I))
        if got != pos or len(got) != cnt:
            fails.append(f"stripe (L={L}, P={P}, I={I}, r={r}) = {got}, expected {pos}")
    for L in (0, 1, 5, 16, 37, 100):
        for P, I in ((2, 2), (4, 2), (3, 4), (1, 8)):
            for r in range(P):
                closed = (L // (I * P)) * I + min(max(L % (I * P) - r * I, 0), I)
                if stripe_len(L, P, r, I) != closed:
                    fails.append(f"stripe length (L={L}, P={P}, I={I}, r={r}) is not the closed form")
    return fails


def check_interleave_stripe_partial(stripe_partial, gather_stripe, place_logical_rows, gqa_attention, seed=8):
    """With interleave, partner r's partial equals attention over the keys found in r's pool by physical addressing."""
    fails = []
    rng = np.random.default_rng(seed)
    for page_size, P, I in ((8, 2, 2), (16, 4, 2), (16, 2, 4)):
        hkv, hq, d, L = 2, 4, 3, 45
        npg = (L + page_size - 1) // page_size
        num_pages = 1 + npg + 2
        bt = np.concatenate([rng.permutation(np.arange(1, num_pages))[:npg], [0, 0]])
        k = rng.standard_normal((L, hkv, d))
        v = rng.standard_normal((L, hkv, d))
        q = rng.standard_normal((2, hq, d))
        kp = place_logical_rows([k], [bt], [L], page_size, P, num_pages, interleave=I)
        vp = place_logical_rows([v], [bt], [L], page_size, P, num_pages, interleave=I)
        for r in range(P):
            kr = gather_stripe(kp[r], bt, L, page_size, P, r, I)
            vr = gather_stripe(vp[r], bt, L, page_size, P, r, I)
            ref_o, ref_l = gqa_attention(q, kr, vr, 0.5)
            o, l = stripe_partial(q, k, v, P, r, 0.5, I)
            if np.max(np.abs(o - ref_o)) > 1e-13 or np.max(np.abs(l - ref_l)) > 1e-13:
                fails.append(f"stripe {r} (page_size {page_size}, P {P}, I {I}) does not attend its pool's keys")
    return fails


# ------------------------------------------------------------------------------------------------------ fp8
def check_e4m3(e4m3_value, dequantize):
    """Code values against the hand-decoded table and torch's float8_e4m3fn (a library routine) for all 256 codes;
    dequantization is code value times descale."""
    import torch
    fails = []
    for row in read_golden("fp8_e4m3.txt"):
        code, val = row.split()
        got, want = e4m3_value(int(code, 16)), float(val)
        if not ((math.isnan(got) and math.isnan(want)) or (got == want and math.copysign(1, got) == math.copysign(1, want))):
            fails.append(f"code {code}: {got} != {want}")
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = np.array([e4m3_value(c) for c in range(256)])
    if not np.array_equal(np.isnan(mine), np.isnan(lib)) or not np.array_equal(mine[~np.isnan(mine)], lib[~np.isnan(lib)]):
        fails.append("code values differ from torch.float8_e4m3fn")
    codes = np.array([[0x38, 0x40], [0xb8, 0x01]])
    dq = dequantize(codes, 0.37)
    want = np.array([[0.37, 0.74], [-0.37, 0.37 * 2.0 ** -9]])
    if not np.allclose(dq, want, rtol=0, atol=1e-15):
        fails.append(f"dequantize is not code value times descale: {dq}")
    return fails
