"""Seeded sweep of call shapes the named cases do not pin one by one: random row counts, context and in-step lengths
(zero included), partner counts, page sizes, interleave sizes, pool element types, padding rows and both split
schedules, for the decode, extend (mixed), MLA and generic fp32 paths. Every row's merged output and LSE, and every stripe's and the
own-token partial, are compared with the float64 oracle; padding tokens must come out as (0, -inf). The case list is
drawn from a fixed seed on the host, so every run checks the same shapes."""
import numpy as np
import pytest

import workloads
from cp_slot_map_amd import pool
from tests.gpu_helpers import check_padding, compare_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _cases(n=40, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for k in range(n):
        name = ("llama8b", "mixed", "mla", "tiny")[k % 4]
        P = int(rng.choice([1, 2, 4, 8]))
        page = int(rng.choice([16, 32, 64])) if name != "mla" else int(rng.choice([32, 64]))
        inter = [i for i in (1, 2, 4) if page % (i * P) == 0]
        I = int(rng.choice(inter))
        B = int(rng.integers(1, 6))
        ctx = [int(x) for x in rng.integers(0, 2500, size=B)]
        if rng.random() < 0.4:
            ctx[int(rng.integers(0, B))] = int(rng.integers(0, 3))        # empty or near-empty contexts
        kw = dict(batch=B, ctx_lengths=ctx, partners=P, page_size=page, interleave=I,
                  kv_dtype=str(rng.choice(["same", "fp8"])), pad_rows=int(rng.integers(0, 3)))
        if name == "tiny":                                                   # fp32 pools: the generic kernel
            kw["kv_dtype"] = "same"
        if name == "mixed":
            kw["new_lengths"] = [int(x) for x in rng.integers(1, 400 if k % 2 else 40, size=B)]
        if name == "mla":
            kw["num_q_heads"] = int(rng.choice([16, 32, 64, 128]))
        fixed = bool(rng.random() < 0.3)                                     # the call-independent schedule
        out.append((f"{k:02d}-{name}{'-fixed' if fixed else ''}", name, kw, fixed))
    return out


CASES = _cases()


@pytest.mark.parametrize("case,name,kw,fixed", CASES, ids=[c[0] for c in CASES])
def test_sweep_against_the_oracle(case, name, kw, fixed):
    wl = workloads.make(name, **kw)
    say(f"sweep {case}: P={wl.partners} page={wl.page_size} I={wl.interleave} kv={wl.kv_dtype} "
        f"ctx={list(wl.ctx_len)} new={list(wl.new_len)} pad_rows={kw['pad_rows']} fixed_splits={fixed}")
    batch = pool.build_batch(wl, DEV)
    res = pool.run_step(batch, fixed_splits=fixed)
    w = compare_rows(wl, batch, res, range(wl.batch), DEV, check_partials=True)
    check_padding(wl, res)
    say(f"  worst errors {w}")
