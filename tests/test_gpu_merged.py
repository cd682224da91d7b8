"""cp_paged_attn_merged (every stripe's partial and their exact merge in one call) against the two-call path
(cp_paged_attn_partial, then cp_lse_merge told the real token count): the same bits, partials included, on the fused
bf16 decode path and on every path that falls back to the two calls; and against the oracle."""
import numpy as np
import pytest
import torch

import workloads
from cp_slot_map_amd import api, pool
from tests.gpu_helpers import check_padding, compare_rows, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = [
    ("llama8b", dict(batch=7, ctx_lengths=[1, 3, 4, 17, 255, 1031, 4100]), False),
    ("llama8b-pad", dict(batch=4, ctx_lengths=[3, 17, 300, 2100], pad_rows=2, bucket=4 + 7), False),
    ("llama8b-i4", dict(batch=4, ctx_lengths=[3, 17, 517, 2049], interleave=4), False),
    ("llama8b-fp8", dict(batch=5, ctx_lengths=[1, 9, 255, 1031, 4100], kv_dtype="fp8"), False),
    ("llama8b-fixed", dict(batch=7, ctx_lengths=[1, 3, 4, 17, 255, 1031, 4100]), True),
    ("longctx", dict(batch=4, ctx_lengths=[5, 100, 4097, 9001]), False),
    ("llama8b-p16", dict(batch=3, ctx_lengths=[5, 300, 2000], partners=16), False),   # more than 8 stripes: two calls
    ("mla", dict(batch=3, ctx_lengths=[7, 130, 2000]), False),
    ("mla-fp8", dict(batch=3, ctx_lengths=[7, 130, 2000], kv_dtype="fp8"), False),
    ("llama8b-ext", dict(batch=4, new_lengths=[1, 40, 7, 100], ctx_lengths=[500, 3000, 40, 9]), False),   # extend kernel
    ("llama8b-ext8", dict(batch=4, new_lengths=[1, 40, 7, 100], ctx_lengths=[500, 3000, 40, 9], kv_dtype="fp8"), False),
    ("tiny", dict(), False),
]


def _two_calls(batch, wl, out_dtype, fixed_splits):
    o, l = api.paged_attn_partial(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len,
                                  batch.block_table, page_size=wl.page_size, partners=wl.partners, scale=wl.scale,
                                  kind=wl.kind, max_ctx_len=batch.max_ctx_len, max_row_tokens=batch.max_row_tokens,
                                  fixed_splits=fixed_splits, interleave=wl.interleave, k_descale=wl.k_descale,
                                  v_descale=wl.v_descale)
    mo, ml = api.lse_merge([o[s] for s in range(wl.partners)], [l[s] for s in range(wl.partners)],
                           out_dtype=out_dtype, token_count=batch.q_row_start[-1:])
    return mo, ml, o, l


def _merged(batch, wl, out_dtype, fixed_splits):
    T, Hq = batch.q.shape[0], batch.q.shape[1]
    Dv = wl.head_dim_v
    # poisoned outputs: every element the call is responsible for must be written
    o = torch.full((wl.partners, T, Hq, Dv), float("nan"), dtype=torch.float32, device=DEV)
    l = torch.full((wl.partners, T, Hq), float("nan"), dtype=torch.float32, device=DEV)
    mo = torch.full((T, Hq, Dv), float("nan"), dtype=out_dtype, device=DEV)
    ml = torch.full((T, Hq), float("nan"), dtype=torch.float32, device=DEV)
    return api.paged_attn_merged(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len,
                                 batch.block_table, page_size=wl.page_size, partners=wl.partners, scale=wl.scale,
                                 kind=wl.kind, max_ctx_len=batch.max_ctx_len, max_row_tokens=batch.max_row_tokens,
                                 out=o, lse=l, merged=mo, merged_lse=ml, fixed_splits=fixed_splits,
                                 interleave=wl.interleave, k_descale=wl.k_descale, v_descale=wl.v_descale)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
@pytest.mark.parametrize("name,kw,fixed", CASES, ids=[c[0] for c in CASES])
def test_merged_call_matches_two_calls(name, kw, fixed, out_dtype):
    wl = workloads.make(name.split("-")[0], **kw)
    say(f"merged call {name} {out_dtype}")
    batch = pool.build_batch(wl, DEV)
    mo, ml, o, l = _merged(batch, wl, out_dtype, fixed)
    ro, rl, rpo, rpl = _two_calls(batch, wl, out_dtype, fixed)
    torch.cuda.synchronize()
    assert torch.equal(mo, ro) and torch.equal(ml, rl), "merged output differs from the two-call path"
    assert torch.equal(o, rpo) and torch.equal(l, rpl), "partials differ from the partial call's"
    if out_dtype == torch.float32:
        w = compare_rows(wl, batch, (mo, ml, o, l, None), range(wl.batch), DEV)
        say(f"  worst errors {w}")
    check_padding(wl, (mo, ml, o, l, None))


@pytest.mark.parametrize("name", ["llama8b", "longctx"])
def test_merged_call_full_size(name):
    """The configuration the benchmark times: the fused call's merged bf16 output and partials equal the two-call
    path's at full size, and every row's merged result matches the oracle."""
    wl = workloads.make(name)
    say(f"merged call full size {name}")
    batch = pool.build_batch(wl, DEV, fill=0.0)
    mo, ml, o, l = _merged(batch, wl, torch.bfloat16, False)
    ro, rl, rpo, rpl = _two_calls(batch, wl, torch.bfloat16, False)
    torch.cuda.synchronize()
    assert torch.equal(mo, ro) and torch.equal(ml, rl)
    assert torch.equal(o, rpo) and torch.equal(l, rpl)
    rng = np.random.default_rng(5)
    part_rows = sorted(set([int(np.argmin(wl.ctx_len)), int(np.argmax(wl.ctx_len))] +
                           [int(x) for x in rng.choice(wl.batch, size=3, replace=False)]))
    w = compare_rows(wl, batch, (mo, ml, o, l, None), range(wl.batch), DEV, check_partials=part_rows)
    say(f"  worst errors {w}")
    del batch, mo, ml, o, l, ro, rl, rpo, rpl
    torch.cuda.empty_cache()
