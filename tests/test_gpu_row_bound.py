"""Rows with more query tokens than the host bound max_row_tokens.

Each call attends only the first max_row_tokens tokens of every row; those match the same call given the true bound
(to the output tolerance, since the launch shape and so the split of the context may differ), and every token past
the bound comes out as padding, (0, -inf), in every stripe's partial, the merged output and the own-token output.
Outputs start poisoned with NaN so that a token no kernel writes fails the check. One case per kernel path: the bf16
decode kernel (balanced, fixed splits, fp8 pools, fused merge), the extend kernel, MLA (bf16 and fp8 latent pools),
the generic kernel and both own-token kernels; a bound of zero turns every real token into padding."""
import numpy as np
import pytest
import torch

import workloads
from cp_slot_map_amd import api, pool
from tests.gpu_helpers import check_lse, check_out, say

pytestmark = pytest.mark.gpu
DEV = "cuda"

_DEC = dict(batch=5, new_lengths=[1, 3, 2, 4, 1], ctx_lengths=[17, 300, 1031, 4100, 5])
_EXT = dict(batch=4, new_lengths=[1, 40, 7, 100], ctx_lengths=[500, 3000, 40, 9])
_MLA = dict(batch=3, new_lengths=[1, 3, 2], ctx_lengths=[7, 130, 2000])

PAGED = [
    # id, workload, overrides, understated bound, fixed splits
    ("decode", "llama8b", _DEC, 2, False),
    ("decode-zero", "llama8b", _DEC, 0, False),
    ("decode-fixed", "llama8b", _DEC, 2, True),
    ("decode-fp8", "llama8b", dict(_DEC, kv_dtype="fp8"), 3, False),
    ("extend", "llama8b", _EXT, 33, False),            # 33 tokens x 4 heads a kv head: the extend kernel
    ("extend-to-decode", "llama8b", _EXT, 3, False),   # 3 x 4 rows: the decode kernel takes the call
    ("mla", "mla", _MLA, 1, False),
    ("mla-zero", "mla", _MLA, 0, False),
    ("mla-fp8", "mla", dict(_MLA, kv_dtype="fp8"), 2, False),
    ("generic", "tiny", dict(new_lengths=[1, 3, 2, 1]), 1, False),
    ("generic-zero", "tiny", dict(new_lengths=[1, 3, 2, 1]), 0, False),
]


def _paged(batch, wl, bound, fixed, merged):
    T, Hq, Dv = batch.q.shape[0], batch.q.shape[1], wl.head_dim_v
    o = torch.full((wl.partners, T, Hq, Dv), float("nan"), dtype=torch.float32, device=DEV)
    l = torch.full((wl.partners, T, Hq), float("nan"), dtype=torch.float32, device=DEV)
    kw = dict(page_size=wl.page_size, partners=wl.partners, scale=wl.scale, kind=wl.kind,
              max_ctx_len=batch.max_ctx_len, max_row_tokens=bound, out=o, lse=l, fixed_splits=fixed,
              interleave=wl.interleave, k_descale=wl.k_descale, v_descale=wl.v_descale)
    args = (batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len, batch.block_table)
    if not merged:
        api.paged_attn_partial(*args, **kw)
        return o, l, None, None
    mo = torch.full((T, Hq, Dv), float("nan"), dtype=torch.float32, device=DEV)
    ml = torch.full((T, Hq), float("nan"), dtype=torch.float32, device=DEV)
    api.paged_attn_merged(*args, merged=mo, merged_lse=ml, **kw)
    return o, l, mo, ml


def _check_bound(qrs, bound, under, full, what):
    """under/full: (out [..., T, H, D], lse [..., T, H]) with the token axis second to last of lse."""
    (uo, ul), (fo, fl) = [(x.detach().cpu(), y.detach().cpu()) for x, y in (under, full)]
    nbad = 0
    for b in range(len(qrs) - 1):
        t0, t1 = int(qrs[b]), int(qrs[b + 1])
        k = min(t1 - t0, bound)
        if k > 0:
            check_out(uo[..., t0:t0 + k, :, :], fo[..., t0:t0 + k, :, :].double().numpy(), f"{what} row {b} out")
            check_lse(ul[..., t0:t0 + k, :], fl[..., t0:t0 + k, :].double().numpy(), f"{what} row {b} lse")
        if t0 + k < t1:
            nbad += t1 - t0 - k
            assert torch.all(uo[..., t0 + k:t1, :, :] == 0), f"{what} row {b}: tokens past the bound not zero"
            assert torch.all(torch.isneginf(ul[..., t0 + k:t1, :])), f"{what} row {b}: lse past the bound not -inf"
    assert nbad > 0, "the case has no token past the bound"
    return nbad


@pytest.mark.parametrize("merged", [False, True], ids=["partial", "merged"])
@pytest.mark.parametrize("case,name,kw,bound,fixed", PAGED, ids=[c[0] for c in PAGED])
def test_paged_tokens_past_the_row_bound(case, name, kw, bound, fixed, merged):
    wl = workloads.make(name, **kw)
    batch = pool.build_batch(wl, DEV)
    qrs = wl.q_row_start
    true_bound = int(np.max(np.diff(qrs)))
    assert bound < true_bound
    say(f"row bound {case} {'merged' if merged else 'partial'}: bound {bound} of {true_bound}")
    uo, ul, umo, uml = _paged(batch, wl, bound, fixed, merged)
    fo, fl, fmo, fml = _paged(batch, wl, true_bound, fixed, merged)
    torch.cuda.synchronize()
    n = _check_bound(qrs, bound, (uo, ul), (fo, fl), f"{case} partials")
    if merged:
        _check_bound(qrs, bound, (umo, uml), (fmo, fml), f"{case} merged")
    t = wl.num_tokens
    assert torch.all(torch.isneginf(ul[:, t:])) and torch.all(uo[:, t:] == 0)   # the bucket's padding tokens
    say(f"  {n} tokens past the bound came out as padding")


OWN = [
    # id, dtype, head dim, query heads, kv heads, row lengths, bound
    ("bf16", torch.bfloat16, 128, 32, 8, [1, 40, 7, 100, 0], 33),
    ("bf16-zero", torch.bfloat16, 128, 32, 8, [1, 40, 7, 100, 0], 0),
    ("generic-f32", torch.float32, 64, 4, 1, [1, 9, 3, 17], 4),
    ("generic-bf16", torch.bfloat16, 64, 8, 2, [5, 1, 12], 2),
]


@pytest.mark.parametrize("case,dtype,D,Hq,Hkv,lens,bound", OWN, ids=[c[0] for c in OWN])
def test_own_token_tokens_past_the_row_bound(case, dtype, D, Hq, Hkv, lens, bound):
    g = torch.Generator().manual_seed(77)
    T = sum(lens) + 3                                  # three padding tokens at the end of the bucket
    q = torch.randn(T, Hq, D, generator=g).to(dtype).to(DEV)
    k = torch.randn(T, Hkv, D, generator=g).to(dtype).to(DEV)
    v = torch.randn(T, Hkv, D, generator=g).to(dtype).to(DEV)
    qrs = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu = torch.from_numpy(qrs).to(DEV)
    say(f"own-token row bound {case}: bound {bound} of {max(lens)}")
    res = []
    for mrt in (bound, max(lens)):
        o = torch.full((T, Hq, D), float("nan"), dtype=torch.float32, device=DEV)
        l = torch.full((T, Hq), float("nan"), dtype=torch.float32, device=DEV)
        api.own_token_attn(q, k, v, cu, scale=D ** -0.5, max_row_tokens=mrt, out=o, lse=l)
        res.append((o, l))
    torch.cuda.synchronize()
    _check_bound(qrs, bound, res[0], res[1], f"own {case}")
    o, l = res[0]
    assert torch.all(o[sum(lens):] == 0) and torch.all(torch.isneginf(l[sum(lens):]))
