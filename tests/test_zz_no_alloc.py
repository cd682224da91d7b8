"""The no-allocation partial call (cp_paged_attn_partial_noalloc) against cp_paged_attn_partial with a caller
workspace: same kernels, so the same bits, on two calls in a row (the second smaller, after the first left its
contents in the shared static scratch), through the C ABI."""
import pytest
import torch

import workloads
from cp_slot_map_amd import _lib, api, pool

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(batch, wl, fixed_splits=False):
    common = dict(page_size=wl.page_size, partners=wl.partners, scale=wl.scale, kind=wl.kind,
                  max_ctx_len=batch.max_ctx_len, max_row_tokens=batch.max_row_tokens, fixed_splits=fixed_splits,
                  interleave=wl.interleave, k_descale=wl.k_descale, v_descale=wl.v_descale)
    args = (batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len, batch.block_table)
    ro, rl = api.paged_attn_partial(*args, **common)
    o = torch.full_like(ro, float("nan"))
    l = torch.full_like(rl, float("nan"))
    api.paged_attn_partial_noalloc(*args, out=o, lse=l, **common)
    torch.cuda.synchronize()
    return (ro, rl), (o, l)


CASES = [
    ("llama8b", dict(batch=6, ctx_lengths=[3, 17, 300, 2100, 8192, 77]), dict(batch=2, ctx_lengths=[900, 5])),
    ("longctx", dict(batch=3, ctx_lengths=[4097, 20000, 9]), dict(batch=1, ctx_lengths=[33])),
    ("mla", dict(batch=3, ctx_lengths=[7, 130, 5000]), dict(batch=2, ctx_lengths=[2, 64])),
    ("mixed", dict(batch=4, new_lengths=[1, 40, 3, 100], ctx_lengths=[0, 300, 2000, 50], pad_rows=1),
     dict(batch=2, new_lengths=[5, 1], ctx_lengths=[10, 0])),
    ("llama8b-fp8", dict(batch=5, ctx_lengths=[3, 300, 2100, 8192, 77], kv_dtype="fp8"),
     dict(batch=2, ctx_lengths=[900, 5], kv_dtype="fp8")),
    ("mla-fp8", dict(batch=3, ctx_lengths=[7, 130, 5000], kv_dtype="fp8"), dict(batch=1, ctx_lengths=[64], kv_dtype="fp8")),
]


@pytest.mark.parametrize("fixed_splits", [False, True], ids=["balanced", "fixed"])
@pytest.mark.parametrize("name,big,small", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_workspace_call(name, big, small, fixed_splits):
    print(f"noalloc {name} fixed_splits={fixed_splits}", flush=True)
    for kw in (big, small):                     # two calls in a row, the second with a smaller input
        wl = workloads.make(name.split("-")[0], **kw)
        batch = pool.build_batch(wl, DEV)
        (ro, rl), (o, l) = _both(batch, wl, fixed_splits)
        assert torch.equal(o, ro) and torch.equal(l, rl)


def test_noalloc_refuses_a_call_past_the_scratch():
    """A call whose workspace would exceed the static scratch is refused on the host, before anything is enqueued."""
    lib = _lib.load()
    cap = api.noalloc_scratch_bytes()
    assert cap == 64 << 20
    # MLA with a few long rows splits each stripe into many chunks, each with a record of Hq * 515 floats
    wl = workloads.make("mla", batch=8, ctx_lengths=[16384] * 8)
    batch = pool.build_batch(wl, DEV, fill=0.0)
    need = api.paged_attn_workspace_size(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len,
                                         batch.block_table, page_size=wl.page_size, partners=wl.partners,
                                         scale=wl.scale, kind="mla", max_ctx_len=batch.max_ctx_len,
                                         max_row_tokens=batch.max_row_tokens)
    assert need > cap
    o = torch.zeros((wl.partners, wl.bucket, wl.num_q_heads, 512), dtype=torch.float32, device=DEV)
    l = torch.zeros((wl.partners, wl.bucket, wl.num_q_heads), dtype=torch.float32, device=DEV)
    with pytest.raises(_lib.CpattnError, match="scratch"):
        api.paged_attn_partial_noalloc(batch.q, batch.k_pool, batch.v_pool, batch.q_row_start, batch.ctx_len,
                                       batch.block_table, page_size=wl.page_size, partners=wl.partners,
                                       scale=wl.scale, kind="mla", max_ctx_len=batch.max_ctx_len,
                                       max_row_tokens=batch.max_row_tokens, out=o, lse=l)
    torch.cuda.synchronize()
    assert torch.all(o == 0)                    # nothing ran
    assert lib.cp_paged_attn_noalloc_scratch_bytes() == cap
