"""Slot placement of a context-parallel paged pool, in plain Python/numpy integers.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check and the CPU baseline use it.

Source: mstar PR #1124, "Context / Sequence Parallel 1/5: split the KV cache by position across GPUs (DCP)",
PR description and commit message. A pool with context parallelism spreads each page's token slots over P partners:
the token in logical slot s is kept by partner s mod P, at index floor(s / P) of that partner's own pool, while the
page ids in every block table stay the logical ones. A written token goes to its owner's real slot; every other rank
writes it to the sink page. The review thread on resident planning adds that each partner's pool holds page_size / P
slots a page.

Interleave: the vLLM compare view "[Core] Add explicit layer parallel plans" (FlashAttentionMetadataBuilder) reads a
KV-cache interleave size I from the parallel config but the pages state no placement for it. Reading taken: runs of I
consecutive logical slots go to one partner, partners in turn, and each partner packs its runs densely, so slot s is
kept by partner floor(s / I) mod P at index floor(s / (I * P)) * I + s mod I. I = 1 is the PR's rule.

Readings where the pages are silent (each listed in the design notes):
* slot s is a global logical slot, page_id * page_size + offset;
* I * P must divide page_size (otherwise the partner pools would not have whole pages): refused with ValueError;
* a negative slot marks a padding token that is written nowhere: partner -1, physical slot -1.
"""
from __future__ import annotations

import numpy as np


def _check(page_size: int, P: int, interleave: int = 1) -> None:
    if P < 1 or page_size < 1 or interleave < 1:
        raise ValueError(f"need P, page_size, interleave >= 1 (got {P}, {page_size}, {interleave})")
    if page_size % (P * interleave):
        raise ValueError(f"P * interleave = {P * interleave} must divide page_size={page_size}")


def slot_map(logical_slot, page_size: int, P: int, interleave: int = 1):
    """Map logical slots to (partner, physical slot). Negative slots give (-1, -1).

    Returns two int64 numpy arrays of the input's shape.
    """
    _check(page_size, P, interleave)
    I = interleave
    s = np.asarray(logical_slot, dtype=np.int64)
    partner = np.full(s.shape, -1, dtype=np.int64)
    phys = np.full(s.shape, -1, dtype=np.int64)
    flat_s, flat_p, flat_q = s.reshape(-1), partner.reshape(-1), phys.reshape(-1)
    for i, v in enumerate(flat_s.tolist()):       # plain Python integers: no vectorised shortcut to get wrong
        if v >= 0:
            flat_p[i] = (v // I) % P
            flat_q[i] = (v // (I * P)) * I + v % I
    return partner, phys


def slot_map_rank(logical_slot, page_size: int, P: int, rank: int, sink_slot: int, interleave: int = 1):
    """Per-rank write view: the owner writes the physical slot, every other rank writes ``sink_slot``.

    Negative (padding) slots give -1 on every rank: they are written nowhere.
    """
    if not 0 <= rank < P:
        raise ValueError(f"rank {rank} outside [0, {P})")
    partner, phys = slot_map(logical_slot, page_size, P, interleave)
    out = np.where(partner == rank, phys, np.int64(sink_slot))
    return np.where(partner < 0, np.int64(-1), out).astype(np.int64)


def stripe_positions(ctx_len: int, P: int, r: int, interleave: int = 1) -> np.ndarray:
    """Positions of a row's context that partner r holds: the t in [0, ctx_len) with floor(t / I) mod P == r.

    This follows from the slot rule when I * P divides page_size: slot = page * page_size + t mod page_size, so
    floor(slot / I) mod P == floor(t / I) mod P. The positions come out in increasing order (the stripe's local order).
    """
    I = interleave
    return np.array([t for t in range(int(ctx_len)) if (t // I) % P == r], dtype=np.int64)


def stripe_len(ctx_len: int, P: int, r: int, interleave: int = 1) -> int:
    return int(len(stripe_positions(ctx_len, P, r, interleave)))


def place_logical_rows(rows_kv, block_table, ctx_len, page_size: int, P: int, num_pages: int, fill=np.nan,
                       interleave: int = 1):
    """Write every row's logical context into P partner pools through :func:`slot_map`.

    ``rows_kv[b]`` is an array [ctx_len[b], ...] of per-token entries. Each pool is a dense array of
    ``num_pages * page_size // P`` physical slots; untouched slots keep ``fill``. Returns a list of P pools.
    """
    _check(page_size, P, interleave)
    pp = page_size // P
    feat = np.asarray(rows_kv[0]).shape[1:] if len(rows_kv) else ()
    pools = [np.full((num_pages * pp,) + tuple(feat), fill, dtype=np.float64) for _ in range(P)]
    for b, kv in enumerate(rows_kv):
        kv = np.asarray(kv, dtype=np.float64)
        for t in range(int(ctx_len[b])):
            page = int(block_table[b][t // page_size])
            s = page * page_size + t % page_size
            partner, phys = slot_map([s], page_size, P, interleave)
            pools[int(partner[0])][int(phys[0])] = kv[t]
    return pools


def gather_stripe(pool, block_table_row, ctx_len: int, page_size: int, P: int, r: int, interleave: int = 1):
    """Read back partner r's share of one row from its pool, in local order, by applying the slot rule per position.

    Local token j of stripe r is the j-th position t (in increasing order) with floor(t / I) mod P == r; its logical
    slot is page(t) * page_size + t mod page_size and it sits at that slot's physical index.
    """
    pos = stripe_positions(ctx_len, P, r, interleave)
    out = []
    for t in pos.tolist():
        s = int(block_table_row[t // page_size]) * page_size + t % page_size
        _, phys = slot_map([s], page_size, P, interleave)
        out.append(np.asarray(pool[int(phys[0])]))
    if not out:
        return np.zeros((0,) + tuple(np.asarray(pool).shape[1:]), dtype=np.float64)
    return np.stack(out)
