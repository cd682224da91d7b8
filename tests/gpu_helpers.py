"""Shared pieces of the GPU parity tests: tolerances, comparisons and the oracle side of a batch.

Tolerances (bf16 or fp32 inputs, fp32 accumulation):

* every output, elementwise: |gpu - ref| <= 2e-3 + 1e-2 * |ref|;
* every fp32 output (the per-stripe partials, the own-token partial and an fp32 merged result) also on its own:
  max |gpu - ref| <= 2e-3. A bf16 merged result is held to the elementwise bound only, since one bf16 rounding of a
  value of magnitude x already moves it by up to x * 2^-9;
* LSE: |gpu - ref| <= 1e-4 absolute, with -inf matching -inf exactly;
* integer and addressing results: bit-exact.

Every comparison records its worst absolute error under the running test's id (``MARGINS``); the test session prints
them at the end, so a run's record shows how close each case came to its bound.
"""
from __future__ import annotations

import os

import numpy as np
import torch

import oracle
import workloads

OUT_ABS, OUT_REL, LSE_ABS = 2e-3, 1e-2, 1e-4

# test id -> {"out": worst |d| of any output, "out32": worst of fp32 outputs, "lse": worst |d| of an lse,
#             "rel": worst |d| / (2e-3 + 1e-2 |ref|) of any output}
MARGINS = {}


def _test_id():
    cur = os.environ.get("PYTEST_CURRENT_TEST", "?")
    return cur.rsplit(" (", 1)[0]


def _record(key, value):
    m = MARGINS.setdefault(_test_id(), {})
    m[key] = max(m.get(key, 0.0), float(value))


def say(msg):
    print(msg, flush=True)


def _host(x):
    if hasattr(x, "detach"):
        return x.detach().float().cpu().numpy().astype(np.float64), x.dtype == torch.float32
    return np.asarray(x, dtype=np.float64), True


def check_out(gpu, ref, what=""):
    """Output check: the elementwise bound for every dtype, plus max-abs 2e-3 when the GPU result is fp32."""
    g, is_f32 = _host(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    if not g.size:
        return 0.0
    err = np.abs(g - ref)
    bound = OUT_ABS + OUT_REL * np.abs(ref)
    worst = float(err.max())
    _record("out", worst)
    _record("rel", float((err / bound).max()))
    bad = err > bound
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, max abs err "
                           f"{worst:.3e}")
    if is_f32:
        _record("out32", worst)
        assert worst <= OUT_ABS, f"{what}: fp32 output max abs err {worst:.3e} > {OUT_ABS:g}"
    return worst


def check_lse(gpu, ref, what=""):
    g, _ = _host(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    ginf, rinf = np.isneginf(g), np.isneginf(ref)
    assert np.array_equal(ginf, rinf), f"{what}: -inf pattern differs ({int(ginf.sum())} vs {int(rinf.sum())})"
    fin = ~rinf
    assert np.all(np.isfinite(g[fin])), f"{what}: non-finite lse"
    err = np.abs(g[fin] - ref[fin])
    worst = float(err.max()) if err.size else 0.0
    _record("lse", worst)
    assert worst <= LSE_ABS, f"{what}: lse max abs err {worst:.3e}"
    return worst


def compare_rows(wl, batch, res, rows, device, check_partials=True):
    """Compare a step's GPU results on `rows` with the oracle; returns worst errors.

    ``check_partials``: True (every row in ``rows``), False, or a collection of rows whose per-stripe and own-token
    partials are compared as well; the merged output and LSE are compared on every row in ``rows``. The oracle runs
    on a few host threads (numpy releases the interpreter lock in its kernels) while the next rows are regenerated.
    """
    from concurrent.futures import ThreadPoolExecutor

    mo, ml, po, pl, own = res
    qrs = wl.q_row_start
    rows = [int(b) for b in rows if int(wl.new_len[b]) > 0]
    part_rows = set(rows) if check_partials is True else set() if not check_partials else set(map(int, check_partials))
    worst = {"out": 0.0, "lse": 0.0, "part_out": 0.0, "part_lse": 0.0}
    # GPU results of the rows to compare, on the host once
    mo_h, ml_h = mo.detach().cpu(), ml.detach().cpu()
    po_h, pl_h = (po.detach().cpu(), pl.detach().cpu()) if part_rows else (None, None)
    own_h = (own[0].detach().cpu(), own[1].detach().cpu()) if (own is not None and part_rows) else None

    def host_inputs(b):
        rv = workloads.row_values(wl, b, device)
        q, k, v = rv.q.cpu(), rv.k_ctx.cpu(), rv.v_ctx.cpu()
        if wl.kv_dtype == "fp8":    # the pools hold E4M3 codes: what they stand for, by the oracle's own decoding
            k = oracle.dequantize_e4m3(k.view(torch.uint8), wl.k_descale)
            v = oracle.dequantize_e4m3(v.view(torch.uint8), wl.v_descale)
        kn = rv.k_new.cpu() if rv.k_new is not None else None
        vn = rv.v_new.cpu() if rv.v_new is not None else None
        return q, k, v, kn, vn

    def oracle_row(b, inputs):
        q, k, v, kn, vn = inputs
        parts = None
        if b in part_rows:
            parts, _ = oracle.row_partials(q, k, v, wl.partners, wl.scale, kn, vn, interleave=wl.interleave)
        full = oracle.row_attention(q, k, v, wl.scale, kn, vn)
        return b, parts, full

    with ThreadPoolExecutor(max_workers=6) as ex:
        futs = [ex.submit(oracle_row, b, host_inputs(b)) for b in rows]
        for f in futs:
            b, parts, full = f.result()
            n = int(wl.new_len[b])
            t0 = int(qrs[b])
            if parts is not None:
                for r in range(wl.partners):
                    worst["part_out"] = max(worst["part_out"], check_out(po_h[r, t0:t0 + n], parts[r][0],
                                                                         f"row {b} stripe {r} out"))
                    worst["part_lse"] = max(worst["part_lse"], check_lse(pl_h[r, t0:t0 + n], parts[r][1],
                                                                         f"row {b} stripe {r} lse"))
                if own_h is not None:
                    check_out(own_h[0][t0:t0 + n], parts[-1][0], f"row {b} own out")
                    check_lse(own_h[1][t0:t0 + n], parts[-1][1], f"row {b} own lse")
            worst["out"] = max(worst["out"], check_out(mo_h[t0:t0 + n], full[0], f"row {b} merged out"))
            worst["lse"] = max(worst["lse"], check_lse(ml_h[t0:t0 + n], full[1], f"row {b} merged lse"))
    return worst


def check_padding(wl, res, partial_rows_written=True):
    """Tokens past the real ones come out as (0, -inf) in every partial and in the merge (with the padding-lse-only
    flag, partial_rows_written=False: the partials' lse is -inf and their rows are not looked at)."""
    mo, ml, po, pl, own = res
    t = wl.num_tokens
    if t >= wl.bucket:
        return
    assert torch.all(mo[t:] == 0) and torch.all(torch.isneginf(ml[t:]))
    assert torch.all(torch.isneginf(pl[:, t:]))
    if partial_rows_written:
        assert torch.all(po[:, t:] == 0)
    if own is not None:
        assert torch.all(torch.isneginf(own[1][t:]))
        if partial_rows_written:
            assert torch.all(own[0][t:] == 0)
