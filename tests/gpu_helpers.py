"""Shared pieces of the GPU parity tests: tolerances, comparisons and the oracle side of a batch.

Tolerances (stated for bf16 inputs with fp32 accumulation): outputs |gpu - ref| <= 2e-3 + 1e-2 * |ref| elementwise,
LSE within 1e-4 absolute with -inf matching -inf exactly; integer and addressing results bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads

OUT_ABS, OUT_REL, LSE_ABS = 2e-3, 1e-2, 1e-4


def say(msg):
    print(msg, flush=True)


def check_out(gpu, ref, what=""):
    g = gpu.detach().float().cpu().numpy().astype(np.float64) if hasattr(gpu, "detach") else np.asarray(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    err = np.abs(g - ref)
    bad = err > OUT_ABS + OUT_REL * np.abs(ref)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside tolerance, max abs err "
                           f"{err.max():.3e}")
    return float(err.max()) if err.size else 0.0


def check_lse(gpu, ref, what=""):
    g = gpu.detach().float().cpu().numpy().astype(np.float64) if hasattr(gpu, "detach") else np.asarray(gpu)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, f"{what}: shape {g.shape} vs {ref.shape}"
    ginf, rinf = np.isneginf(g), np.isneginf(ref)
    assert np.array_equal(ginf, rinf), f"{what}: -inf pattern differs ({int(ginf.sum())} vs {int(rinf.sum())})"
    fin = ~rinf
    assert np.all(np.isfinite(g[fin])), f"{what}: non-finite lse"
    err = np.abs(g[fin] - ref[fin])
    assert (err <= LSE_ABS).all(), f"{what}: lse max abs err {err.max():.3e}"
    return float(err.max()) if err.size else 0.0


def row_oracle(wl, b, device):
    """Oracle partials and merged result of row b (values regenerated on `device`, copied to the host)."""
    rv = workloads.row_values(wl, b, device)
    q = rv.q.cpu()
    k, v = rv.k_ctx.cpu(), rv.v_ctx.cpu()
    if wl.kv_dtype == "fp8":        # the pools hold E4M3 codes: what they stand for, by the oracle's own decoding
        k = oracle.dequantize_e4m3(k.view(torch.uint8), wl.k_descale)
        v = oracle.dequantize_e4m3(v.view(torch.uint8), wl.v_descale)
    kn = rv.k_new.cpu() if rv.k_new is not None else None
    vn = rv.v_new.cpu() if rv.v_new is not None else None
    parts, merged = oracle.row_partials(q, k, v, wl.partners, wl.scale, kn, vn, interleave=wl.interleave)
    full = oracle.row_attention(q, k, v, wl.scale, kn, vn)
    return parts, merged, full


def compare_rows(wl, batch, res, rows, device, check_partials=True):
    """Compare a step's GPU results on `rows` with the oracle; returns worst errors."""
    mo, ml, po, pl, own = res
    qrs = wl.q_row_start
    worst = {"out": 0.0, "lse": 0.0, "part_out": 0.0, "part_lse": 0.0}
    for b in rows:
        n = int(wl.new_len[b])
        if n == 0:
            continue
        t0 = int(qrs[b])
        parts, merged, full = row_oracle(wl, b, device)
        if check_partials:
            for r in range(wl.partners):
                worst["part_out"] = max(worst["part_out"], check_out(po[r, t0:t0 + n], parts[r][0], f"row {b} stripe {r} out"))
                worst["part_lse"] = max(worst["part_lse"], check_lse(pl[r, t0:t0 + n], parts[r][1], f"row {b} stripe {r} lse"))
            if own is not None:
                check_out(own[0][t0:t0 + n], parts[-1][0], f"row {b} own out")
                check_lse(own[1][t0:t0 + n], parts[-1][1], f"row {b} own lse")
        worst["out"] = max(worst["out"], check_out(mo[t0:t0 + n], full[0], f"row {b} merged out"))
        worst["lse"] = max(worst["lse"], check_lse(ml[t0:t0 + n], full[1], f"row {b} merged lse"))
    return worst


def check_padding(wl, res):
    """Tokens past the real ones come out as (0, -inf) in every partial and in the merge."""
    mo, ml, po, pl, own = res
    t = wl.num_tokens
    if t >= wl.bucket:
        return
    assert torch.all(mo[t:] == 0) and torch.all(torch.isneginf(ml[t:]))
    assert torch.all(po[:, t:] == 0) and torch.all(torch.isneginf(pl[:, t:]))
    if own is not None:
        assert torch.all(own[0][t:] == 0) and torch.all(torch.isneginf(own[1][t:]))
