"""Dequantization of fp8 KV pools, in plain Python/numpy.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check and the CPU baseline use it.

Source: the vLLM compare view "[Core] Add explicit layer parallel plans" passes per-tensor k_descale and v_descale to
its flash_attn_varlen_func calls (the context call over the paged cache and the own-token call). Readings where the
pages are silent (listed in the design notes): an fp8 pool stores OCP 8-bit E4M3 codes (1 sign bit, 4 exponent bits
with bias 7, 3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; all-ones exponent with all-ones
mantissa is NaN; there are no infinities), and the value a code stands for is its decoded number times the tensor's
descale factor.
"""
from __future__ import annotations

import numpy as np


def e4m3_value(code: int) -> float:
    """The number an OCP E4M3 code stands for (code in 0..255)."""
    code = int(code)
    if not 0 <= code <= 255:
        raise ValueError(f"code {code} is not a byte")
    sign = -1.0 if code & 0x80 else 1.0
    exp = (code >> 3) & 0xF
    man = code & 0x7
    if exp == 0xF and man == 0x7:
        return float("nan")
    if exp == 0:
        return sign * (man / 8.0) * 2.0 ** -6
    return sign * (1.0 + man / 8.0) * 2.0 ** (exp - 7)


def dequantize_e4m3(codes, descale: float) -> np.ndarray:
    """float64 array of code values times descale; ``codes`` is any integer array (or torch uint8 tensor)."""
    if hasattr(codes, "detach"):
        codes = codes.detach().to("cpu").numpy()
    c = np.asarray(codes).astype(np.int64)
    table = np.array([e4m3_value(i) for i in range(256)], dtype=np.float64)
    return table[c] * float(descale)
