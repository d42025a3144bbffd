"""fp64 CPU oracle for the fp8 (e4m3) attention forward.

TEST INFRASTRUCTURE ONLY (same rule as ``oracle.attention``): only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` use it; it
shares nothing with the HIP library.

What the path computes (ml-notes page, the notes on reduced-precision attention:
low-precision operands with high-precision accumulation and softmax statistics):
Q, K and V arrive as 8-bit e4m3 codes with one fp32 dequantisation factor per
tensor, x = decode(code) * descale.  The result is the plain attention of the
dequantised tensors (``oracle.attention.attention_forward``), so the oracle is that
definition applied to the decoded inputs.  How far an fp8 kernel may be from it
(the probabilities it feeds the matrix core are 8-bit too) is a property of the
kernel, bounded in its tests, not part of this definition.

e4m3 ("e4m3fn", the OCP 8-bit float): 1 sign bit, 4 exponent bits with bias 7,
3 mantissa bits; exponent field 0 encodes subnormals m/8 * 2^-6; no infinities;
the codes with all exponent and mantissa bits set (0x7F, 0xFF) are NaN.  Largest
finite magnitude 448, smallest subnormal 2^-9.
"""

from __future__ import annotations

import numpy as np

__all__ = ["decode_e4m3", "E4M3_MAX", "dequantize", "attention_forward_fp8",
           "attention_forward_fp8_rows"]

E4M3_MAX = 448.0


def decode_e4m3(codes) -> np.ndarray:
    """fp64 values of e4m3 codes (any integer array of 0..255)."""
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(m / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def dequantize(codes, descale: float) -> np.ndarray:
    if hasattr(codes, "numpy"):
        codes = codes.detach().cpu().numpy()
    return decode_e4m3(codes) * float(descale)


def attention_forward_fp8(q8, k8, v8, descale_q, descale_k, descale_v, scale, causal, **kw):
    """(O, LSE) of attention over the dequantised inputs, in fp64."""
    import oracle.attention as A
    q = dequantize(q8, descale_q)
    k = dequantize(k8, descale_k)
    v = dequantize(v8, descale_v)
    return A.attention_forward(q, k, v, scale, causal, **kw)


def attention_forward_fp8_rows(q8, k8, v8, descale_q, descale_k, descale_v, scale, causal, picks):
    """O and LSE of individually picked rows (b, h, i) of the same definition: the
    rows of ``attention_forward_fp8``, each computed against its whole key/value head
    (for checking rows of problems too large to evaluate whole)."""
    import oracle.attention as A
    q = dequantize(q8, descale_q)
    k = dequantize(k8, descale_k)
    v = dequantize(v8, descale_v)
    return A.attention_forward_rows(q, k, v, scale, causal, picks)
