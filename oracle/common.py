"""Rounding and error helpers shared by the oracle modules (test infrastructure).

The chain stores its intermediate and its output in fp16 (or bf16).  The
oracle rounds exactly there, once, with round-to-nearest-even from the float64
value (``numpy.float16`` conversion from float64 is correctly rounded, ties to
even; bf16 rounding is written out below), keeping subnormals.
"""

import numpy as np

# Quiet NaN that a producer substitutes for any NaN result so that it can never
# store the all-ones sentinel pattern (sentinel guide, 4.6.4.3 Producer Rules:
# the producer must never emit the sentinel; a NaN result is replaced).
CANON_NAN_FP16 = np.uint16(0x7E00)
SENTINEL_FP16 = np.uint16(0xFFFF)


def rne_fp16(x):
    """Round a float64 array to fp16, nearest-even, subnormals kept."""
    return np.asarray(x, dtype=np.float64).astype(np.float16)


def canon_nan_fp16(h):
    """Replace every fp16 NaN bit pattern by the canonical quiet NaN 0x7E00.

    Follows the sentinel guide, 4.6.4.3 (canonicalisation): results are
    canonicalised before they are stored so the reserved pattern never leaks.
    Non-NaN values, including -0.0 and infinities, are left untouched.
    """
    h = np.asarray(h, dtype=np.float16).copy()
    bits = h.view(np.uint16)
    bits[np.isnan(h)] = CANON_NAN_FP16
    return h


# bfloat16: fp32's sign and 8-bit exponent (bias 127) with 7 fraction bits, so
# 8 significant bits, normals from 2^-126, subnormals down to 2^-133.  numpy
# has no bf16 type: values travel as uint16 bit patterns, and the rounding is
# done here in float64 arithmetic.  Canonical quiet NaN for stored results
# (the sentinel guide's producer rule, as for fp16): 0x7FC0.
CANON_NAN_BF16 = np.uint16(0x7FC0)


def rne_bf16(x):
    """Round float64 values to the nearest bf16 value, ties to even, keeping
    subnormals; values from the top binade that round past the largest finite
    value become infinities.  Returns float64 arrays of bf16 values (NaN and
    infinities pass through).  For |x| in [2^E, 2^(E+1)) the spacing of bf16
    values is 2^(max(E, -126) - 7); x divided by that power of two is exact,
    and numpy's round() rounds half to even."""
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)  # a = m 2^e, m in [0.5, 1): E = e - 1
    q = np.ldexp(1.0, np.maximum(e.astype(np.int64) - 1, -126) - 7)
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.round(a / q) * q
        r = np.where(r >= 2.0 ** 128, np.inf, r)
        return np.where(np.isfinite(x), np.copysign(r, x), x)


def bf16_bits(v):
    """Bit patterns of float64 values that are bf16 values (exact: a bf16
    value is an fp32 value whose low 16 bits are zero); NaN -> 0x7FC0."""
    v = np.asarray(v, dtype=np.float64)
    b = (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    b[np.isnan(v)] = CANON_NAN_BF16
    return b


def bf16_values(bits):
    """float64 values of bf16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def normwise_rel_err(got, ref):
    """max_i |got_i - ref_i| / max_i |ref_i| in float64 (0 if ref is all zero
    and got equals it).  The bound is read normwise because an elementwise
    ratio is undefined at zero-valued outputs."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    num = np.max(np.abs(g - r)) if g.size else 0.0
    den = np.max(np.abs(r)) if r.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else np.inf
    return float(num / den)
