"""Rounding and error helpers shared by the oracle modules (test infrastructure).

The chain stores its intermediate and its output in fp16.  The oracle rounds
exactly there, once, with round-to-nearest-even from the float64 value
(``numpy.float16`` conversion from float64 is correctly rounded, ties to even),
keeping fp16 subnormals.
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
