"""Oracle for the MLP chain X.W1 -> GeLU -> .W2 (test infrastructure only).

Follows the cuSync paper, section "GPT Models" and Fig. "Architecture of two
building blocks of GPT models" (a): the first GeMM is fused with GeLU,
XW1 = GeLU(X x W1) with X:[B,H], W1:[H,4H/8]; the second GeMM is
XW12 = XW1 x W2 with W2:[4H/8,H].  Readings where the page is silent:

* GeLU is the exact form 0.5 x (1 + erf(x / sqrt 2)) (the page never defines
  it); the tanh approximation is available as an option.
* No bias (none is shown).
* The intermediate XW1 is stored in fp16 (the page's fp16 weights), so it is
  rounded once to fp16, nearest-even, after GeLU; any NaN is canonicalised
  (sentinel guide, 4.6.4.3) so every sync policy stores the same bits.
* Weights are row-major K x N exactly as the shapes are written.

The contraction itself is a library matmul in float64 on the exact input
values: the plain definition A[i,j] = sum_k X[i,k] W1[k,j].
"""

import numpy as np
from scipy.special import erf

from .common import rne_fp16, canon_nan_fp16, rne_bf16, bf16_bits, bf16_values


def gelu_erf(x):
    """Exact GeLU, x * Phi(x) with Phi the standard normal CDF, in float64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


def gelu_tanh(x):
    """tanh approximation of GeLU (opt-in), in float64."""
    x = np.asarray(x, dtype=np.float64)
    c = np.sqrt(2.0 / np.pi)
    return 0.5 * x * (1.0 + np.tanh(c * (x + 0.044715 * x ** 3)))


_ACTS = {
    "erf": gelu_erf,
    "tanh": gelu_tanh,
    "none": lambda a: np.asarray(a, dtype=np.float64),
}


def mlp_chain(X, W1, W2, act="erf"):
    """Full MLP chain on fp16 inputs.

    Returns ``(G, Z, Y)``:
      G  float64 [M,F]  activation of the accumulated first product, before
                        rounding (compared with the GPU's fp32 intermediate);
      Z  float16 [M,F]  the stored intermediate, RNE(G) with NaN canonicalised;
      Y  float16 [M,H]  RNE(Z x W2).
    """
    X = np.asarray(X, dtype=np.float16)
    W1 = np.asarray(W1, dtype=np.float16)
    W2 = np.asarray(W2, dtype=np.float16)
    M, H = X.shape
    H1, F = W1.shape
    F2, H2 = W2.shape
    if H1 != H or F2 != F:
        raise ValueError("shape mismatch: X[M,H] W1[H,F] W2[F,H2]")
    A = X.astype(np.float64) @ W1.astype(np.float64)
    G = _ACTS[act](A)
    Z = canon_nan_fp16(rne_fp16(G))
    Y = rne_fp16(Z.astype(np.float64) @ W2.astype(np.float64))
    return G, Z, Y


def mlp_chain_rows(X, W1, W2, rows, act="erf"):
    """The chain restricted to the given rows of X.

    Each output row depends only on the same input row (both products are
    row-wise in X), so this equals ``mlp_chain(X, ...)`` at those rows; it lets
    the full-size parity tests check sampled rows in seconds.
    """
    rows = np.asarray(rows, dtype=np.int64)
    return mlp_chain(np.asarray(X)[rows], W1, W2, act=act)


def mlp_chain_bf16(Xb, W1b, W2b, act="erf"):
    """The MLP chain with bf16 storage: inputs are bf16 bit patterns (uint16).

    Returns ``(G, Zb, Yb)``: G float64 as in ``mlp_chain``; Zb the stored
    intermediate's bits, RNE_bf16(G) with NaN canonicalised to 0x7FC0; Yb the
    bits of RNE_bf16(Z x W2).  Same products and readings as the fp16 chain;
    only the rounding at the two stores differs.
    """
    X, W1, W2 = (bf16_values(b) for b in (Xb, W1b, W2b))
    M, H = X.shape
    if W1.shape[0] != H or W2.shape[0] != W1.shape[1]:
        raise ValueError("shape mismatch: X[M,H] W1[H,F] W2[F,H2]")
    G = _ACTS[act](X @ W1)
    Zb = bf16_bits(rne_bf16(G))
    Yb = bf16_bits(rne_bf16(bf16_values(Zb) @ W2))
    return G, Zb, Yb
