"""Oracle for the dependent 3x3 conv pair (test infrastructure only).

Follows the cuSync paper, section "ResNet" and Table "Input/output image size,
kernel size, and input/output channels for each pair of Conv2D in ResNet-38":
each layer performs two Conv2D operations with the same kernel size and
channels.  Readings where the page is silent: NHWC activations, RSCK filters
(reduction index (r, s, c), output channels contiguous), zero padding, ReLU
between the two convolutions only, no bias or normalisation; the intermediate
is stored in fp16 (rounded once, NaN canonicalised), or in bf16 by
``conv_chain_bf16`` (the same products; only the rounding at the two stores
differs).
"""

import numpy as np

from .common import rne_fp16, canon_nan_fp16, rne_bf16, bf16_bits, bf16_values


def conv2d_nhwc(X, W, pad=1, stride=1):
    """Direct convolution (cross-correlation, as in deep-learning Conv2D).

    out[n,p,q,k] = sum_{r,s,c} Xpad[n, p*stride + r, q*stride + s, c] * W[r,s,c,k]

    written as a sum over the R*S taps of a library matmul over c, in float64.
    X: [N,H,W,C], W: [R,S,C,K] -> [N,P,Q,K] float64.
    """
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W, dtype=np.float64)
    N, H, Wd, C = X.shape
    R, S, C2, K = W.shape
    if C2 != C:
        raise ValueError("channel mismatch")
    P = (H + 2 * pad - R) // stride + 1
    Q = (Wd + 2 * pad - S) // stride + 1
    Xp = np.zeros((N, H + 2 * pad, Wd + 2 * pad, C), dtype=np.float64)
    Xp[:, pad:pad + H, pad:pad + Wd, :] = X
    out = np.zeros((N, P, Q, K), dtype=np.float64)
    for r in range(R):
        for s in range(S):
            patch = Xp[:, r:r + stride * (P - 1) + 1:stride,
                       s:s + stride * (Q - 1) + 1:stride, :]
            out += patch @ W[r, s]
    return out


def conv_chain(X, Wa, Wb, pad=1, stride=1):
    """Z = RNE16(ReLU(conv(X, Wa))), Y = RNE16(conv(Z, Wb)).

    Returns ``(G, Z, Y)`` with G the float64 ReLU output before rounding.
    """
    X = np.asarray(X, dtype=np.float16)
    A = conv2d_nhwc(X, np.asarray(Wa, np.float16), pad, stride)
    # ReLU as "negative -> 0, otherwise unchanged": a NaN stays NaN (and is
    # then canonicalised) and -0.0 stays -0.0.
    G = np.where(A < 0.0, 0.0, A)
    Z = canon_nan_fp16(rne_fp16(G))
    Y = rne_fp16(conv2d_nhwc(Z, np.asarray(Wb, np.float16), pad, stride))
    return G, Z, Y


def conv_chain_bf16(Xb, Wab, Wbb, pad=1, stride=1):
    """The conv pair with bf16 storage: inputs are bf16 bit patterns (uint16).

    Returns ``(G, Zb, Yb)``: G the float64 ReLU output before rounding (as in
    ``conv_chain``); Zb the stored intermediate's bits, RNE_bf16(G) with NaN
    canonicalised to 0x7FC0; Yb the bits of RNE_bf16(conv(Z, Wb)).
    """
    X, Wa, Wb = (bf16_values(b) for b in (Xb, Wab, Wbb))
    A = conv2d_nhwc(X, Wa, pad, stride)
    G = np.where(A < 0.0, 0.0, A)
    Zb = bf16_bits(rne_bf16(G))
    Yb = bf16_bits(rne_bf16(conv2d_nhwc(bf16_values(Zb), Wb, pad, stride)))
    return G, Zb, Yb
