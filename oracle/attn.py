"""Oracle for the attention-score chain Q.K^T -> row softmax -> .V
(test infrastructure only).

Follows the cuSync paper, section "GPT Models" and Fig. "Architecture of two
building blocks of GPT models" (b), which fuses a dot product, Softmax and
Dropout and synchronises its rows with the producer (section "Synchronization
Policies", RowSync).  Readings where the page is silent or garbled: the chain
computed per (batch, head) is Sc = RNE16(scale * Q K^T) (scores stored in
fp16, NaN canonicalised), P = softmax over the key axis in float64, and
O = RNE16(P V); no mask and no dropout (the page gives no dropout RNG);
``scale`` is a parameter.  Tensors are [B, heads, S, d], contiguous.
``attn_chain_bf16`` is the same chain with the scores and the output stored
in bf16 (inputs given as bf16 bit patterns).
"""

import numpy as np

from .common import rne_fp16, canon_nan_fp16, rne_bf16, bf16_bits, bf16_values


def softmax_rows(S):
    """Numerically stable softmax along the last axis, float64:
    p = exp(s - max s) / sum exp(s - max s)."""
    S = np.asarray(S, dtype=np.float64)
    m = np.max(S, axis=-1, keepdims=True)
    e = np.exp(S - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def attn_chain(Q, K, V, scale=1.0):
    """Full attention chain.  Returns ``(A, Sc, P, O)``: A the float64 scaled
    scores before rounding, Sc their stored fp16 values, P the float64
    probabilities and O the fp16 output [B, heads, S, d]."""
    Q = np.asarray(Q, dtype=np.float16).astype(np.float64)
    K = np.asarray(K, dtype=np.float16).astype(np.float64)
    V = np.asarray(V, dtype=np.float16).astype(np.float64)
    A = np.float64(scale) * (Q @ np.swapaxes(K, -1, -2))
    Sc = canon_nan_fp16(rne_fp16(A))
    P = softmax_rows(Sc.astype(np.float64))
    O = rne_fp16(P @ V)
    return A, Sc, P, O


def attn_chain_rows(Q, K, V, b, h, rows, scale=1.0):
    """The chain for one (batch b, head h) restricted to the given query rows.

    A query row's output depends on its own scores only (softmax is per row),
    so this equals the full chain at those rows.  Returns ``(A, Sc, P, O)``
    for the selected rows, shapes [len(rows), S] and [len(rows), d].
    """
    rows = np.asarray(rows, dtype=np.int64)
    q = np.asarray(Q, dtype=np.float16)[b, h, rows][None, None]
    k = np.asarray(K, dtype=np.float16)[b, h][None, None]
    v = np.asarray(V, dtype=np.float16)[b, h][None, None]
    A, Sc, P, O = attn_chain(q, k, v, scale)
    return A[0, 0], Sc[0, 0], P[0, 0], O[0, 0]


def attn_chain_bf16(Qb, Kb, Vb, scale=1.0):
    """The attention chain with bf16 storage: Qb, Kb, Vb are bf16 bit patterns
    (uint16) [B, heads, S, d].  Returns ``(A, Scb, P, Ob)``: A the float64
    scaled scores before rounding, Scb the stored scores' bits
    RNE_bf16(A) (NaN canonicalised to 0x7FC0), P the float64 softmax of the
    stored scores and Ob the bits of RNE_bf16(P V)."""
    Q, K, V = (bf16_values(b) for b in (Qb, Kb, Vb))
    A = np.float64(scale) * (Q @ np.swapaxes(K, -1, -2))
    Scb = bf16_bits(rne_bf16(A))
    P = softmax_rows(bf16_values(Scb))
    Ob = bf16_bits(rne_bf16(P @ V))
    return A, Scb, P, Ob


def attn_chain_bf16_rows(Qb, Kb, Vb, b, h, rows, scale=1.0):
    """``attn_chain_bf16`` for one (batch b, head h) at the given query rows
    (a row's output depends on its own scores only)."""
    rows = np.asarray(rows, dtype=np.int64)
    q = np.asarray(Qb, dtype=np.uint16)[b, h, rows][None, None]
    k = np.asarray(Kb, dtype=np.uint16)[b, h][None, None]
    v = np.asarray(Vb, dtype=np.uint16)[b, h][None, None]
    A, Scb, P, Ob = attn_chain_bf16(q, k, v, scale)
    return A[0, 0], Scb[0, 0], P[0, 0], Ob[0, 0]
