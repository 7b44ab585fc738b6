"""Oracle for the three-kernel self-attention block (test infrastructure only).

Follows the cuSync paper, section "GPT Models", Fig. "Architecture of two
building blocks of GPT models" (b) (one GPU's share of the 8-way model
parallel layer), and section "Synchronization Policies", paragraph
StridedSync, with the use case in "Self-Attention":

  stage 1  XQKV = X Wqkv, stored fp16: X [M, H], Wqkv [H, 3 Hs], Hs = heads * d.
           Its columns are three equal slices; the first holds the queries, the
           second the values paired with the queries in the score product and
           the third the vectors the probabilities weight (the page's listing
           names them XQ, XV, XK in that order).
  stage 2  per head h (columns h*d .. (h+1)*d of each slice): the fused dot
           product, O_h = softmax_rows(scale * Q_h S2_h^T) S3_h, stored fp16
           into XDot [M, Hs].  The M rows are the tokens of the batch.
  stage 3  Y = XDot W2, stored fp16: W2 [Hs, H].

Readings where the page is silent or garbled: no mask and no dropout (the page
gives no dropout generator); ``scale`` is a parameter; the scores and the
probabilities are not stored, so they are not rounded (float64 here); the
page's column slices are taken in their stated order.  The bf16 variant keeps
every step and rounds each of the three stores to bf16 (nearest, ties to
even) instead of fp16; the pages name no bf16 case.
"""

import numpy as np

from .common import rne_fp16, rne_bf16, bf16_bits, bf16_values
from .attn import softmax_rows


def selfattn_chain(X, Wqkv, W2, heads, d, scale):
    """Returns ``(XQKV, XDot, Y)`` as fp16 arrays."""
    X = np.asarray(X, dtype=np.float16).astype(np.float64)
    Wqkv = np.asarray(Wqkv, dtype=np.float16).astype(np.float64)
    W2 = np.asarray(W2, dtype=np.float16).astype(np.float64)
    Hs = heads * d
    assert Wqkv.shape[1] == 3 * Hs and W2.shape[0] == Hs
    XQKV = rne_fp16(X @ Wqkv)
    q = XQKV[:, :Hs].astype(np.float64)
    s2 = XQKV[:, Hs:2 * Hs].astype(np.float64)
    s3 = XQKV[:, 2 * Hs:].astype(np.float64)
    out = np.empty((X.shape[0], Hs), dtype=np.float64)
    for h in range(heads):
        c = slice(h * d, (h + 1) * d)
        P = softmax_rows(np.float64(scale) * (q[:, c] @ s2[:, c].T))
        out[:, c] = P @ s3[:, c]
    XDot = rne_fp16(out)
    Y = rne_fp16(XDot.astype(np.float64) @ W2)
    return XQKV, XDot, Y


def selfattn_rows(X, Wqkv, W2, heads, d, scale, rows, return_qkv=False):
    """The chain at selected token rows.  Row i of XDot needs row i of the
    query slice and every row of the other two slices, so all of XQKV is
    computed; XDot and Y only at ``rows``.  Returns ``(XDot, Y)``, or
    ``(XQKV, XDot, Y)`` with the whole stage-1 result if ``return_qkv``."""
    X = np.asarray(X, dtype=np.float16).astype(np.float64)
    Wqkv = np.asarray(Wqkv, dtype=np.float16).astype(np.float64)
    W2 = np.asarray(W2, dtype=np.float16).astype(np.float64)
    Hs = heads * d
    rows = np.asarray(rows, dtype=np.int64)
    XQKV = rne_fp16(X @ Wqkv)
    q = XQKV[rows, :Hs].astype(np.float64)
    s2 = XQKV[:, Hs:2 * Hs].astype(np.float64)
    s3 = XQKV[:, 2 * Hs:].astype(np.float64)
    out = np.empty((len(rows), Hs), dtype=np.float64)
    for h in range(heads):
        c = slice(h * d, (h + 1) * d)
        out[:, c] = softmax_rows(np.float64(scale) * (q[:, c] @ s2[:, c].T)) @ s3[:, c]
    XDot = rne_fp16(out)
    Y = rne_fp16(XDot.astype(np.float64) @ W2)
    if return_qkv:
        return XQKV, XDot, Y
    return XDot, Y


def _selfattn_bf16(X, Wqkv, W2, heads, d, scale, rows):
    """The chain on float64 values of bf16 inputs, with bf16 stores; XDot and
    Y at ``rows`` (all rows when None).  Returns float64 bf16 values."""
    Hs = heads * d
    assert Wqkv.shape[1] == 3 * Hs and W2.shape[0] == Hs
    XQKV = rne_bf16(X @ Wqkv)
    r = slice(None) if rows is None else np.asarray(rows, dtype=np.int64)
    q = XQKV[r, :Hs]
    s2 = XQKV[:, Hs:2 * Hs]
    s3 = XQKV[:, 2 * Hs:]
    out = np.empty((q.shape[0], Hs), dtype=np.float64)
    for h in range(heads):
        c = slice(h * d, (h + 1) * d)
        out[:, c] = softmax_rows(np.float64(scale) * (q[:, c] @ s2[:, c].T)) @ s3[:, c]
    XDot = rne_bf16(out)
    Y = rne_bf16(XDot @ W2)
    return XQKV, XDot, Y


def selfattn_chain_bf16(Xb, Wqkvb, W2b, heads, d, scale):
    """The chain with bf16 storage: inputs are bf16 bit patterns (uint16).
    Returns the bits ``(XQKVb, XDotb, Yb)`` (NaN canonicalised to 0x7FC0)."""
    X, Wqkv, W2 = (bf16_values(b) for b in (Xb, Wqkvb, W2b))
    return tuple(bf16_bits(v) for v in _selfattn_bf16(X, Wqkv, W2, heads, d, scale, None))


def selfattn_rows_bf16(Xb, Wqkvb, W2b, heads, d, scale, rows):
    """``selfattn_chain_bf16`` at selected token rows: the bits ``(XDotb, Yb)``
    of those rows (all of XQKV is needed for them)."""
    X, Wqkv, W2 = (bf16_values(b) for b in (Xb, Wqkvb, W2b))
    _, XDot, Y = _selfattn_bf16(X, Wqkv, W2, heads, d, scale, rows)
    return bf16_bits(XDot), bf16_bits(Y)
