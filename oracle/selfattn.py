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
page's column slices are taken in their stated order.
"""

import numpy as np

from .common import rne_fp16
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
