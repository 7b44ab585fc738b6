"""Pins of the self-attention chain oracle (cuSync paper, Fig. "Architecture
of two building blocks of GPT models" (b), section "Self-Attention",
paragraph StridedSync): brute-force loops, closed forms, an independent
softmax routine and the StridedSync dependency groups."""

import math

import numpy as np
import pytest
import scipy.special

import oracle
from tile_level_sync_amd import inputs


def _f16(a):
    return np.asarray(a, dtype=np.float16)


def _brute(X, Wqkv, W2, heads, d, scale):
    """Explicit loops: every product and sum spelled out."""
    X, Wqkv, W2 = (np.asarray(a, dtype=np.float16).astype(float).tolist() for a in (X, Wqkv, W2))
    M, H, Hs = len(X), len(X[0]), heads * d
    qkv = [[float(np.float16(sum(X[i][k] * Wqkv[k][c] for k in range(H)))) for c in range(3 * Hs)]
           for i in range(M)]
    dot = [[0.0] * Hs for _ in range(M)]
    for h in range(heads):
        for i in range(M):
            s = [scale * sum(qkv[i][h * d + t] * qkv[j][Hs + h * d + t] for t in range(d))
                 for j in range(M)]
            mx = max(s)
            e = [math.exp(v - mx) for v in s]
            z = sum(e)
            for t in range(d):
                dot[i][h * d + t] = float(np.float16(
                    sum(e[j] / z * qkv[j][2 * Hs + h * d + t] for j in range(M))))
    y = [[float(np.float16(sum(dot[i][k] * W2[k][c] for k in range(Hs)))) for c in range(H)]
         for i in range(M)]
    return np.array(qkv), np.array(dot), np.array(y)


@pytest.mark.parametrize("scale", [1.0, 0.5])
def test_brute_force(scale):
    M, H, heads, d = 5, 6, 2, 3
    X = inputs.normal_fp16((M, H), 1.0, 1, 0)
    Wqkv = inputs.normal_fp16((H, 3 * heads * d), 0.5, 1, 1)
    W2 = inputs.normal_fp16((heads * d, H), 0.5, 1, 2)
    q, dot, y = oracle.selfattn_chain(X, Wqkv, W2, heads, d, scale)
    qb, dotb, yb = _brute(X, Wqkv, W2, heads, d, scale)
    np.testing.assert_array_equal(q.astype(float), qb)
    np.testing.assert_allclose(dot.astype(float), dotb, rtol=2e-3, atol=1e-6)
    np.testing.assert_allclose(y.astype(float), yb, rtol=5e-3, atol=1e-4)


def test_identity_projection_matches_library_softmax():
    """Wqkv = [E | E | E] copies the first Hs input columns into each slice,
    so head h attends over X's own columns: compare with scipy's softmax."""
    M, H, heads, d = 7, 8, 2, 4
    Hs = heads * d
    X = inputs.normal_fp16((M, H), 0.5, 2, 0)
    E = np.zeros((H, Hs), np.float16)
    E[np.arange(Hs), np.arange(Hs)] = 1
    Wqkv = np.concatenate([E, E, E], axis=1)
    W2 = np.zeros((Hs, H), np.float16)
    W2[np.arange(Hs), np.arange(Hs)] = 1
    scale = 0.25
    q, dot, y = oracle.selfattn_chain(X, Wqkv, W2, heads, d, scale)
    xs = X[:, :Hs].astype(np.float64)
    for h in range(heads):
        c = slice(h * d, (h + 1) * d)
        ref = scipy.special.softmax(scale * xs[:, c] @ xs[:, c].T, axis=1) @ xs[:, c]
        np.testing.assert_allclose(dot[:, c].astype(float), ref, rtol=2e-3, atol=1e-4)
    np.testing.assert_array_equal(y[:, :Hs], dot)   # W2 = identity on the first Hs columns
    assert not np.any(y[:, Hs:])


def test_zero_queries_give_token_mean():
    M, H, heads, d = 9, 8, 2, 4
    Hs = heads * d
    X = inputs.normal_fp16((M, H), 1.0, 3, 0)
    Wqkv = inputs.normal_fp16((H, 3 * Hs), 0.5, 3, 1)
    Wqkv[:, :Hs] = 0
    W2 = inputs.normal_fp16((Hs, H), 0.5, 3, 2)
    q, dot, _ = oracle.selfattn_chain(X, Wqkv, W2, heads, d, 1.0)
    mean = q[:, 2 * Hs:].astype(np.float64).mean(axis=0)
    np.testing.assert_allclose(dot.astype(float), np.broadcast_to(mean, dot.shape), rtol=2e-3,
                               atol=1e-5)


def test_head_permutation_equivariance():
    M, H, heads, d = 6, 8, 3, 2
    Hs = heads * d
    X = inputs.normal_fp16((M, H), 1.0, 4, 0)
    Wqkv = inputs.normal_fp16((H, 3 * Hs), 0.5, 4, 1)
    W2 = inputs.normal_fp16((Hs, H), 0.5, 4, 2)
    perm = [2, 0, 1]
    cols = np.concatenate([np.arange(p * d, (p + 1) * d) for p in perm])
    Wp = np.concatenate([Wqkv[:, k * Hs:(k + 1) * Hs][:, cols] for k in range(3)], axis=1)
    _, dot, y = oracle.selfattn_chain(X, Wqkv, W2, heads, d, 0.7)
    _, dotp, yp = oracle.selfattn_chain(X, Wp, W2[cols], heads, d, 0.7)
    np.testing.assert_array_equal(dotp, dot[:, cols])
    np.testing.assert_allclose(yp.astype(float), y.astype(float), rtol=2e-3, atol=1e-4)


def test_rows_subset_equals_full():
    M, H, heads, d = 11, 8, 2, 4
    X = inputs.normal_fp16((M, H), 1.0, 5, 0)
    Wqkv = inputs.normal_fp16((H, 3 * heads * d), 0.5, 5, 1)
    W2 = inputs.normal_fp16((heads * d, H), 0.5, 5, 2)
    qkv, dot, y = oracle.selfattn_chain(X, Wqkv, W2, heads, d, 0.3)
    rows = [0, 4, 10]
    dr, yr = oracle.selfattn_rows(X, Wqkv, W2, heads, d, 0.3, rows)
    np.testing.assert_array_equal(dr, dot[rows])
    np.testing.assert_array_equal(yr, y[rows])
    q, dr2, yr2 = oracle.selfattn_rows(X, Wqkv, W2, heads, d, 0.3, rows, return_qkv=True)
    np.testing.assert_array_equal(q, qkv)
    np.testing.assert_array_equal(dr2, dr)
    np.testing.assert_array_equal(yr2, yr)


@pytest.mark.parametrize("bn1", [2, 4])
def test_stage2_deps_are_the_strided_groups(bn1):
    """With column tiles no wider than a head, the XQKV column tiles stage-2
    item (r, h) reads are exactly the StridedSync group of head h's tiles,
    over every row tile for the two non-query slices."""
    M, heads, d, BM = 10, 3, 4, 4
    Hs = heads * d
    stride = Hs // bn1
    for r in range(3):
        for h in range(heads):
            deps = oracle.selfattn_stage2_deps(r, h, M, Hs, d, BM, bn1)
            cols = {c for _, c in deps}
            expect = set()
            for sub in range(d // bn1):
                expect |= oracle.strided_group(h * (d // bn1) + sub, stride)
            assert cols == expect
            mt = (M + BM - 1) // BM
            for c in cols:
                rows = {i for i, cc in deps if cc == c}
                assert rows == ({r} if c < stride else set(range(mt)))
