"""Pins for the attention-chain oracle: brute force, uniform and one-hot
softmax, a library softmax.  CPU only."""

import math

import numpy as np
import pytest
from scipy.special import softmax as sp_softmax

import oracle
from tile_level_sync_amd import inputs


def _brute_attn(Q, K, V, scale):
    B, Hh, S, d = Q.shape
    O = np.zeros((B, Hh, S, d), np.float16)
    for b in range(B):
        for h in range(Hh):
            q, k, v = (t[b, h].astype(float).tolist() for t in (Q, K, V))
            for i in range(S):
                row = []
                for j in range(S):
                    a = 0.0
                    for c in range(d):
                        a += q[i][c] * k[j][c]
                    row.append(float(np.float16(scale * a)))
                m = max(row)
                e = [math.exp(x - m) for x in row]
                tot = sum(e)
                for c in range(d):
                    O[b, h, i, c] = np.float16(sum(e[j] / tot * v[j][c] for j in range(S)))
    return O


@pytest.mark.parametrize("scale", [1.0, 0.25])
def test_attn_brute_force(scale):
    Q, K, V = inputs.attn_inputs(2, 2, 6, 4, seed=3)
    _, _, _, O = oracle.attn_chain(Q, K, V, scale)
    Ob = _brute_attn(Q, K, V, scale)
    np.testing.assert_allclose(O.astype(float), Ob.astype(float), rtol=2e-3, atol=2e-4)


def test_softmax_matches_library_and_rows_sum_to_one():
    S = inputs.normal_fp16((7, 33), 5.0, 1, 0).astype(np.float64)
    P = oracle.softmax_rows(S)
    np.testing.assert_allclose(P, sp_softmax(S, axis=-1), rtol=1e-13, atol=0)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-14)


def test_zero_queries_give_column_mean_of_v():
    _, K, V = inputs.attn_inputs(1, 3, 16, 8, seed=2)
    Q = np.zeros_like(K)
    _, _, P, O = oracle.attn_chain(Q, K, V, 1.0)
    np.testing.assert_allclose(P, 1.0 / 16, rtol=0, atol=1e-16)
    exp = oracle.rne_fp16(V.astype(np.float64).mean(axis=2, keepdims=True))
    np.testing.assert_array_equal(O, np.broadcast_to(exp, O.shape))


def test_dominant_key_gives_one_hot():
    S, d = 8, 4
    Q = np.zeros((1, 1, S, d), np.float16)
    K = np.zeros((1, 1, S, d), np.float16)
    V = inputs.normal_fp16((1, 1, S, d), 1.0, 4, 2)
    Q[..., 0] = 1.0
    K[0, 0, 5, 0] = 200.0  # score 200 against 0: softmax is one-hot on key 5
    _, _, P, O = oracle.attn_chain(Q, K, V, 1.0)
    np.testing.assert_array_equal(O[0, 0], np.broadcast_to(V[0, 0, 5], (S, d)))


def test_rows_subset_equals_full():
    Q, K, V = inputs.attn_inputs(2, 3, 32, 8, seed=5)
    _, _, _, O = oracle.attn_chain(Q, K, V, 0.5)
    _, _, _, Or = oracle.attn_chain_rows(Q, K, V, 1, 2, [0, 7, 31], 0.5)
    np.testing.assert_array_equal(Or.view(np.uint16), O[1, 2, [0, 7, 31]].view(np.uint16))
