"""Pins for the MLP-chain oracle: textbook values, IEEE rounding facts,
closed forms and brute force.  CPU only."""

import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import mlp as omlp
from tile_level_sync_amd import inputs


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def test_rne_fp16_ieee_facts(golden_dir):
    g = _golden(golden_dir, "ieee_binary16_rounding.json")
    for case in g["cases"]:
        with np.errstate(over="ignore"):
            h = oracle.rne_fp16(np.array([case["value"]]))
        assert int(h.view(np.uint16)[0]) == int(case["bits"], 16), case


def test_canon_nan_only_touches_nans():
    bits = np.array([0xFFFF, 0x7E00, 0x7C01, 0xFC00, 0x8000, 0x3C00, 0xFE12],
                    dtype=np.uint16)
    out = oracle.canon_nan_fp16(bits.view(np.float16)).view(np.uint16)
    assert list(out) == [0x7E00, 0x7E00, 0x7E00, 0xFC00, 0x8000, 0x3C00, 0x7E00]


def test_gelu_textbook_phi(golden_dir):
    g = _golden(golden_dir, "normal_cdf.json")["phi"]
    for xs, phi in g.items():
        x = float(xs)
        assert omlp.gelu_erf(x) == pytest.approx(x * phi, rel=1e-15, abs=0)
        # GeLU(-x) = -x (1 - Phi(x))
        assert omlp.gelu_erf(-x) == pytest.approx(-x * (1 - phi), rel=1e-13, abs=1e-17)
    assert omlp.gelu_erf(0.0) == 0.0


def test_gelu_odd_identity():
    x = np.linspace(-8, 8, 4001)
    np.testing.assert_allclose(omlp.gelu_erf(x) - omlp.gelu_erf(-x), x, rtol=0, atol=1e-14)
    np.testing.assert_allclose(omlp.gelu_tanh(x) - omlp.gelu_tanh(-x), x, rtol=0, atol=1e-14)


def test_gelu_tanh_close_to_exact():
    # The tanh form approximates x*Phi(x) to a few 1e-4 in absolute terms.
    x = np.linspace(-8, 8, 16001)
    assert np.max(np.abs(omlp.gelu_tanh(x) - omlp.gelu_erf(x))) < 1e-3


def _brute_mlp(X, W1, W2, act):
    """Pure-Python loops: A[i][j] = sum_k X[i][k] W1[k][j] in k order,
    activation with math.erf / math.tanh, fp16 rounding of Z and Y."""
    M, H = X.shape
    F = W1.shape[1]
    H2 = W2.shape[1]
    Xl, W1l, W2l = X.astype(float).tolist(), W1.astype(float).tolist(), W2.astype(float).tolist()
    G = [[0.0] * F for _ in range(M)]
    for i in range(M):
        for j in range(F):
            a = 0.0
            for k in range(H):
                a += Xl[i][k] * W1l[k][j]
            if act == "erf":
                G[i][j] = 0.5 * a * (1.0 + math.erf(a / math.sqrt(2.0)))
            elif act == "tanh":
                c = math.sqrt(2.0 / math.pi)
                G[i][j] = 0.5 * a * (1.0 + math.tanh(c * (a + 0.044715 * a ** 3)))
            else:
                G[i][j] = a
    Z = np.array(G, dtype=np.float64).astype(np.float16)
    Zl = Z.astype(float).tolist()
    Y = [[0.0] * H2 for _ in range(M)]
    for i in range(M):
        for j in range(H2):
            y = 0.0
            for k in range(F):
                y += Zl[i][k] * W2l[k][j]
            Y[i][j] = y
    return np.array(G), Z, np.array(Y).astype(np.float16)


@pytest.mark.parametrize("shape", [(1, 1, 1), (2, 3, 5), (5, 7, 3), (16, 8, 12)])
@pytest.mark.parametrize("act", ["erf", "tanh", "none"])
def test_mlp_brute_force(shape, act):
    M, H, F = shape
    X = inputs.normal_fp16((M, H), 1.0, 7, 0)
    W1 = inputs.normal_fp16((H, F), 0.5, 7, 1)
    W2 = inputs.normal_fp16((F, H), 0.5, 7, 2)
    G, Z, Y = oracle.mlp_chain(X, W1, W2, act=act)
    Gb, Zb, Yb = _brute_mlp(X, W1, W2, act)
    np.testing.assert_allclose(G, Gb, rtol=1e-12, atol=1e-12)
    # rounding order may flip a last bit only at an exact fp16 tie
    assert np.mean(Z.view(np.uint16) == Zb.view(np.uint16)) > 0.99
    np.testing.assert_allclose(Y.astype(float), Yb.astype(float), rtol=2e-3, atol=1e-6)


def test_mlp_exact_small_integers():
    # entries in {-2..2}/16: every product and partial sum is exact, so the
    # pre-activation accumulator equals the exact rational sum.
    M, H, F = 8, 64, 24
    X = inputs.small_int_fp16((M, H), 3, 0)
    W1 = inputs.small_int_fp16((H, F), 3, 1)
    W2 = inputs.small_int_fp16((F, H), 3, 2)
    G, Z, Y = oracle.mlp_chain(X, W1, W2, act="none")
    Xf = [[Fraction(float(v)) for v in row] for row in X]
    W1f = [[Fraction(float(v)) for v in row] for row in W1]
    for i in range(M):
        for j in range(F):
            exact = sum(Xf[i][k] * W1f[k][j] for k in range(H))
            assert G[i, j] == float(exact)


def test_mlp_identity_embedding_gives_elementwise_gelu():
    M, H, F = 16, 32, 48
    X = inputs.normal_fp16((M, H), 1.5, 11, 0)
    W1 = np.zeros((H, F), np.float16)
    W1[np.arange(H), np.arange(H)] = 1.0
    W2 = inputs.normal_fp16((F, H), 0.1, 11, 2)
    G, Z, Y = oracle.mlp_chain(X, W1, W2)
    np.testing.assert_array_equal(Z[:, :H], oracle.rne_fp16(omlp.gelu_erf(X.astype(np.float64))))
    assert np.all(Z[:, H:] == 0)


def test_mlp_identity_w2_gives_y_equal_z():
    M, H = 12, 40
    X = inputs.normal_fp16((M, H), 1.0, 5, 0)
    W1 = inputs.normal_fp16((H, H), 0.3, 5, 1)
    W2 = np.eye(H, dtype=np.float16)
    G, Z, Y = oracle.mlp_chain(X, W1, W2)
    # values equal; a -0.0 in Z becomes +0.0 in Y (it is summed with +0.0 terms)
    np.testing.assert_array_equal(Y.astype(np.float64), Z.astype(np.float64))


def test_mlp_zero_input_gives_zero():
    X = np.zeros((4, 16), np.float16)
    W1 = inputs.normal_fp16((16, 8), 1.0, 1, 1)
    W2 = inputs.normal_fp16((8, 16), 1.0, 1, 2)
    G, Z, Y = oracle.mlp_chain(X, W1, W2)
    assert np.all(Z == 0) and np.all(Y == 0)


def test_mlp_row_independence_and_rows_subset():
    M, H, F = 32, 24, 40
    X, W1, W2 = inputs.mlp_inputs(M, H, F, seed=9)
    _, _, Y = oracle.mlp_chain(X, W1, W2)
    perm = np.random.default_rng(0).permutation(M)
    _, _, Yp = oracle.mlp_chain(X[perm], W1, W2)
    np.testing.assert_array_equal(Yp.view(np.uint16), Y[perm].view(np.uint16))
    rows = [0, 5, 31]
    _, _, Yr = oracle.mlp_chain_rows(X, W1, W2, rows)
    np.testing.assert_array_equal(Yr.view(np.uint16), Y[rows].view(np.uint16))


def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle (on the CPU) and check that the
    brute-force pin rejects each one."""
    X = inputs.normal_fp16((5, 7), 1.0, 2, 0)
    W1 = inputs.normal_fp16((7, 3), 0.5, 2, 1)
    W2 = inputs.normal_fp16((3, 7), 0.5, 2, 2)
    Gb, _, Yb = _brute_mlp(X, W1, W2, "erf")
    mistakes = {
        "dropped half": lambda x: x * (1.0 + omlp.erf(np.asarray(x, float) / np.sqrt(2.0))),
        "wrong sign": lambda x: 0.5 * x * (1.0 - omlp.erf(np.asarray(x, float) / np.sqrt(2.0))),
        "no sqrt2": lambda x: 0.5 * x * (1.0 + omlp.erf(np.asarray(x, float))),
    }
    for name, bad in mistakes.items():
        monkeypatch.setitem(omlp._ACTS, "erf", bad)
        G, _, _ = oracle.mlp_chain(X, W1, W2)
        assert not np.allclose(G, Gb, rtol=1e-6, atol=1e-9), name
    monkeypatch.setitem(omlp._ACTS, "erf", omlp.gelu_erf)
    # transposed second operand (square case so the shapes still fit)
    W2sq = inputs.normal_fp16((7, 7), 0.5, 2, 3)
    W1sq = inputs.normal_fp16((7, 7), 0.5, 2, 4)
    _, _, Yok = oracle.mlp_chain(X, W1sq, W2sq)
    _, _, Ybad = oracle.mlp_chain(X, W1sq, W2sq.T.copy())
    _, _, Ybr = _brute_mlp(X, W1sq, W2sq, "erf")
    np.testing.assert_allclose(Yok.astype(float), Ybr.astype(float), rtol=2e-3, atol=1e-6)
    assert not np.allclose(Ybad.astype(float), Ybr.astype(float), rtol=2e-3, atol=1e-6)
