"""Pins of the oracle's bf16 rounding and bf16 MLP chain (CPU)."""

import json
import os

import numpy as np
import pytest

import oracle
from tile_level_sync_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bf16_rounding.json")


def test_bf16_format_facts():
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        v = c.get("value", 1.0)
        got = int(oracle.bf16_bits(oracle.rne_bf16(np.array([v])))[0])
        assert got == int(c["bits"], 16), c


def test_bf16_matches_the_fp32_bit_trick():
    """An independent route for fp32 inputs: add 0x7FFF plus the lowest kept
    bit to the fp32 pattern and keep the upper half (exact for non-NaN fp32,
    subnormals included)."""
    rng = np.random.default_rng(5)
    a = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),   # fp32 subnormals
        (rng.standard_normal(20000) * 3e38).astype(np.float32),    # near the top
        rng.integers(0, 2 ** 32, 50000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    a = a[np.isfinite(a)]
    u = a.view(np.uint32).astype(np.uint64)
    trick = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    got = oracle.bf16_bits(oracle.rne_bf16(a.astype(np.float64)))
    np.testing.assert_array_equal(got, trick)


def test_bf16_rounding_of_doubles_is_not_double_rounded():
    """A float64 just above a bf16 tie whose fp32 rounding lands exactly on
    the tie: rounding via fp32 would go to even (down), direct rounding up."""
    x = 1 + 2 ** -8 + 2 ** -40
    assert np.float32(x) == np.float32(1 + 2 ** -8)
    assert int(oracle.bf16_bits(oracle.rne_bf16(np.array([x])))[0]) == 0x3F81


def test_bf16_roundtrip_and_nan():
    b = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    v = oracle.bf16_values(b)
    finite = np.isfinite(v)
    np.testing.assert_array_equal(oracle.bf16_bits(oracle.rne_bf16(v[finite])), b[finite])
    assert (oracle.bf16_bits(v[np.isnan(v)]) == 0x7FC0).all()


@pytest.mark.parametrize("act", ["erf", "none"])
def test_bf16_chain_brute_force(act):
    Xb, W1b, W2b = inputs.mlp_inputs_bf16(3, 8, 6, seed=2, x_sigma=1.0, w_sigma=0.5)
    G, Zb, Yb = oracle.mlp_chain_bf16(Xb, W1b, W2b, act=act)
    X, W1, W2 = (oracle.bf16_values(b) for b in (Xb, W1b, W2b))
    for i in range(3):
        for j in range(6):
            s = sum(X[i, k] * W1[k, j] for k in range(8))
            g = oracle.gelu_erf(s) if act == "erf" else s
            assert G[i, j] == pytest.approx(g, rel=1e-12, abs=1e-300)
    Z = oracle.bf16_values(Zb)
    for i in range(3):
        for j in range(8):
            y = sum(Z[i, k] * W2[k, j] for k in range(6))
            assert oracle.bf16_values(Yb)[i, j] == oracle.rne_bf16(np.array([y]))[0]


def test_bf16_chain_small_integers_exact_and_identity():
    # identity W2 gives Y = Z; small integers make every product and sum exact
    Xb = oracle.bf16_bits(np.array([[1.0, -2.0, 0.5], [3.0, 0.0, -1.0]]))
    W1b = oracle.bf16_bits(np.array([[1.0, 0.0], [0.0, 1.0], [2.0, -1.0]]))
    W2b = oracle.bf16_bits(np.eye(2))
    G, Zb, Yb = oracle.mlp_chain_bf16(Xb, W1b, W2b, act="none")
    np.testing.assert_array_equal(G, [[2.0, -2.5], [1.0, 1.0]])
    np.testing.assert_array_equal(Yb, Zb)
    np.testing.assert_array_equal(oracle.bf16_values(Zb), G)
