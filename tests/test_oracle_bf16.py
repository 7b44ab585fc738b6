"""Pins of the oracle's bf16 rounding and bf16 MLP chain (CPU)."""

import json
import math
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


# Values past the fp32 range overflow to infinity on purpose (the top binade).
@pytest.mark.filterwarnings("ignore:overflow encountered in cast")
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


# Every 16-bit pattern round-trips, NaN payloads included.
@pytest.mark.filterwarnings("ignore:invalid value encountered in cast")
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


def _conv_brute(X, W, pad=1):
    """out[n,p,q,k] = sum over taps inside the image of X[n,p+r-pad,q+s-pad,c] W[r,s,c,k],
    by explicit loops (no padding array, no matmul)."""
    N, H, Wd, C = X.shape
    R, S, _, K = W.shape
    out = np.zeros((N, H, Wd, K))
    for n in range(N):
        for p in range(H):
            for q in range(Wd):
                for k in range(K):
                    acc = 0.0
                    for r in range(R):
                        for s in range(S):
                            y, x = p + r - pad, q + s - pad
                            if 0 <= y < H and 0 <= x < Wd:
                                for c in range(C):
                                    acc += X[n, y, x, c] * W[r, s, c, k]
                    out[n, p, q, k] = acc
    return out


def test_bf16_conv_chain_brute_force():
    Xb, Wab, Wbb = inputs.conv_inputs_bf16(1, 4, 5, 3, 2, seed=3, x_sigma=1.0, w_sigma=0.5)
    G, Zb, Yb = oracle.conv_chain_bf16(Xb, Wab, Wbb)
    X, Wa, Wb = (oracle.bf16_values(b) for b in (Xb, Wab, Wbb))
    A = _conv_brute(X, Wa)
    np.testing.assert_allclose(G, np.maximum(A, 0.0), rtol=1e-12, atol=1e-300)
    assert (G == 0.0).any() and (G > 0.0).any()  # ReLU active on both sides
    np.testing.assert_array_equal(Zb, oracle.bf16_bits(oracle.rne_bf16(G)))
    Yr = oracle.rne_bf16(_conv_brute(oracle.bf16_values(Zb), Wb))
    np.testing.assert_array_equal(oracle.bf16_values(Yb), Yr)


def test_bf16_conv_chain_rounds_each_store_to_nearest_even():
    # one row of two pixels, one channel: the first output pixel sums 256 (centre tap)
    # and 1 (right neighbour) = 257, a tie between the bf16 values 256 and 258 that
    # rounds to the even 256; the second pixel has no right neighbour: 256
    Xb = oracle.bf16_bits(np.ones((1, 1, 2, 1)))
    Wa = np.zeros((3, 3, 1, 1))
    Wa[1, 1, 0, 0], Wa[1, 2, 0, 0] = 256.0, 1.0
    Wb = np.zeros((3, 3, 1, 1))
    Wb[1, 1, 0, 0] = 1.0
    G, Zb, Yb = oracle.conv_chain_bf16(Xb, oracle.bf16_bits(Wa), oracle.bf16_bits(Wb))
    np.testing.assert_array_equal(G.ravel(), [257.0, 256.0])
    np.testing.assert_array_equal(oracle.bf16_values(Zb).ravel(), [256.0, 256.0])
    np.testing.assert_array_equal(Yb, Zb)
    # the fp16 chain keeps 257 (11 significant bits)
    _, Z16, _ = oracle.conv_chain(oracle.bf16_values(Xb).astype(np.float16),
                                  Wa.astype(np.float16), Wb.astype(np.float16))
    assert Z16.ravel()[0] == 257.0


def test_bf16_conv_chain_matches_fp16_chain_on_small_integers():
    rng = np.random.default_rng(5)
    X = rng.integers(-1, 2, size=(2, 5, 4, 3)).astype(np.float64)
    Wa = rng.integers(-1, 2, size=(3, 3, 3, 4)).astype(np.float64)
    Wb = rng.integers(-1, 2, size=(3, 3, 4, 4)).astype(np.float64)
    # |Z| <= 27 and |Y| <= 9 * 4 * 27 = 972 < 2^10: every value below is exact in fp16,
    # and the bf16 chain agrees wherever the fp16 result needs at most 8 significant bits
    G, Zb, Yb = oracle.conv_chain_bf16(*(oracle.bf16_bits(a) for a in (X, Wa, Wb)))
    G16, Z16, Y16 = oracle.conv_chain(X.astype(np.float16), Wa.astype(np.float16),
                                      Wb.astype(np.float16))
    np.testing.assert_array_equal(G, G16)
    np.testing.assert_array_equal(oracle.bf16_values(Zb), Z16.astype(np.float64))
    y16 = Y16.astype(np.float64)
    exact8 = np.abs(y16) <= 256
    np.testing.assert_array_equal(oracle.bf16_values(Yb)[exact8], y16[exact8])
    np.testing.assert_array_equal(oracle.bf16_values(Yb), oracle.rne_bf16(y16))


def test_bf16_attn_chain_brute_force():
    Qb, Kb, Vb = inputs.attn_inputs_bf16(1, 2, 5, 4, seed=4)
    scale = 0.5
    A, Scb, P, Ob = oracle.attn_chain_bf16(Qb, Kb, Vb, scale)
    Q, K, V = (oracle.bf16_values(b) for b in (Qb, Kb, Vb))
    for h in range(2):
        for i in range(5):
            a = [scale * sum(Q[0, h, i, c] * K[0, h, j, c] for c in range(4)) for j in range(5)]
            np.testing.assert_allclose(A[0, h, i], a, rtol=1e-12, atol=1e-300)
            sc = oracle.rne_bf16(np.array(a))
            np.testing.assert_array_equal(oracle.bf16_values(Scb[0, h, i]), sc)
            e = [math.exp(x - max(sc)) for x in sc]
            p = [x / sum(e) for x in e]
            np.testing.assert_allclose(P[0, h, i], p, rtol=1e-12)
            o = [sum(p[j] * V[0, h, j, c] for j in range(5)) for c in range(4)]
            np.testing.assert_array_equal(oracle.bf16_values(Ob[0, h, i]),
                                          oracle.rne_bf16(np.array(o)))


def test_bf16_attn_chain_closed_forms():
    # equal scores give the uniform average of V; one dominant score picks its V row
    S, d = 4, 2
    Q = np.zeros((1, 1, S, d)); K = np.zeros((1, 1, S, d))
    V = np.arange(S * d, dtype=np.float64).reshape(1, 1, S, d)
    _, Scb, P, Ob = oracle.attn_chain_bf16(*(oracle.bf16_bits(x) for x in (Q, K, V)))
    np.testing.assert_allclose(P, 0.25)
    np.testing.assert_array_equal(oracle.bf16_values(Ob)[0, 0],
                                  np.tile(V[0, 0].mean(axis=0), (S, 1)))
    Q[0, 0, :, 0] = 1.0
    K[0, 0, 2, 0] = 100.0  # score 100 for key 2, 0 for the others: P ~ e_2
    _, _, P, Ob = oracle.attn_chain_bf16(*(oracle.bf16_bits(x) for x in (Q, K, V)))
    np.testing.assert_allclose(P[0, 0, :, 2], 1.0, rtol=1e-12)
    np.testing.assert_array_equal(oracle.bf16_values(Ob)[0, 0], np.tile(V[0, 0, 2], (S, 1)))
    # a row subset equals the full chain at those rows
    Qb, Kb, Vb = inputs.attn_inputs_bf16(2, 2, 8, 4, seed=6)
    full = oracle.attn_chain_bf16(Qb, Kb, Vb, 0.7)
    part = oracle.attn_chain_bf16_rows(Qb, Kb, Vb, 1, 0, [6, 1], 0.7)
    for f, q in zip(full, part):
        np.testing.assert_array_equal(f[1, 0, [6, 1]], q)


@pytest.mark.parametrize("scale", [1.0, 0.35])
def test_bf16_selfattn_chain_brute_force(scale):
    M, H, heads, d = 5, 4, 2, 2
    Hs = heads * d
    Xb, Wqb, W2b = inputs.selfattn_inputs_bf16(M, H, heads, d, seed=8, w_sigma=0.5)
    Qb, Db, Yb = oracle.selfattn_chain_bf16(Xb, Wqb, W2b, heads, d, scale)
    X, Wq, W2 = (oracle.bf16_values(b) for b in (Xb, Wqb, W2b))
    rb = lambda x: float(oracle.rne_bf16(np.array([x]))[0])
    qkv = [[rb(sum(X[i, k] * Wq[k, j] for k in range(H))) for j in range(3 * Hs)]
           for i in range(M)]
    np.testing.assert_array_equal(oracle.bf16_values(Qb), np.array(qkv))
    dot = [[0.0] * Hs for _ in range(M)]
    for h in range(heads):
        for i in range(M):
            a = [scale * sum(qkv[i][h * d + c] * qkv[j][Hs + h * d + c] for c in range(d))
                 for j in range(M)]
            e = [math.exp(x - max(a)) for x in a]
            p = [x / sum(e) for x in e]
            for c in range(d):
                dot[i][h * d + c] = rb(sum(p[j] * qkv[j][2 * Hs + h * d + c] for j in range(M)))
    np.testing.assert_array_equal(oracle.bf16_values(Db), np.array(dot))
    y = [[rb(sum(dot[i][c] * W2[c, j] for c in range(Hs))) for j in range(H)] for i in range(M)]
    np.testing.assert_array_equal(oracle.bf16_values(Yb), np.array(y))


def test_bf16_selfattn_chain_closed_forms():
    M, H, heads, d = 8, 4, 2, 2
    Hs = heads * d
    Xb, Wqb, W2b = inputs.selfattn_inputs_bf16(M, H, heads, d, seed=9, w_sigma=0.5)
    # a zero query slice gives every token the mean of its head's third slice
    # (M = 8: the weights 1/8 and the sums are exact)
    Wq0 = Wqb.copy()
    Wq0[:, :Hs] = 0
    Qb, Db, _ = oracle.selfattn_chain_bf16(Xb, Wq0, W2b, heads, d, 1.0)
    s3 = oracle.bf16_values(Qb)[:, 2 * Hs:]
    np.testing.assert_array_equal(oracle.bf16_values(Db),
                                  np.tile(oracle.rne_bf16(s3.sum(axis=0) / 8.0), (M, 1)))
    # the first store rounds to nearest even: 256 + 1 = 257 is a tie -> 256
    X = np.zeros((M, H)); X[:, 0] = 256.0; X[:, 1] = 1.0
    W = np.zeros((H, 3 * Hs)); W[0, :] = 1.0; W[1, :] = 1.0
    Qb, _, _ = oracle.selfattn_chain_bf16(oracle.bf16_bits(X), oracle.bf16_bits(W), W2b,
                                          heads, d, 1.0)
    np.testing.assert_array_equal(oracle.bf16_values(Qb), 256.0)
    # permuting the heads permutes XDot's columns and leaves Y
    perm = [1, 0]
    cols = np.concatenate([np.arange(p * d, (p + 1) * d) for p in perm])
    Wp = np.concatenate([Wqb[:, k * Hs:(k + 1) * Hs][:, cols] for k in range(3)], axis=1)
    _, Db, Yb = oracle.selfattn_chain_bf16(Xb, Wqb, W2b, heads, d, 0.6)
    _, Dp, Yp = oracle.selfattn_chain_bf16(Xb, Wp, W2b[cols], heads, d, 0.6)
    np.testing.assert_array_equal(Dp, Db[:, cols])
    np.testing.assert_allclose(oracle.bf16_values(Yp), oracle.bf16_values(Yb), rtol=2.0 ** -7)
    # the rows variant equals the full chain at those rows
    Dr, Yr = oracle.selfattn_rows_bf16(Xb, Wqb, W2b, heads, d, 0.6, [7, 2])
    np.testing.assert_array_equal(Dr, Db[[7, 2]])
    np.testing.assert_array_equal(Yr, Yb[[7, 2]])
