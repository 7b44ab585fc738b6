"""Pins for the conv-pair oracle: brute force, a library 2-D correlation,
delta and shifted-delta filters.  CPU only."""

import numpy as np
import pytest
from scipy.signal import correlate2d

import oracle
from tile_level_sync_amd import inputs


def _brute_conv(X, W, pad, stride):
    N, H, Wd, C = X.shape
    R, S, _, K = W.shape
    P = (H + 2 * pad - R) // stride + 1
    Q = (Wd + 2 * pad - S) // stride + 1
    Xl = X.astype(float)
    Wl = W.astype(float)
    out = np.zeros((N, P, Q, K))
    for n in range(N):
        for p in range(P):
            for q in range(Q):
                for k in range(K):
                    acc = 0.0
                    for r in range(R):
                        for s in range(S):
                            y, x = p * stride + r - pad, q * stride + s - pad
                            if 0 <= y < H and 0 <= x < Wd:
                                for c in range(C):
                                    acc += Xl[n, y, x, c] * Wl[r, s, c, k]
                    out[n, p, q, k] = acc
    return out


@pytest.mark.parametrize("pad,stride", [(1, 1), (0, 1), (1, 2), (2, 1)])
def test_conv_brute_force(pad, stride):
    X = inputs.normal_fp16((2, 6, 5, 3), 1.0, 4, 0)
    W = inputs.normal_fp16((3, 3, 3, 4), 0.5, 4, 1)
    np.testing.assert_allclose(oracle.conv2d_nhwc(X, W, pad, stride),
                               _brute_conv(X, W, pad, stride), rtol=1e-12, atol=1e-12)


def test_conv_single_channel_matches_library_correlation():
    X = inputs.normal_fp16((1, 9, 7, 1), 1.0, 8, 0)
    W = inputs.normal_fp16((3, 3, 1, 1), 1.0, 8, 1)
    ref = correlate2d(X[0, :, :, 0].astype(float), W[:, :, 0, 0].astype(float),
                      mode="same", boundary="fill", fillvalue=0)
    np.testing.assert_allclose(oracle.conv2d_nhwc(X, W)[0, :, :, 0], ref, rtol=1e-12, atol=1e-12)


def test_delta_filter_is_identity_and_chain_gives_relu():
    C = 8
    X = inputs.normal_fp16((2, 7, 7, C), 1.0, 5, 0)
    D = np.zeros((3, 3, C, C), np.float16)
    D[1, 1] = np.eye(C, dtype=np.float16)
    np.testing.assert_array_equal(oracle.conv2d_nhwc(X, D), X.astype(np.float64))
    G, Z, Y = oracle.conv_chain(X, D, D)
    relu = np.where(X < 0, np.float16(0), X)
    np.testing.assert_array_equal(Z.astype(np.float64), relu.astype(np.float64))
    np.testing.assert_array_equal(Y.astype(np.float64), relu.astype(np.float64))


@pytest.mark.parametrize("r,s", [(0, 0), (0, 2), (2, 1), (1, 0)])
def test_shifted_delta_pins_halo_and_padding(r, s):
    C = 4
    X = inputs.normal_fp16((1, 6, 5, C), 1.0, 6, 0)
    D = np.zeros((3, 3, C, C), np.float16)
    D[r, s] = np.eye(C, dtype=np.float16)
    out = oracle.conv2d_nhwc(X, D)
    # out[p, q] = X[p + r - 1, q + s - 1] inside the image, 0 outside
    exp = np.zeros_like(out)
    for p in range(6):
        for q in range(5):
            y, x = p + r - 1, q + s - 1
            if 0 <= y < 6 and 0 <= x < 5:
                exp[0, p, q] = X[0, y, x]
    np.testing.assert_array_equal(out, exp)


def test_conv_exact_small_integers():
    X = inputs.small_int_fp16((1, 5, 5, 16), 2, 0)
    W = inputs.small_int_fp16((3, 3, 16, 8), 2, 1)
    a = oracle.conv2d_nhwc(X, W)
    b = _brute_conv(X, W, 1, 1)
    np.testing.assert_array_equal(a, b)  # all sums exact
