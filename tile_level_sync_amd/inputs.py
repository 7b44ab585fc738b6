"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module holds no arithmetic of the chains: it only draws random tensors.
Each tensor comes from its own PCG64 stream, ``SeedSequence(seed,
spawn_key=(stream,))``, so the weights of a workload do not depend on its
batch size and the draw order does not matter.  Values are float32 normal
draws times sigma, rounded to fp16 (nearest-even).

Workload shapes (the pages' GPT-3 MLP slice, its attention heads and the
ResNet-38 56x56x64 conv layer) are exposed as functions below; no dataset or
trained weight is involved anywhere.
"""

import numpy as np

# stream ids: first operand, then the two weights
_STREAM = {"X": 0, "W1": 1, "W2": 2, "Wa": 1, "Wb": 2, "Q": 0, "K": 1, "V": 2, "Wqkv": 1}


def _rng(seed, stream):
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(stream,))))


def normal_fp16(shape, sigma, seed, stream):
    """N(0, sigma^2) draws rounded to fp16."""
    g = _rng(seed, stream)
    a = g.standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(sigma)
    return a.astype(np.float16)


def small_int_fp16(shape, seed, stream, lo=-2, hi=2, scale=2.0 ** -4):
    """Integers in [lo, hi] times a power of two, as fp16.  Products and sums
    of such values stay exact in fp32 for the sizes the tests use."""
    g = _rng(seed, stream)
    a = g.integers(lo, hi + 1, size=shape).astype(np.float32) * np.float32(scale)
    return a.astype(np.float16)


# --- MLP chain: X[M,H] . W1[H,F] -> GeLU -> . W2[F,H] -------------------------

GPT3_H = 12288          # GPT-3 hidden size
GPT3_F = 6144           # one GPU's share of the 4H MLP width under 8-way sharding
GPT3_MS = (256, 512, 1024, 2048)


def mlp_inputs(M, H, F, seed=0, x_sigma=1.0, w_sigma=0.02):
    X = normal_fp16((M, H), x_sigma, seed, _STREAM["X"])
    W1 = normal_fp16((H, F), w_sigma, seed, _STREAM["W1"])
    W2 = normal_fp16((F, H), w_sigma, seed, _STREAM["W2"])
    return X, W1, W2


def mlp_weights(H, F, seed=0, w_sigma=0.02):
    return (normal_fp16((H, F), w_sigma, seed, _STREAM["W1"]),
            normal_fp16((F, H), w_sigma, seed, _STREAM["W2"]))


def normal_bf16_bits(shape, sigma, seed, stream):
    """N(0, sigma^2) draws (float32, as normal_fp16 draws them) rounded to bf16,
    nearest-even on the fp32 bit pattern; returned as uint16 bit patterns."""
    a = _rng(seed, stream).standard_normal(size=shape, dtype=np.float32)
    a *= np.float32(sigma)
    u = a.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def mlp_inputs_bf16(M, H, F, seed=0, x_sigma=1.0, w_sigma=0.02):
    """The MLP chain's inputs in bf16 (uint16 bit patterns), same streams as
    mlp_inputs."""
    return (normal_bf16_bits((M, H), x_sigma, seed, _STREAM["X"]),
            normal_bf16_bits((H, F), w_sigma, seed, _STREAM["W1"]),
            normal_bf16_bits((F, H), w_sigma, seed, _STREAM["W2"]))


def mlp_x(M, H, seed=0, x_sigma=1.0):
    return normal_fp16((M, H), x_sigma, seed, _STREAM["X"])


def tiny_mlp_inputs(seed=0):
    """X[64x256], W1[256x1024], W2[1024x256], all N(0, 0.02)."""
    return mlp_inputs(64, 256, 1024, seed=seed, x_sigma=0.02, w_sigma=0.02)


# --- conv pair: NHWC activations, RSCK filters --------------------------------

def conv_inputs(N, Hh, Ww, C, K, R=3, S=3, seed=0, x_sigma=1.0, w_sigma=0.02):
    X = normal_fp16((N, Hh, Ww, C), x_sigma, seed, _STREAM["X"])
    Wa = normal_fp16((R, S, C, K), w_sigma, seed, _STREAM["Wa"])
    Wb = normal_fp16((R, S, K, K), w_sigma, seed, _STREAM["Wb"])
    return X, Wa, Wb


def conv_inputs_bf16(N, Hh, Ww, C, K, R=3, S=3, seed=0, x_sigma=1.0, w_sigma=0.02):
    """The conv pair's inputs in bf16 (uint16 bit patterns), same streams as
    conv_inputs."""
    return (normal_bf16_bits((N, Hh, Ww, C), x_sigma, seed, _STREAM["X"]),
            normal_bf16_bits((R, S, C, K), w_sigma, seed, _STREAM["Wa"]),
            normal_bf16_bits((R, S, K, K), w_sigma, seed, _STREAM["Wb"]))


# The dependent 3x3 conv pairs of ResNet-38 (cuSync paper, section "ResNet"
# and its table of conv layers): (image side, channels).
RESNET38_PAIRS = ((56, 64), (28, 128), (14, 256), (7, 512))


def resnet_pair_inputs(batch=32, seed=0, side=56, channels=64):
    """A ResNet-38 layer pair: side x side images, channels -> channels ->
    channels (default the first pair, 56x56, 64 channels)."""
    return conv_inputs(batch, side, side, channels, channels, seed=seed)


# --- attention chain: [B, heads, S, d] ----------------------------------------

def attn_inputs(B, heads, S, d, seed=0, sigma=1.0):
    return tuple(normal_fp16((B, heads, S, d), sigma, seed, _STREAM[n])
                 for n in ("Q", "K", "V"))


def attn_inputs_bf16(B, heads, S, d, seed=0, sigma=1.0):
    """The attention chain's inputs in bf16 (uint16 bit patterns), same
    streams as attn_inputs."""
    return tuple(normal_bf16_bits((B, heads, S, d), sigma, seed, _STREAM[n])
                 for n in ("Q", "K", "V"))


# --- self-attention block: X [M, H], Wqkv [H, 3 heads d], W2 [heads d, H] ---
# One GPU's share of GPT-3's 8-way model-parallel layer: H = 12288, 12 heads
# of 128 (cuSync paper, Fig. "Architecture of two building blocks of GPT
# models" (b): QKV [H, 3H/8], W2 [H/8, H]).
GPT3_SA_HEADS = 12


def selfattn_inputs(M, H, heads, d=128, seed=0, x_sigma=1.0, w_sigma=0.02):
    X = normal_fp16((M, H), x_sigma, seed, _STREAM["X"])
    Wqkv = normal_fp16((H, 3 * heads * d), w_sigma, seed, _STREAM["Wqkv"])
    W2 = normal_fp16((heads * d, H), w_sigma, seed, _STREAM["W2"])
    return X, Wqkv, W2


def selfattn_inputs_bf16(M, H, heads, d=128, seed=0, x_sigma=1.0, w_sigma=0.02):
    """The self-attention block's inputs in bf16 (uint16 bit patterns), same
    streams as selfattn_inputs."""
    return (normal_bf16_bits((M, H), x_sigma, seed, _STREAM["X"]),
            normal_bf16_bits((H, 3 * heads * d), w_sigma, seed, _STREAM["Wqkv"]),
            normal_bf16_bits((heads * d, H), w_sigma, seed, _STREAM["W2"]))
