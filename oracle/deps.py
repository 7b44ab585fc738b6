"""Brute-force tile dependency sets (test infrastructure only).

For a consumer tile, enumerate every output element it computes, every
intermediate element that element reads, and the producer tile that writes
it.  The result is the exact set a sync policy must wait for.  It pins the
closed-form ranges the library uses for TileSync / RowSync (cuSync paper,
section "Synchronization Policies": a consumer GeMM tile depends on the whole
row of producer tiles) and for the halo-aware reading of Conv2DTileSync (the
page maps output tile [i, j] to a single input tile, which ignores the 3x3
halo; the reading kept here is the exact read set).

Pure Python loops: meant for small shapes only.
"""


def mlp_consumer_deps(i, j, M, H, F, BM, BN1, BN2):
    """Producer tiles (row, col) of Z[M,F] read by consumer tile (i, j) of
    Y = Z W2 with Y:[M,H], tiles BM x BN1 (producer) and BM x BN2 (consumer)."""
    deps = set()
    for r in range(i * BM, min((i + 1) * BM, M)):
        for c in range(j * BN2, min((j + 1) * BN2, H)):
            for f in range(F):  # Y[r, c] = sum_f Z[r, f] W2[f, c]
                deps.add((r // BM, f // BN1))
    return deps


def conv_consumer_deps(i, N, Hh, Ww, C, BM, BN1, R=3, S=3, pad=1, stride=1):
    """Producer tiles (m-tile, channel-tile) of the intermediate Z read by the
    consumer tile of output pixels [i*BM, (i+1)*BM) (flattened n, p, q).

    Z is NHWC [N, Hh, Ww, C] produced in tiles of BM flattened pixels x BN1
    channels; the consumer convolution reads every channel of every in-bounds
    input pixel of its R x S window (zero padding reads nothing)."""
    P = (Hh + 2 * pad - R) // stride + 1
    Q = (Ww + 2 * pad - S) // stride + 1
    npix_out = N * P * Q
    deps = set()
    for m in range(i * BM, min((i + 1) * BM, npix_out)):
        n, rem = divmod(m, P * Q)
        p, q = divmod(rem, Q)
        for r in range(R):
            for s in range(S):
                y = p * stride + r - pad
                x = q * stride + s - pad
                if 0 <= y < Hh and 0 <= x < Ww:
                    src = (n * Hh + y) * Ww + x
                    for c in range(C):
                        deps.add((src // BM, c // BN1))
    return deps


def attn_consumer_deps(ti, S, BM, BN):
    """Producer score tiles (ti', tj) of one (batch, head) read by the consumer
    row block ti: the softmax of a row needs every score in the row."""
    deps = set()
    for r in range(ti * BM, min((ti + 1) * BM, S)):
        for c in range(S):
            deps.add((r // BM, c // BN))
    return deps


def toy_example_deps():
    """The cuSync paper's motivating example (section "Motivation"):
    C[12,8] = A[12,8] B[8,8] and E[12,8] = C D with 4x4 tiles.  Returns
    {consumer tile (i, j): set of producer tiles} for all six E tiles."""
    return {(i, j): mlp_consumer_deps(i, j, M=12, H=8, F=8, BM=4, BN1=4, BN2=4)
            for i in range(3) for j in range(2)}


def selfattn_stage2_deps(r, h, M, Hs, d, BM, BN1):
    """Tiles (row tile, column tile) of XQKV [M, 3 Hs] (tiles BM x BN1) read by
    the stage-2 item of token rows [r*BM, (r+1)*BM) and head h: its query rows
    in the first slice, and every row of head h's columns in the other two."""
    deps = set()
    for i in range(r * BM, min((r + 1) * BM, M)):
        for c in range(h * d, (h + 1) * d):
            deps.add((i // BM, c // BN1))                      # query slice, own rows
            for j in range(M):                                  # scores need every token
                deps.add((j // BM, (Hs + c) // BN1))
                deps.add((j // BM, (2 * Hs + c) // BN1))
    return deps


def strided_group(col, stride):
    """The producer column tiles that share one StridedSync semaphore with
    column tile ``col`` (cuSync paper, paragraph StridedSync: tiles ``stride``
    apart share a semaphore): {col mod stride + k * stride, k = 0, 1, 2}."""
    base = col % stride
    return {base, base + stride, base + 2 * stride}
