"""Pins for the brute-force dependency sets: the cuSync paper's worked
example and hand-derived halo cases.  CPU only."""

import json
import os

import oracle


def test_toy_example_matches_paper(golden_dir):
    with open(os.path.join(golden_dir, "paper_toy_example.json")) as f:
        g = json.load(f)
    deps = oracle.toy_example_deps()
    for key, want in g["consumer_deps"].items():
        i, j = map(int, key.split(","))
        assert deps[(i, j)] == {tuple(t) for t in want}


def test_mlp_deps_are_whole_producer_row():
    for (M, H, F, BM, BN1, BN2) in [(8, 12, 16, 4, 4, 6), (6, 5, 9, 2, 3, 5)]:
        for i in range(-(-M // BM)):
            for j in range(-(-H // BN2)):
                got = oracle.mlp_consumer_deps(i, j, M, H, F, BM, BN1, BN2)
                assert got == {(i, c) for c in range(-(-F // BN1))}


def test_conv_deps_hand_cases():
    # 1 image 8x8 (64 pixels), tiles of 16 pixels (two image rows).
    # Tile 0 (rows 0-1) reads rows 0-2 -> producer tiles 0,1.
    # Tile 1 (rows 2-3) reads rows 1-4 -> tiles 0,1,2.
    # Tile 3 (rows 6-7) reads rows 5-7 -> tiles 2,3.
    d = lambda i: oracle.conv_consumer_deps(i, 1, 8, 8, 4, 16, 4)
    assert d(0) == {(0, 0), (1, 0)}
    assert d(1) == {(0, 0), (1, 0), (2, 0)}
    assert d(3) == {(2, 0), (3, 0)}
    # two output-channel tiles in the producer: every channel tile is needed
    d2 = oracle.conv_consumer_deps(1, 1, 8, 8, 8, 16, 4)
    assert d2 == {(t, c) for t in (0, 1, 2) for c in (0, 1)}


def test_conv_deps_tile_smaller_than_halo():
    # tile of 4 pixels on an 8-wide image: the 1-pixel halo spans 9 flat pixels,
    # so a middle tile needs producer tiles two away.
    d = oracle.conv_consumer_deps(4, 1, 8, 8, 2, 4, 2)  # pixels 16..19 = row 2, cols 0-3
    assert d == {(t, 0) for t in (2, 3, 4, 5, 6, 7)}


def test_attn_deps_whole_score_row():
    assert oracle.attn_consumer_deps(1, 8, 2, 4) == {(1, 0), (1, 1)}
