"""Host-side library logic (no GPU): exported symbols, planning helpers and
the Conv2DTileSync halo range, against the pages' numbers and the oracle's
brute-force dependency sets."""

import ctypes
import json
import os
import shutil
import subprocess
import re

import numpy as np
import pytest
from fractions import Fraction

import oracle
import tile_level_sync_amd as tls

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    src = open(os.path.join(ROOT, "include", "tlsync.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(chain_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = tls.load()
    names = _header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(lib, n), n
        assert n in tls.SIGNATURES, n


def test_struct_layouts_match_c(tmp_path):
    """Compile a C probe against the header and compare sizeof/offsetof with
    the ctypes mirrors."""
    probe = tmp_path / "probe.c"
    fields = {
        "chain_mlp_args": [f for f, _ in tls.chain_mlp_args._fields_],
        "chain_conv_args": [f for f, _ in tls.chain_conv_args._fields_],
        "chain_attn_args": [f for f, _ in tls.chain_attn_args._fields_],
        "chain_selfattn_args": [f for f, _ in tls.chain_selfattn_args._fields_],
        "chain_tile_info": [f for f, _ in tls.chain_tile_info._fields_],
        "chain_plan": [f for f, _ in tls.chain_plan._fields_],
        "chain_selfattn_plan_info": [f for f, _ in tls.chain_selfattn_plan_info._fields_],
        "chain_trace_rec": [f for f, _ in tls.chain_trace_rec._fields_],
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "tlsync.h"', "int main(void){"]
    for st, fs in fields.items():
        lines.append('printf("%s %%zu\\n", sizeof(%s));' % (st, st))
        for f in fs:
            lines.append('printf("%s.%s %%zu\\n", offsetof(%s, %s));' % (st, f, st, f))
    lines.append("return 0;}")
    probe.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    r = subprocess.run(["gcc", "-I" + os.path.join(ROOT, "include"), str(probe), "-o", str(exe)],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout
    out = os.popen(str(exe)).read().split("\n")
    got = dict(l.rsplit(" ", 1) for l in out if l)
    for st, fs in fields.items():
        cls = getattr(tls, st)
        assert int(got[st]) == ctypes.sizeof(cls), st
        for f in fs:
            assert int(got["%s.%s" % (st, f)]) == getattr(cls, f).offset, (st, f)


def test_strerror_and_argument_errors_without_gpu():
    lib = tls.load()
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.chain_strerror(code)
    a = tls.chain_mlp_args()  # all null: rejected before any device call
    assert lib.chain_mlp_ex(ctypes.byref(a)) == tls.CHAIN_EINVAL
    c = tls.chain_conv_args()
    assert lib.chain_conv_ex(ctypes.byref(c)) == tls.CHAIN_EINVAL
    at = tls.chain_attn_args()
    assert lib.chain_attn_ex(ctypes.byref(at)) == tls.CHAIN_EINVAL
    assert lib.chain_mlp_workspace_bytes(64, 200, 1024, 1, 0, -1) == 0  # H not a multiple of 64


def test_bf16_acceptance_without_gpu():
    """bf16 is accepted by the MLP chain's and the conv pair's checks for the
    tile configurations that have bf16 instances (the automatic ones) and
    refused with CHAIN_EUNSUPPORTED otherwise; the attention and
    self-attention chains take it, all before any device call."""
    lib = tls.load()
    buf = np.zeros(1 << 16, dtype=np.uint8)
    base = buf.ctypes.data + (-buf.ctypes.data) % 64
    c = tls.chain_conv_args()
    c.X = c.Wa = c.Wb = c.Y = base
    c.N, c.Hh, c.Ww, c.C, c.K, c.R, c.S, c.pad, c.stride = 1, 8, 8, 64, 64, 3, 3, 1, 1
    c.policy, c.dtype = tls.POLICIES["conv2d_tilesync"], tls.DTYPES["bf16"]
    c.tile_cfg = 2  # configuration 1 (256 x 64, three stages): fp16 only
    assert lib.chain_conv_ex(ctypes.byref(c)) == tls.CHAIN_EUNSUPPORTED
    pol, bf = tls.POLICIES["conv2d_tilesync"], tls.DTYPES["bf16"]
    # tile_cfg: -1 automatic, k configuration k
    assert lib.chain_conv_workspace_bytes(1, 8, 8, 64, 64, 3, 3, 1, 1, pol, bf, -1) > 0
    assert lib.chain_conv_workspace_bytes(1, 8, 8, 64, 64, 3, 3, 1, 1, pol, bf, 3) > 0
    assert lib.chain_conv_workspace_bytes(1, 8, 8, 64, 64, 3, 3, 1, 1, pol, bf, 4) > 0
    assert lib.chain_conv_workspace_bytes(1, 8, 8, 64, 64, 3, 3, 1, 1, pol, bf, 0) > 0
    assert lib.chain_conv_workspace_bytes(1, 8, 8, 64, 64, 3, 3, 1, 1, pol, bf, 1) == 0
    assert lib.chain_conv_workspace_bytes(1, 8, 8, 64, 64, 3, 3, 1, 1, pol,
                                          tls.DTYPES["f16"], 1) > 0
    for pol in ("serial", "tilesync", "rowsync", "sentinel"):
        assert lib.chain_attn_workspace_bytes(1, 2, 256, 128, tls.POLICIES[pol], bf, -1) > 0, pol
    assert lib.chain_attn_workspace_bytes(1, 2, 256, 128, tls.POLICIES["rowsync"], 7, -1) == 0
    sa = tls.POLICIES["stridedsync"]
    assert lib.chain_selfattn_workspace_bytes(256, 1024, 2, 128, sa, tls.DTYPES["f16"]) > 0
    assert lib.chain_selfattn_workspace_bytes(256, 1024, 2, 128, sa, bf) > 0
    assert lib.chain_selfattn_workspace_bytes(256, 1024, 2, 128, sa, 7) == 0
    assert lib.chain_mlp_workspace_bytes(256, 512, 768, 1, tls.DTYPES["bf16"], -1) > 0
    assert lib.chain_mlp_workspace_bytes(256, 512, 768, 1, tls.DTYPES["bf16"], 2) == 0


def test_sentinel_ring_argument_errors_without_gpu():
    """A ring only with the sentinel policy, 2..16 slots and no z_out: all
    rejected by the host checks before any device call."""
    lib = tls.load()
    buf = np.zeros(1 << 16, dtype=np.uint8)  # host memory, 16-byte aligned
    base = buf.ctypes.data + (-buf.ctypes.data) % 64

    def args(policy, slots, z_out=False):
        a = tls.chain_mlp_args()
        a.X = a.W1 = a.W2 = a.Y = base
        a.M, a.H, a.F = 64, 256, 1024
        a.policy = policy
        a.z_ring = base
        a.ring_slots = slots
        if z_out:
            a.z_out = base
        return a

    for a in (args(tls.POLICIES["tilesync"], 2), args(tls.POLICIES["serial"], 2),
              args(tls.POLICIES["sentinel"], 1), args(tls.POLICIES["sentinel"], 17),
              args(tls.POLICIES["sentinel"], 2, z_out=True)):
        assert lib.chain_mlp_ex(ctypes.byref(a)) == tls.CHAIN_EINVAL
    with pytest.raises(ValueError):
        tls.SentinelRing(64, 1024, slots=1, device="cpu")


def test_wave_model_reproduces_paper_tables(golden_dir):
    with open(os.path.join(golden_dir, "paper_wave_tables.json")) as f:
        g = json.load(f)
    for row in g["rows"]:
        frac, serial, fused = tls.chain_wave_model(row["blocks"], row["slots"])
        for fw, want in zip(frac, row["kernel_waves"]):
            assert round(fw, 1) == pytest.approx(want), row
        assert serial == row["stream_sync_waves"], row
        assert round(fused, 1) == pytest.approx(row["fine_grained_waves"]), row


def test_toy_example_waves(golden_dir):
    with open(os.path.join(golden_dir, "paper_toy_example.json")) as f:
        w = json.load(f)["waves"]
    _, serial, fused = tls.chain_wave_model(w["blocks_per_kernel"], w["slots"])
    assert serial == w["stream_sync_waves"]
    assert -(-sum(w["blocks_per_kernel"]) // w["slots"]) == w["fine_grained_waves"]
    assert fused == pytest.approx(3.0)


def test_mlp_plan_tile_counts():
    p = tls.chain_mlp_plan(2048, 12288, 6144)
    cfg = tls.tile_configs()[p["tile_cfg"]]
    assert p["row_tiles"] == 2048 // cfg["bm"]
    assert p["producer_tiles"] == p["row_tiles"] * 6144 // cfg["bn1"]
    assert p["consumer_tiles"] == p["row_tiles"] * 12288 // cfg["bn2"]
    # ragged M rounds the row tiles up
    q = tls.chain_mlp_plan(300, 512, 768, tile_cfg=0)
    assert q["row_tiles"] == 5


@pytest.mark.parametrize("M,bm,bn,splits", [(1, 128, 128, (4, 2)), (64, 128, 128, (4, 2)),
                                             (128, 128, 128, (4, 2)), (256, 128, 128, (4, 1)),
                                             (384, 128, 128, (2, 1)), (512, 256, 128, (2, 1)),
                                             (1024, 128, 192, (1, 1)), (2048, 256, 192, (1, 1))])
def test_mlp_auto_plan_on_the_gpt3_slice(M, bm, bn, splits):
    """The automatic tile and K-split choice for H = 12288, F = 6144: one wave
    of split work items at most (one and a half for the producer GEMM of
    tiles up to 128 x 128), more splits for the weight-streaming small
    batches."""
    p = tls.chain_mlp_plan(M, 12288, 6144)
    cfg = tls.tile_configs()[p["tile_cfg"]]
    assert (cfg["bm"], cfg["bn1"]) == (bm, bn)
    assert (p["split_k1"], p["split_k2"]) == splits
    assert p["producer_tiles"] * p["split_k1"] <= (384 if bm * bn <= 128 * 128 else 256)
    assert p["consumer_tiles"] * p["split_k2"] <= 256 or p["split_k2"] == 1


@pytest.mark.parametrize("batch,side,ch", [(b, s, c) for b in (1, 8, 32)
                                            for s, c in ((56, 64), (28, 128), (14, 256), (7, 512))])
def test_conv_auto_plan_on_the_resnet38_pairs(batch, side, ch):
    """The automatic conv tile: 128 x 64 pixels x channels with K steps of 32
    and a four-stage ring for a short reduction (64 channels) over at least
    32768 pixels, with K steps of 64 and
    a three-stage ring for 128 channels over at least 16384 pixels, else
    64 x 64 with four stages; K splits only while tiles x splits fit the 512
    resident workgroups of the 64 x 64 tile with at least 16 K steps per
    split, and the largest such split is taken."""
    p = tls.chain_conv_plan(batch, side, side, ch, ch)
    npix = batch * side * side
    wide = ch <= 64 and npix >= 32768
    mid = 64 < ch <= 128 and npix >= 16384
    assert p["tile_cfg"] == (9 if wide else 0 if mid else 3)
    bm = 128 if wide or mid else 64
    assert p["row_tiles"] == -(-npix // bm)
    assert p["prod_col_tiles"] == p["cons_col_tiles"] == ch // 64
    tiles = p["row_tiles"] * ch // 64
    assert p["producer_tiles"] == p["consumer_tiles"] == tiles
    ksteps = 9 * ch // 64
    ok = [s for s in (1, 2, 4, 8)
          if s == 1 or (tiles * s <= 512 and ksteps % s == 0 and ksteps // s >= 16)]
    assert p["split_k1"] == p["split_k2"] == max(ok)


# The split the rule above gives for each ResNet-38 pair (batch, side) -> S,
# written out so that a change of the rule shows up as a diff here.
@pytest.mark.parametrize("batch,side,ch,split", [
    (1, 56, 64, 1), (8, 56, 64, 1), (32, 56, 64, 1),
    (1, 28, 128, 1), (8, 28, 128, 1), (32, 28, 128, 1),
    (1, 14, 256, 2), (8, 14, 256, 2), (32, 14, 256, 1),
    (1, 7, 512, 4), (8, 7, 512, 4), (32, 7, 512, 2)])
def test_conv_auto_split_table(batch, side, ch, split):
    p = tls.chain_conv_plan(batch, side, side, ch, ch)
    assert (p["split_k1"], p["split_k2"]) == (split, split)


def test_conv_plan_explicit_config_and_errors():
    p = tls.chain_conv_plan(2, 9, 13, 64, 128, tile_cfg=2)  # 128 x 128 tiles
    assert p["tile_cfg"] == 2 and p["row_tiles"] == -(-2 * 9 * 13 // 128) and p["prod_col_tiles"] == 1
    with pytest.raises(tls.ChainError):
        tls.chain_conv_plan(1, 8, 8, 64, 64, tile_cfg=2)  # 64 channels: not a 128-wide tile
    with pytest.raises(tls.ChainError):
        tls.chain_conv_plan(1, 8, 8, 48, 64)  # channels not a multiple of 64


@pytest.mark.parametrize("M,ks1,ks2,tail,kst", [(1, 4, 1, 0, 1), (16, 4, 1, 0, 1), (256, 3, 1, 0, 1),
                                                 (512, 3, 1, 0, 1), (640, 1, 1, 0, 1),
                                                 (768, 1, 1, 0, 1), (1024, 1, 2, 32, 4),
                                                 (2048, 1, 2, 64, 4), (4096, 1, 1, 128, 2)])
def test_selfattn_auto_plan_on_the_gpt3_shard(M, ks1, ks2, tail, kst):
    """H = 12288, 12 heads of 128: while its tiles fit one wave of the 256 CUs
    the XQKV projection splits along K into the S (<= 4, dividing the 192 K
    steps, at least 16 steps each) that needs the fewest rounds of 1 / S of a
    tile, the smaller S on a tie, if that takes at most two thirds of the
    unsplit rounds; past one wave, the same rule splits only the
    tiles after the last whole wave (the tail, last in item order); the
    attention stage splits along the keys while its items x splits fit one
    wave with at least 8 key blocks per split."""
    def rounds_over_s(tiles, s):
        return Fraction(-(-tiles * s // 256), s)

    def best(tiles):
        ok = [s for s in (1, 2, 3, 4) if 192 % s == 0 and 192 // s >= 16]
        s = min(ok, key=lambda s: (rounds_over_s(tiles, s), s))
        return s if rounds_over_s(tiles, s) <= Fraction(2, 3) * rounds_over_s(tiles, 1) else 1
    p = tls.chain_selfattn_plan(M, 12288, 12)
    assert (p["split_k1"], p["split_keys"]) == (ks1, ks2)
    assert (p["tail_tiles"], p["split_k_tail"]) == (tail, kst)
    rt = p["row_tile"]
    assert p["row_tiles"] == -(-M // rt)
    assert p["stage1_tiles"] == p["row_tiles"] * 36
    assert p["query_blocks"] == -(-M // 256) and p["key_blocks"] == -(-M // 64)
    assert p["stage1_items"] == (p["stage1_tiles"] - tail) * ks1 + tail * kst
    assert p["stage2_items"] == p["query_blocks"] * 12 * ks2
    assert p["stage3_items"] == p["row_tiles"] * 12288 // p["col_tile"]
    if p["stage1_tiles"] <= 256:
        assert ks1 == best(p["stage1_tiles"]) and tail == 0
    else:
        assert ks1 == 1 and tail == p["stage1_tiles"] % 256
        if tail:
            assert kst == best(tail)
    if ks2 > 1:
        assert p["stage2_items"] <= 256 and p["key_blocks"] // ks2 >= 8


def test_selfattn_plan_split_requests():
    # explicit splits are honoured; a key split that leaves a split without
    # keys, a K split that does not divide the K steps and out-of-range
    # requests are refused
    p = tls.chain_selfattn_plan(1000, 256, 2, split_k=2, split_keys=16)
    assert (p["split_k1"], p["split_keys"], p["key_blocks"]) == (2, 16, 16)
    # an explicit split applies to every tile: no tail split
    q = tls.chain_selfattn_plan(2048, 12288, 12, split_k=1)
    assert (q["tail_tiles"], q["split_k_tail"], q["stage1_items"]) == (0, 1, 576)
    assert p["stage2_items"] == 4 * 2 * 16
    for kw in ({"split_keys": 5}, {"split_keys": 17}, {"split_keys": -1}, {"split_k": 3},
               {"split_k": 17}):
        with pytest.raises(tls.ChainError):
            tls.chain_selfattn_plan(1000, 256, 2, **kw)
    with pytest.raises(tls.ChainError):  # d must be 128
        tls.chain_selfattn_plan(256, 256, 2, d=64)


@pytest.mark.parametrize("N,Hh,Ww,bm", [(1, 8, 8, 16), (1, 8, 8, 4), (2, 7, 5, 8), (3, 56, 56, 256),
                                        (2, 9, 13, 32)])
def test_conv_halo_range_covers_brute_force(N, Hh, Ww, bm):
    npix = N * Hh * Ww
    for t in range(-(-npix // bm)):
        lo, hi = tls.chain_conv_dep_range(t, N, Hh, Ww, bm)
        exact = {i for i, _ in oracle.conv_consumer_deps(t, N, Hh, Ww, 1, bm, 1)}
        rng = set(range(lo, hi + 1))
        assert exact <= rng, (t, exact, rng)
        # a contiguous superset that adds at most the neighbouring tile on each side
        assert min(exact) - lo <= 1 and hi - max(exact) <= 1, (t, exact, rng)


def test_first_item_knob_argument_errors_without_gpu():
    """debug_first_skip takes 0 or 1 (conv pair and attention chain); anything
    else is refused with CHAIN_EINVAL before any device call."""
    lib = tls.load()
    buf = np.zeros(1 << 16, dtype=np.uint8)
    base = buf.ctypes.data + (-buf.ctypes.data) % 64
    c = tls.chain_conv_args()
    c.X = c.Wa = c.Wb = c.Y = base
    c.N, c.Hh, c.Ww, c.C, c.K, c.R, c.S, c.pad, c.stride = 1, 8, 8, 64, 64, 3, 3, 1, 1
    c.policy, c.dtype = tls.POLICIES["conv2d_tilesync"], tls.DTYPES["f16"]
    for v in (-1, 2):
        c.debug_first_skip = v
        assert lib.chain_conv_ex(ctypes.byref(c)) == tls.CHAIN_EINVAL, v
    at = tls.chain_attn_args()
    at.Q = at.K = at.V = at.O = base
    at.B, at.heads, at.S, at.d, at.scale = 1, 1, 128, 128, 1.0
    at.policy, at.dtype = tls.POLICIES["rowsync"], tls.DTYPES["f16"]
    for v in (-1, 2):
        at.debug_first_skip = v
        assert lib.chain_attn_ex(ctypes.byref(at)) == tls.CHAIN_EINVAL, v
