"""Source check of the publish invariant the readiness protocol rests on.

A producer posts its flag with a relaxed atomic after draining its stores
(no release fence), and a consumer may take the light acquire.  That is only
correct if every store of data another workgroup reads inside the launch
(intermediates, split partials, a refilled sentinel slot) is a device-scope
store, written through to the level every XCD reads.  The kernels route those
stores through publish16/publish8 (device-scope by construction) and final
outputs through store_out16/store_out8.  This test reads the HIP sources and
checks that (a) no other code issues a raw buffer store, (b) every publish
goes to a buffer of published data and every store_out to an output, and
(c) no published buffer is written by a plain pointer store."""

import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "tile_level_sync_amd", "csrc")

PUBLISHED_BASES = {"p.Z", "p.Sc", "p.QKV", "p.Dot", "p.part1", "p.part2", "part", "dst"}
OUTPUT_BASES = {"p.Y", "p.O", "out"}  # out: the calibration copy


def _sources():
    out = {}
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip")):
            text = open(os.path.join(CSRC, name)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            text = "\n".join(re.sub(r"//.*$", "", l) for l in text.splitlines())
            out[name] = text
    return out


def test_raw_stores_only_in_the_helpers():
    for name, text in _sources().items():
        raw = re.findall(r"raw_buffer_store|buffer_store_|global_store_|flat_store_", text)
        if name == "device.h":
            assert len(raw) == 4, raw  # the bodies of the four store helpers
        else:
            assert not raw, (name, raw)
    dev = _sources()["device.h"]
    for fn, aux in (("publish16", "kAuxAgent"), ("publish8", "kAuxAgent"),
                    ("store_out16", "kAuxNone"), ("store_out8", "kAuxNone")):
        body = re.search(r"void %s\([^)]*\)\s*\{([^}]*)\}" % fn, dev).group(1)
        assert aux in body, fn


def test_every_store_goes_to_its_kind_of_buffer():
    n_pub = n_out = 0
    for name, text in _sources().items():
        if name == "device.h":
            continue
        bases = dict(re.findall(r"auto\s+(\w+)\s*=\s*make_rsrc\(\s*([\w.]+)", text))
        for var in re.findall(r"\bpublish(?:16|8)\(\s*(\w+)\s*,", text):
            assert bases.get(var) in PUBLISHED_BASES, (name, var, bases.get(var))
            n_pub += 1
        for var in re.findall(r"\bstore_out(?:16|8)\(\s*(\w+)\s*,", text):
            assert bases.get(var) in OUTPUT_BASES, (name, var, bases.get(var))
            n_out += 1
        for var, base in bases.items():
            if base in PUBLISHED_BASES:
                # a resource over published data is only ever stored through publish
                assert not re.search(r"\bstore_out(?:16|8)\(\s*%s\s*," % var, text), (name, var)
    assert n_pub >= 8 and n_out >= 4, (n_pub, n_out)


def test_no_plain_pointer_store_into_published_buffers():
    pat = re.compile(r"(\bp\.(?:Z|Sc|QKV|Dot|part1|part2)\b|\bpart\b|\bpp\b)[^;=]*\]\s*=[^=]")
    for name, text in _sources().items():
        for line in text.splitlines():
            assert not pat.search(line), (name, line.strip())
