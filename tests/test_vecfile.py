"""Vector files in the format of "qwen35moe CPU-reference golden vectors",
section "File format", and the on-disk case cache built on them.

The byte-level test writes the header and payload the section describes by
hand (struct.pack of little-endian values after one ASCII line) and checks
that the writer produces exactly those bytes and the reader takes them back;
the rest round-trips every element type the synthetic cases use and checks
that malformed files are rejected."""
import os
import struct

import numpy as np
import pytest

import synth
from synth import vecfile


def test_bytes_are_the_pages_layout(tmp_path):
    p = str(tmp_path / "v.bin")
    vals = np.array([1.5, -0.0, 3.0e-8], np.float32)
    vecfile.write_vector(p, "router_logits", vals, 0x9E3779B9)
    expect = b"PNGOLDEN1 router_logits f32 3 seed=0x9E3779B9\n" + struct.pack("<3f", 1.5, -0.0, 3.0e-8)
    assert open(p, "rb").read() == expect
    ints = b"PNGOLDEN1 topk_idx i32 4 seed=0x9E3779B9\n" + struct.pack("<4i", 7, -1, 0, 2 ** 31 - 1)
    q = str(tmp_path / "i.bin")
    open(q, "wb").write(ints)
    name, kind, seed, got = vecfile.read_vector(q)
    assert (name, kind, seed) == ("topk_idx", "i32", 0x9E3779B9)
    assert got.dtype == np.int32 and got.tolist() == [7, -1, 0, 2 ** 31 - 1]


@pytest.mark.parametrize("a", [
    np.arange(-5, 7, dtype=np.float32) / 3,
    np.array([[1, -2], [3, 2 ** 31 - 1]], np.int32),
    np.arange(256, dtype=np.uint8),
    synth.bf16_bits(np.array([1.0, -2.5, 3.0e38, 1e-40], np.float32)),
], ids=["f32", "i32", "u8", "bf16"])
def test_round_trip(tmp_path, a):
    p = str(tmp_path / "t.bin")
    vecfile.write_vector(p, "t", a, 0x1234)
    name, kind, seed, got = vecfile.read_vector(p)
    assert name == "t" and seed == 0x1234
    assert got.dtype == a.dtype and np.array_equal(got, a.reshape(-1))
    if a.dtype == np.uint16:
        # a bf16 tensor is a u8 file of its little-endian bytes
        head = open(p, "rb").read().split(b"\n", 1)[0]
        assert head == b"PNGOLDEN1 t.bf16 u8 %d seed=0x00001234" % (2 * a.size)


@pytest.mark.parametrize("blob", [
    b"PNGOLDEN2 x f32 1 seed=0x1\n\0\0\0\0",          # wrong magic
    b"PNGOLDEN1 x f64 1 seed=0x1\n" + b"\0" * 8,       # dtype outside the format
    b"PNGOLDEN1 x f32 2 seed=0x1\n\0\0\0\0",           # short payload
    b"PNGOLDEN1 x f32 1 seed=0x1\n\0\0\0\0\0",         # trailing byte
    b"PNGOLDEN1 x f32 1 seed=0x1",                     # no newline
    b"PNGOLDEN1 x.bf16 u8 3 seed=0x1\n\0\0\0",         # odd byte count for bf16
])
def test_malformed_files_are_rejected(tmp_path, blob):
    p = str(tmp_path / "bad.bin")
    open(p, "wb").write(blob)
    with pytest.raises(ValueError):
        vecfile.read_vector(p)


def _same(a, b):
    assert a.name == b.name and a.T == b.T and a.w_dtype == b.w_dtype and a.norm_eps == b.norm_eps
    assert sorted(a.t) == sorted(b.t)
    for k in a.t:
        x, y = np.asarray(a.t[k]), np.asarray(b.t[k])
        assert x.dtype == y.dtype and x.shape == y.shape and np.array_equal(x.view(np.uint8), y.view(np.uint8)), k


@pytest.mark.parametrize("name,T,over", [
    ("tiny_fp32", 5, {}),
    ("gptoss20b_mxfp4", 3, dict(E=4, H=64, F=64)),
    ("qwen35moe_prefill_zipf", 9, dict(E=8, H=64, F=64, Fs=64)),
])
def test_case_cache_round_trip(tmp_path, name, T, over):
    d = str(tmp_path / "cache")
    first = vecfile.cached_case(d, name, T, **over)
    _same(first, synth.make_case(name, T=T, **over))
    keys = sorted(os.listdir(d))
    assert len(keys) == 2 and any("-weights-" in k for k in keys)
    stamp = {k: os.stat(os.path.join(d, k, "case.json")).st_mtime_ns for k in keys}
    again = vecfile.cached_case(d, name, T, **over)      # read back, not regenerated
    _same(again, first)
    assert {k: os.stat(os.path.join(d, k, "case.json")).st_mtime_ns for k in keys} == stamp
    other = vecfile.cached_case(d, name, T + 2, **over)  # weights shared, tokens per T
    _same(other, synth.make_case(name, T=T + 2, **over))
    assert len(os.listdir(d)) == 3
