"""Self-describing vector files, and an on-disk cache of synthetic cases in
that format.

Format ("qwen35moe CPU-reference golden vectors", section "File format"):
the first line is ASCII, ended by a newline, of the form
``PNGOLDEN1 <name> <dtype> <count> seed=0x<8 hex digits>``; the rest of the
file is exactly ``count`` little-endian values of ``dtype``, which is
``f32`` (IEEE-754 binary32), ``i32`` (two's-complement 32-bit) or ``u8``
(raw bytes).  The header holds the flat count only; shapes come from the
case the file belongs to.

This layer stores bf16 tensors (kept as their 16-bit patterns) as ``u8``
files of their little-endian bytes, with ``.bf16`` appended to the name, so
every file stays within the three dtypes of the format.  A cached case is a
directory: one ``<tensor>.bin`` per tensor plus ``case.json`` with the
case's configuration and each tensor's shape and element type.

Only storage lives here: no arithmetic of the layer."""
from __future__ import annotations

import dataclasses
import json
import os
import re
import tempfile

import numpy as np

MAGIC = "PNGOLDEN1"
_DTYPES = {"f32": np.dtype("<f4"), "i32": np.dtype("<i4"), "u8": np.dtype("u1")}
_HEADER = re.compile(r"^PNGOLDEN1 (\S+) (f32|i32|u8) ([0-9]+) seed=0x([0-9A-Fa-f]{1,8})$")


def _kind(a: np.ndarray) -> str:
    if a.dtype == np.float32:
        return "f32"
    if a.dtype == np.int32:
        return "i32"
    if a.dtype == np.uint8:
        return "u8"
    if a.dtype == np.uint16:
        return "bf16"
    raise ValueError("no vector-file dtype for %s" % a.dtype)


def write_vector(path: str, name: str, values: np.ndarray, seed: int) -> None:
    """Write one tensor.  float32 / int32 / uint8 arrays keep their dtype;
    uint16 arrays (bf16 bit patterns) are written as u8 bytes under
    ``name + ".bf16"``."""
    if not name or any(ch.isspace() for ch in name):
        raise ValueError("vector name must be one non-empty word: %r" % name)
    a = np.ascontiguousarray(values)
    kind = _kind(a)
    if kind == "bf16":
        name, kind, payload = name + ".bf16", "u8", a.astype("<u2").view(np.uint8).reshape(-1)
    else:
        payload = a.astype(_DTYPES[kind]).reshape(-1)
    header = "%s %s %s %d seed=0x%08X\n" % (MAGIC, name, kind, payload.size, seed & 0xFFFFFFFF)
    with open(path, "wb") as f:
        f.write(header.encode("ascii"))
        f.write(payload.tobytes())


def read_vector(path: str):
    """Read one file: (name, dtype, seed, flat values).  A ``.bf16`` name
    comes back as uint16 values under the name without the suffix.  Raises
    ValueError on a malformed header or a payload of the wrong length."""
    with open(path, "rb") as f:
        data = f.read()
    nl = data.find(b"\n")
    if nl < 0:
        raise ValueError("%s: no header line" % path)
    try:
        line = data[:nl].decode("ascii")
    except UnicodeDecodeError as e:
        raise ValueError("%s: header is not ASCII" % path) from e
    m = _HEADER.match(line)
    if not m:
        raise ValueError("%s: not a %s header: %r" % (path, MAGIC, line[:80]))
    name, kind, count, seed = m.group(1), m.group(2), int(m.group(3)), int(m.group(4), 16)
    dt = _DTYPES[kind]
    body = data[nl + 1:]
    if len(body) != count * dt.itemsize:
        raise ValueError("%s: payload holds %d bytes, header says %d x %d" % (path, len(body), count, dt.itemsize))
    values = np.frombuffer(body, dtype=dt).copy()
    if kind == "u8" and name.endswith(".bf16"):
        if count % 2:
            raise ValueError("%s: odd byte count for a bf16 vector" % path)
        return name[:-5], "bf16", seed, values.view("<u2").astype(np.uint16)
    return name, kind, seed, values.astype(dt.newbyteorder("="))


_SCALARS = ("name", "T", "H", "E", "k", "F", "Fs", "gating", "norm_topk_prob", "weights_scale", "act", "alpha",
            "limit", "x_dtype", "w_dtype", "router_dtype", "drawn_logits", "act_quant", "norm_eps")


def save_case(case, directory: str, seed: int, tensors=None) -> None:
    """Write the tensors of ``case`` named in ``tensors`` (all by default) and
    its configuration to ``directory`` (created if missing; files are written
    under temporary names and moved into place, so a reader never sees a
    half-written case)."""
    os.makedirs(directory, exist_ok=True)
    meta = {"format": MAGIC, "seed": seed & 0xFFFFFFFF,
            "config": {f: getattr(case, f) for f in _SCALARS},
            "tensors": {}}
    for tname, a in case.t.items():
        if tensors is not None and tname not in tensors:
            continue
        a = np.asarray(a)
        fd, tmp = tempfile.mkstemp(dir=directory, suffix=".tmp")
        os.close(fd)
        write_vector(tmp, tname, a, seed)
        os.replace(tmp, os.path.join(directory, tname + ".bin"))
        meta["tensors"][tname] = {"shape": list(a.shape), "kind": _kind(a)}
    fd, tmp = tempfile.mkstemp(dir=directory, suffix=".tmp")
    with os.fdopen(fd, "w") as f:
        json.dump(meta, f, indent=1, sort_keys=True)
    os.replace(tmp, os.path.join(directory, "case.json"))


def load_case(directory: str):
    """The case saved by save_case, tensors restored to their shapes."""
    from . import Case
    with open(os.path.join(directory, "case.json")) as f:
        meta = json.load(f)
    if meta.get("format") != MAGIC:
        raise ValueError("%s: not a cached case" % directory)
    fields = {f.name for f in dataclasses.fields(Case)}
    c = Case(**{k: v for k, v in meta["config"].items() if k in fields})
    for tname, info in meta["tensors"].items():
        name, kind, seed, values = read_vector(os.path.join(directory, tname + ".bin"))
        if name != tname or kind != info["kind"] or seed != meta["seed"]:
            raise ValueError("%s: file %s.bin holds %s/%s/seed 0x%08X" % (directory, tname, name, kind, seed))
        c.t[tname] = values.reshape(info["shape"])
    return c


# tensors that depend on the token count; the rest (weights) do not
TOKEN_TENSORS = ("x", "logits")


def case_key(name: str, T: int | None, seed: int, **overrides) -> str:
    """Directory name of a cached case part: configuration, tokens (None for
    the weights), seed and any shape overrides."""
    extra = "".join("-%s%s" % (k, overrides[k]) for k in sorted(overrides))
    part = "weights" if T is None else "T%d" % T
    return "%s-%s-seed%08X%s" % (name, part, seed & 0xFFFFFFFF, extra)


def cached_case(cache_dir: str, name: str, T: int, seed: int | None = None, **overrides):
    """make_case(name, T, seed, **overrides), read from ``cache_dir`` when a
    previous call saved it there, else generated and saved.  The weights are
    kept once per (case, seed, overrides), the token tensors per T."""
    from . import BASE_SEED, make_case
    seed = BASE_SEED if seed is None else seed
    wdir = os.path.join(cache_dir, case_key(name, None, seed, **overrides))
    tdir = os.path.join(cache_dir, case_key(name, T, seed, **overrides))
    if os.path.exists(os.path.join(wdir, "case.json")) and os.path.exists(os.path.join(tdir, "case.json")):
        c = load_case(tdir)
        c.t.update(load_case(wdir).t)
        return c
    c = make_case(name, T=T, seed=seed, **overrides)
    if not os.path.exists(os.path.join(wdir, "case.json")):
        save_case(c, wdir, seed, [k for k in c.t if k not in TOKEN_TENSORS])
    save_case(c, tdir, seed, [k for k in c.t if k in TOKEN_TENSORS])
    return c
