"""The cache layout the public header states is the one the append writes
(CPU only).  A caller that fills a paged cache by any route other than
pkv_append must be able to do it from the header alone: its inline offset
helpers, compiled here with gcc from include/pkv.h, must name the element
that the oracle's append writes for every (block, head, token, dim)."""
import os
import subprocess

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "layout", "elem_offsets.c")


@pytest.fixture(scope="module")
def offsets_tool(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("layout") / "elem_offsets")
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    SRC, "-o", exe], check=True)
    return exe


def _header_offsets(exe, rows):
    text = "".join(" ".join(str(int(x)) for x in r) + "\n" for r in rows)
    out = subprocess.run([exe], input=text, capture_output=True, text=True, check=True).stdout
    return np.array([[int(x) for x in ln.split()] for ln in out.splitlines()], dtype=np.int64)


GRID = [(bs, D, dt) for bs in (16, 32) for D in (64, 128) for dt in ("f32", "bf16")]


@pytest.mark.parametrize("bs,D,dt", GRID)
def test_header_tile_offsets_equal_oracle_tile_index(offsets_tool, bs, D, dt):
    es = 4 if dt == "f32" else 2
    code = 0 if dt == "f32" else 1
    rows, want = [], []
    for t in range(bs):
        for d in range(D):
            rows.append((4, 2, bs, D, code, 0, 0, t, d))
            want.append(oracle.tile_index(t, d, bs, D, es))
    got = _header_offsets(offsets_tool, rows)
    assert np.array_equal(got, np.array(want, dtype=np.int64))


@pytest.mark.parametrize("bs,D,dt", GRID)
def test_header_offsets_locate_what_append_writes(offsets_tool, bs, D, dt):
    # One row per sampled (block, token) slot, each element a distinct value;
    # after the oracle's append, the header's offset of (block, head, t, d)
    # must hold element d of that row's head.
    Hkv, nb = 3, 5
    es = 4 if dt == "f32" else 2
    code = 0 if dt == "f32" else 1
    npdt = np.float32 if dt == "f32" else np.uint16
    g = np.random.default_rng(bs * 1000 + D + es)
    slots = g.choice(nb * bs, size=7, replace=False).astype(np.int32)
    T = len(slots)
    vals = np.arange(1, T * Hkv * D + 1).reshape(T, Hkv, D)
    k = vals.astype(npdt)
    v = (vals + 50000).astype(npdt)
    kc = np.zeros((nb, Hkv, bs, D), dtype=npdt)
    vc = np.zeros_like(kc)
    oracle.append(k, v, slots, kc, vc, bs)
    rows, idx = [], []
    for ti, s in enumerate(slots):
        for h in range(Hkv):
            for d in range(D):
                rows.append((nb, Hkv, bs, D, code, s // bs, h, s % bs, d))
                idx.append((ti, h, d))
    off = _header_offsets(offsets_tool, rows)
    kf, vf = kc.reshape(-1), vc.reshape(-1)
    for (ti, h, d), (ko, vo) in zip(idx, off):
        assert kf[ko] == k[ti, h, d] and vf[vo] == v[ti, h, d], (ti, h, d)
    # and nothing else was written
    assert np.count_nonzero(kf) == T * Hkv * D and np.count_nonzero(vf) == T * Hkv * D
