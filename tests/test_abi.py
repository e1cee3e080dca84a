"""The C ABI library loads, exports every symbol include/pkv.h declares, and
rejects bad host arguments before any launch (CPU only: no kernel runs)."""
import ctypes
import os
import re

import pytest

import paged_kv_cache_indirected_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def _declared():
    """Functions the header declares for the library to export (its static
    inline helpers are compiled into the caller and are not exported)."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    inline = set(re.findall(r"static\s+inline[^(]*?\b(pkv_[a-z0-9_]+)\s*\(", src))
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", src)) - inline)


def test_every_declared_symbol_is_exported():
    names = _declared()
    assert "pkv_decode" in names and "pkv_append" in names and "pkv_prefill_chunk" in names
    lib = ctypes.CDLL(pkv.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing


def test_debug_library_exports_every_declared_symbol():
    """libpkv_debug.so (PKV_DEBUG: synchronising, device-checked calls) is a
    drop-in for libpkv.so: same symbols, same ABI version."""
    path = os.path.join(os.path.dirname(pkv.LIB_PATH), "libpkv_debug.so")
    lib = ctypes.CDLL(path)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    lib.pkv_abi_version.restype = ctypes.c_int
    assert lib.pkv_abi_version() == pkv.abi_version()


def test_abi_version_and_strerror():
    assert pkv.abi_version() == 2
    for code in (pkv.OK, pkv.EINVAL, pkv.EUNSUPPORTED, pkv.ENOBLOCKS, pkv.ESTATE, pkv.EHIP):
        assert pkv.strerror(code) and pkv.strerror(code) != "unknown error code"


L = pkv._lib
FAKE = 0x10000          # a 16-byte aligned address that is never dereferenced
MIS = 0x10004


def _desc(**kw):
    d = dict(num_blocks=64, num_kv_heads=8, block_size=16, head_dim=128, dtype=pkv.BF16)
    d.update(kw)
    return pkv.CacheDescC(**d)


def _decode(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, stride=8, lens=FAKE, B=2, Hq=64, maxL=100,
             scale=0.1, out=FAKE, odt=pkv.F32, pt=0, ws=FAKE, wsb=1 << 30, desc=_desc())
    a.update(kw)
    return L.pkv_decode(a["q"], a["kc"], a["vc"], a["bt"], a["stride"], a["lens"], a["B"], a["Hq"],
                        a["maxL"], a["scale"], a["out"], a["odt"], a["pt"], a["ws"], a["wsb"],
                        ctypes.byref(a["desc"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), pkv.EINVAL),
    (dict(q=MIS), pkv.EINVAL),
    (dict(out=None), pkv.EINVAL),
    (dict(Hq=60), pkv.EINVAL),
    (dict(Hq=128), pkv.EUNSUPPORTED),          # group of 16
    (dict(desc=_desc(head_dim=96)), pkv.EUNSUPPORTED),
    (dict(desc=_desc(block_size=8)), pkv.EUNSUPPORTED),
    (dict(desc=_desc(dtype=7)), pkv.EUNSUPPORTED),
    (dict(desc=_desc(num_blocks=0)), pkv.EINVAL),
    (dict(maxL=16 * 8 + 1), pkv.EINVAL),       # beyond stride * block_size
    (dict(pt=-1), pkv.EINVAL),                 # negative split count
    (dict(pt=70000), pkv.EINVAL),              # split count beyond the grid
    (dict(odt=3), pkv.EINVAL),
    (dict(scale=float("nan")), pkv.EINVAL),
    (dict(B=-1), pkv.EINVAL),
    (dict(maxL=128, pt=4, wsb=16), pkv.EINVAL),    # short workspace
    (dict(maxL=128, pt=0, ws=None), pkv.EINVAL),   # the workspace is always needed
])
def test_decode_rejects(kw, code):
    assert _decode(**kw) == code
    assert pkv._lib.pkv_last_error().decode() != ""


def test_decode_empty_batch_is_a_noop():
    assert _decode(B=0, q=None, out=None) == pkv.OK


def test_workspace_size_rules():
    d = _desc()
    # Prefix sums [B + 1] plus (W + B) partial rows of every query head.
    for B, W in ((4, 1), (4, 37), (32, 128), (3000, 128)):
        n = L.pkv_decode_workspace_bytes(B, 64, 1000, W, ctypes.byref(d))
        bc = min(B, 1024)
        pieces = W + bc
        assert n >= (bc + 1) * 4 + pieces * 64 * 128 * 4 + pieces * 64 * 2 * 4
    assert L.pkv_decode_workspace_bytes(0, 64, 1000, 8, ctypes.byref(d)) == 0
    assert L.pkv_decode_workspace_bytes(4, 64, 1000, -1, ctypes.byref(d)) == 0
    # Library choice: one workgroup per CU over the KV heads (256 CUs when no
    # device can be queried), independent of the batch.
    w = L.pkv_decode_num_splits(32, 64, 4096, ctypes.byref(d))
    assert 1 <= w <= 65535
    assert w == L.pkv_decode_num_splits(1, 64, 16, ctypes.byref(d))
    assert L.pkv_decode_workspace_bytes(32, 64, 4096, 0, ctypes.byref(d)) == \
        L.pkv_decode_workspace_bytes(32, 64, 4096, w, ctypes.byref(d))


def test_append_rejects():
    d = _desc()
    assert L.pkv_append(None, FAKE, FAKE, 4, FAKE, FAKE, ctypes.byref(d), None) == pkv.EINVAL
    assert L.pkv_append(FAKE, FAKE, None, 4, FAKE, FAKE, ctypes.byref(d), None) == pkv.EINVAL
    assert L.pkv_append(FAKE, FAKE, FAKE, -1, FAKE, FAKE, ctypes.byref(d), None) == pkv.EINVAL
    assert L.pkv_append(FAKE, MIS, FAKE, 4, FAKE, FAKE, ctypes.byref(d), None) == pkv.EINVAL
    assert L.pkv_append(FAKE, FAKE, FAKE, 0, FAKE, FAKE, ctypes.byref(d), None) == pkv.OK
    bad = _desc(head_dim=80)
    assert L.pkv_append(FAKE, FAKE, FAKE, 4, FAKE, FAKE, ctypes.byref(bad), None) == pkv.EUNSUPPORTED


def test_prefill_rejects():
    def call(**kw):
        a = dict(q=FAKE, qsl=FAKE, S=2, maxq=16, kc=FAKE, vc=FAKE, bt=FAKE, stride=8, lens=FAKE,
                 maxL=100, Hq=64, scale=0.1, out=FAKE, odt=pkv.F32, desc=_desc())
        a.update(kw)
        return L.pkv_prefill_chunk(a["q"], a["qsl"], a["S"], a["maxq"], a["kc"], a["vc"], a["bt"],
                                   a["stride"], a["lens"], a["maxL"], a["Hq"], a["scale"], a["out"],
                                   a["odt"], None, 0, ctypes.byref(a["desc"]), None)
    assert call(desc=_desc(dtype=pkv.F32)) == pkv.EUNSUPPORTED
    assert call(q=None) == pkv.EINVAL
    assert call(qsl=None) == pkv.EINVAL
    assert call(maxL=10_000) == pkv.EINVAL
    assert call(Hq=12) == pkv.EINVAL
    assert call(S=0) == pkv.OK


def test_pool_create_rejects_empty():
    with pytest.raises(pkv.PkvError):
        pkv.Pool(0)


def test_single_hip_runtime_in_process():
    # libpkv must bind the HIP runtime torch loaded, never a second copy.
    import subprocess
    import sys
    code = ("import re, paged_kv_cache_indirected_amd, torch;"
            "m=open('/proc/self/maps').read();"
            "print(len(set(re.findall(r'(\\S*libamdhip64\\S*)', m))))")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         cwd=ROOT, check=True).stdout.strip()
    assert out == "1"


def test_append_decode_rejects():
    d = _desc()
    f = L.pkv_append_decode
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, FAKE, 2, 64, 100, 0.1, FAKE, pkv.F32, 0,
            FAKE, 1 << 30, ctypes.byref(d), None]
    for i, code in ((0, pkv.EINVAL), (1, pkv.EINVAL), (2, pkv.EINVAL)):
        bad = list(args)
        bad[i] = None
        assert f(*bad) == code
    bad = list(args)
    bad[0] = MIS
    assert f(*bad) == pkv.EINVAL
    bad = list(args)
    bad[9] = 0      # empty batch: a no-op even without rows
    bad[0] = bad[1] = bad[2] = None
    assert f(*bad) == pkv.OK


def test_copy_blocks_rejects():
    d = _desc()
    f = L.pkv_copy_blocks

    def call(sk=FAKE, sv=FAKE, sd=d, dk=FAKE, dv=FAKE, dd=d, si=FAKE, di=FAKE, n=4):
        return f(sk, sv, ctypes.byref(sd), dk, dv, ctypes.byref(dd), si, di, n, None)
    assert call(sk=None) == pkv.EINVAL
    assert call(dv=MIS) == pkv.EINVAL
    assert call(si=None) == pkv.EINVAL
    assert call(n=-1) == pkv.EINVAL
    assert call(dd=_desc(block_size=32)) == pkv.EINVAL          # block shapes differ
    assert call(dd=_desc(dtype=pkv.F32)) == pkv.EINVAL
    assert call(sd=_desc(head_dim=96)) == pkv.EUNSUPPORTED
    assert call(n=0, sk=None, si=None) == pkv.OK                 # empty list: no-op
    # Only the block shape must agree: the caches may differ in size.
    assert call(n=0, dd=_desc(num_blocks=3)) == pkv.OK


def test_decode_cascade_rejects():
    f = L.pkv_decode_cascade

    def call(desc=None, P=32, pb=FAKE, ws=FAKE, wsb=1 << 30, B=2):
        d = desc or _desc()
        return f(FAKE, FAKE, FAKE, pb, P, FAKE, 8, FAKE, B, 64, 100, 0.1, FAKE, pkv.F32, ws, wsb,
                 ctypes.byref(d), None)
    assert call(desc=_desc(dtype=pkv.F32)) == pkv.EUNSUPPORTED
    assert call(P=20) == pkv.EINVAL                    # not a whole number of blocks
    assert call(P=-16) == pkv.EINVAL
    assert call(pb=None) == pkv.EINVAL
    assert call(wsb=64) == pkv.EINVAL                  # short workspace
    assert call(ws=None) == pkv.EINVAL
    assert call(B=0) == pkv.OK
    assert L.pkv_decode_cascade_workspace_bytes(2, 64, 32, 100, ctypes.byref(_desc())) > 0


def test_prefill_workspace_sizes_key_split_states():
    # A short grid (1 sequence x 4 q-tiles x 8 KV heads = 32 workgroups) asks
    # for split states: k fp32 outputs and log2-sum-exps of S * max_query_len
    # * Hq rows, each array 256-byte aligned; a grid of many workgroups, an
    # fp32 cache or a head_dim without a kernel asks for none.
    d = _desc()
    rows = 1 * 64 * 64
    n = L.pkv_prefill_workspace_bytes(1, 64, 64, ctypes.byref(d))
    assert n > 0
    per_split = (rows * d.head_dim * 4 + 255) // 256 * 256 + (rows * 4 + 255) // 256 * 256
    assert n % per_split == 0 and 2 <= n // per_split <= 16
    assert L.pkv_prefill_workspace_bytes(64, 64, 4096, ctypes.byref(d)) == 0
    assert L.pkv_prefill_workspace_bytes(1, 64, 64, ctypes.byref(_desc(dtype=pkv.F32))) == 0
    assert L.pkv_prefill_workspace_bytes(1, 64, 64, ctypes.byref(_desc(head_dim=96))) == 0
    assert L.pkv_prefill_workspace_bytes(0, 64, 64, ctypes.byref(d)) == 0


def _decode_noalloc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, stride=8, lens=FAKE, B=2, Hq=64, maxL=100,
             scale=0.1, out=FAKE, odt=pkv.F32, pt=0, desc=_desc())
    a.update(kw)
    return L.pkv_decode_noalloc(a["q"], a["kc"], a["vc"], a["bt"], a["stride"], a["lens"], a["B"],
                                a["Hq"], a["maxL"], a["scale"], a["out"], a["odt"], a["pt"],
                                ctypes.byref(a["desc"]), None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), pkv.EINVAL),
    (dict(out=MIS), pkv.EINVAL),
    (dict(Hq=128), pkv.EUNSUPPORTED),
    (dict(maxL=16 * 8 + 1), pkv.EINVAL),
    (dict(pt=-1), pkv.EINVAL),
    (dict(odt=3), pkv.EINVAL),
    (dict(B=600), pkv.EINVAL),        # partials beyond the no-allocation scratch
    (dict(B=2, pt=4000), pkv.EINVAL),  # likewise, through the split count
])
def test_decode_noalloc_rejects(kw, code):
    # Rejected on the host, before any device call (none is possible here).
    assert _decode_noalloc(**kw) == code
    assert pkv._lib.pkv_last_error().decode() != ""


def test_decode_noalloc_limit_matches_header():
    src = open(HEADER).read()
    assert "#define PKV_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)" in src
    assert pkv.DECODE_NOALLOC_SCRATCH_BYTES == 16 << 20
    d = _desc()
    # The largest batch that fits at the library's split for 64 query heads.
    fits = [B for B in (1, 32, 256, 400, 600, 1024)
            if L.pkv_decode_workspace_bytes(B, 64, 100, 0, ctypes.byref(d)) <= 16 << 20]
    assert 32 in fits and 256 in fits and 600 not in fits
    assert _decode_noalloc(B=0, q=None, out=None) == pkv.OK
