"""Calls for the debug build of the library (libpkv_debug.so, built with
PKV_DEBUG): valid calls of every checked entry point, and calls that break a
device precondition (block id outside the pool, context length outside its
bounds, append slot or copy id beyond the cache).

test_gpu_debug.py runs `valid_outputs()` in its own process on the release
library and runs this file as a script in a child process with PKV_DEBUG=1:
the child checks that every broken call returns PKV_EINVAL naming the
violation, that the next valid call succeeds again, and saves the valid
calls' outputs for a bitwise comparison with the release build.  Every
broken input here is one the kernels already tolerate (ids and slots out of
range are skipped, lengths clamped), so no call reads or writes outside its
buffers in either build.
"""
from __future__ import annotations

import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
for p in (os.path.dirname(HERE), HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import paged_kv_cache_indirected_amd as pkv  # noqa: E402
import synth  # noqa: E402
from harness import (decode_state, prefill_state, run_decode, run_prefill, say,  # noqa: E402
                     step_state)


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.contiguous()
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16).cpu().numpy()


def _decode_inputs():
    b = synth.custom_decode(61, [1, 17, 40, 300, 33], Hq=16, Hkv=2, D=128, dtype="bf16",
                            block_size=16)
    return b, decode_state(b)


def _wide_inputs():
    # More than 64 sequences: the decode kernel's other set-up path.
    lens = synth.rng(64, 0).integers(1, 60, size=70).tolist()
    b = synth.custom_decode(64, lens, Hq=16, Hkv=2, D=128, dtype="bf16", block_size=16)
    return b, decode_state(b)


def _prefill_inputs():
    p = synth.custom_prefill(62, [0, 100, 37], [20, 64, 3], Hq=16, Hkv=2, D=128, block_size=16)
    return p, prefill_state(p)


def _step_inputs():
    b = synth.custom_decode(63, [40, 1, 17, 300], Hq=16, Hkv=2, D=128, dtype="bf16",
                            block_size=16)
    return b, step_state(b)


def _append_decode(st, scale, slots):
    cache, _, kn, vn, q, tab, lens, mx = st
    B, Hq, D = q.shape
    ws = torch.zeros(pkv.decode_workspace_bytes(B, Hq, mx, cache.desc, 0), dtype=torch.uint8,
                     device=q.device)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=q.device)
    pkv.append_decode(kn, vn, slots, q, cache.k_cache, cache.v_cache, tab, lens, scale, out,
                      cache.desc, mx, workspace=ws)
    torch.cuda.synchronize()
    return out


def _copy(cache, src, dst):
    dk, dv = torch.zeros_like(cache.k_cache), torch.zeros_like(cache.v_cache)
    ids = lambda a: torch.tensor(np.asarray(a, dtype=np.int32), device=cache.device)  # noqa: E731
    pkv.copy_blocks(cache.k_cache, cache.v_cache, cache.desc, dk, dv, cache.desc, ids(src),
                    ids(dst))
    torch.cuda.synchronize()
    return dk, dv


def valid_outputs() -> dict:
    """Outputs of valid calls of every checked entry point, as bit patterns
    (the same in both builds: the checks change no arithmetic)."""
    out = {}
    b, (cache, q, tab, lens, mx) = _decode_inputs()
    out["decode"] = _bits(run_decode(cache, q, tab, lens, mx, b.shape.scale))
    out["decode_one_split"] = _bits(run_decode(cache, q, tab, lens, mx, b.shape.scale,
                                               num_splits=1))
    w, (wc, wq, wtab, wlens, wmx) = _wide_inputs()
    out["decode_wide"] = _bits(run_decode(wc, wq, wtab, wlens, wmx, w.shape.scale))
    p, (pc, pq, qs, ptab, plens, pmx) = _prefill_inputs()
    mq = int(p.chunk.max())
    out["prefill_split"] = _bits(run_prefill(pc, pq, qs, ptab, plens, pmx, p.shape.scale, mq))
    out["prefill_one_pass"] = _bits(run_prefill(pc, pq, qs, ptab, plens, pmx, p.shape.scale, mq,
                                                split=False))
    s, st = _step_inputs()
    out["append_decode"] = _bits(_append_decode(st, s.shape.scale, st[1]))
    out["append_decode_k_cache"] = _bits(st[0].k_cache)
    out["append_decode_v_cache"] = _bits(st[0].v_cache)
    dk, dv = _copy(cache, [0, 3, -1, 5], [1, 2, 4, -3])
    out["copy_k"], out["copy_v"] = _bits(dk), _bits(dv)
    return out


def _expect_einval(what: str, call) -> None:
    try:
        call()
    except pkv.PkvError as e:
        assert e.code == pkv.EINVAL and what in str(e), str(e)
        say(f"  rejected as expected: {e}")
        return
    raise AssertionError(f"no error for a call with {what}")


def broken_calls() -> None:
    """Each broken call fails with PKV_EINVAL naming its violation; the valid
    call after it succeeds (the flags were cleared)."""
    b, (cache, q, tab, lens, mx) = _decode_inputs()
    good = _bits(run_decode(cache, q, tab, lens, mx, b.shape.scale))

    def again():
        assert np.array_equal(_bits(run_decode(cache, q, tab, lens, mx, b.shape.scale)), good)

    say("[debug] decode: block id outside the pool (past the end, then negative)")
    for bad in (cache.desc.num_blocks + 7, -5):
        t2 = tab.clone()
        t2[3, 2] = bad                        # sequence 3 holds 300 tokens: block 2 is read
        _expect_einval("block id outside the pool",
                       lambda: run_decode(cache, q, t2, lens, mx, b.shape.scale))
        again()
    say("[debug] decode: context length above max_context_len, then negative")
    for i, bad in ((1, mx + 1), (0, -1)):
        l2 = lens.clone()
        l2[i] = bad
        _expect_einval("context length",
                       lambda: run_decode(cache, q, tab, l2, mx, b.shape.scale))
        again()

    say("[debug] decode over more than 64 sequences: context length above max_context_len")
    w, (wc, wq, wtab, wlens, wmx) = _wide_inputs()
    l2 = wlens.clone()
    l2[67] = wmx + 3
    _expect_einval("context length", lambda: run_decode(wc, wq, wtab, l2, wmx, w.shape.scale))
    run_decode(wc, wq, wtab, wlens, wmx, w.shape.scale)

    say("[debug] prefill: block id outside the pool, context length below its chunk")
    p, (pc, pq, qs, ptab, plens, pmx) = _prefill_inputs()
    mq = int(p.chunk.max())
    for split in (True, False):
        t2 = ptab.clone()
        t2[1, 3] = -3                          # sequence 1 holds 164 tokens
        _expect_einval("block id outside the pool",
                       lambda: run_prefill(pc, pq, qs, t2, plens, pmx, p.shape.scale, mq,
                                           split=split))
        l2 = plens.clone()
        l2[2] = 2                              # its chunk is 3 rows
        _expect_einval("below its chunk",
                       lambda: run_prefill(pc, pq, qs, ptab, l2, pmx, p.shape.scale, mq,
                                           split=split))
        run_prefill(pc, pq, qs, ptab, plens, pmx, p.shape.scale, mq, split=split)

    say("[debug] append: slot at the end of the cache; negative slots are padding")
    cap = cache.desc.num_blocks * cache.desc.block_size
    kn = torch.zeros((3, cache.desc.num_kv_heads, cache.desc.head_dim), dtype=q.dtype,
                     device=q.device)
    kc0, vc0 = cache.k_cache.clone(), cache.v_cache.clone()
    slots = torch.tensor([-1, cap, -7], dtype=torch.int32, device=q.device)
    _expect_einval("append slot beyond the cache",
                   lambda: pkv.append(kn, kn, slots, cache.k_cache, cache.v_cache, cache.desc))
    pkv.append(kn, kn, torch.tensor([-1, -2, -7], dtype=torch.int32, device=q.device),
               cache.k_cache, cache.v_cache, cache.desc)
    torch.cuda.synchronize()
    assert torch.equal(_bits_t(kc0), _bits_t(cache.k_cache))
    assert torch.equal(_bits_t(vc0), _bits_t(cache.v_cache))

    say("[debug] append: two rows mapped to one slot (into copies of the cache)")
    kc1, vc1 = cache.k_cache.clone(), cache.v_cache.clone()
    dup = torch.tensor([21, -1, 21], dtype=torch.int32, device=q.device)
    _expect_einval("mapped twice", lambda: pkv.append(kn, kn, dup, kc1, vc1, cache.desc))

    say("[debug] append_decode: slot past the end of the cache")
    s, st = _step_inputs()
    sl2 = st[1].clone()
    sl2[2] = st[0].desc.num_blocks * st[0].desc.block_size + 100
    _expect_einval("append slot beyond the cache",
                   lambda: _append_decode(st, s.shape.scale, sl2))

    say("[debug] copy_blocks: destination id past the end; negative ids are padding")
    nb = cache.desc.num_blocks
    _expect_einval("copy block id outside its cache", lambda: _copy(cache, [0, 1], [2, nb]))
    _expect_einval("copy block id outside its cache", lambda: _copy(cache, [nb + 1], [2]))
    _copy(cache, [0, -1], [-4, 2])
    say("[debug] copy_blocks: a destination written twice; a block both source and destination")
    _expect_einval("written twice", lambda: _copy(cache, [0, 1, 4], [2, 2, -1]))
    ids = lambda a: torch.tensor(a, dtype=torch.int32, device=q.device)  # noqa: E731
    _expect_einval("both a source and a destination",
                   lambda: pkv.copy_blocks(kc1, vc1, cache.desc, kc1, vc1, cache.desc,
                                           ids([3, 5]), ids([5, 7])))
    again()


def _bits_t(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int32 if t.element_size() == 4 else torch.int16)


def main(out_dir: str) -> int:
    say(f"[debug] library {os.path.basename(pkv.LIB_PATH)}")
    assert os.path.basename(pkv.LIB_PATH) == "libpkv_debug.so", pkv.LIB_PATH
    say("[debug] valid calls")
    np.savez(os.path.join(out_dir, "valid.npz"), **valid_outputs())
    broken_calls()
    say("[debug] all cases passed")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
