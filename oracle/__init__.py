"""fp64 CPU oracle for paged-KV attention -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The product library never imports, links or calls it,
and it imports nothing from the product package.

The arithmetic lives in ``oracle.c`` (plain C, IEEE double, OpenMP over
(sequence, head) pairs).  This module only marshals numpy arrays into it.
Each function documents the page passage it follows; see ``oracle.c`` for the
definitions and the readings taken where the pages are silent.

Pins (tests/test_oracle_pins.py): brute force in 50-digit mpmath on tiny
inputs, closed forms (mean of V for q = 0, equal-V, two keys with a logit gap
of ln 3, one dominant logit), the exact length-1 case, the GQA head map, the
inclusive causal diagonal, the worked KV-sizing example printed on the
"LLM Inference: KV Cache, Batching & Scheduling" page, and a hand-written
append byte image.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "oracle.c")

F32 = 0
BF16 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (IEEE double, no fast-math) into liboracle.so."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", SRC_PATH, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    i32 = ctypes.c_int
    lib.oracle_decode.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, ctypes.c_double, P, P,
                                  i32, i32]
    lib.oracle_decode.restype = i32
    lib.oracle_decode_weights.argtypes = [i32, i32, i32, i32, i32, P, P, P, P,
                                          ctypes.c_double, i32, i32, P, P]
    lib.oracle_decode_weights.restype = i32
    lib.oracle_prefill.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, ctypes.c_double, P,
                                   P, i32, i32]
    lib.oracle_prefill.restype = i32
    lib.oracle_append.argtypes = [P, P, P, i32, i32, i32, i32, i32, ctypes.c_int64, P, P]
    lib.oracle_append.restype = i32
    lib.oracle_copy_blocks.argtypes = [P, P, ctypes.c_int64, P, P, ctypes.c_int64, P, P, i32, i32,
                                       i32, i32, i32]
    lib.oracle_copy_blocks.restype = i32
    lib.oracle_kv_bytes_per_layer.argtypes = [ctypes.c_int64] * 4
    lib.oracle_kv_bytes_per_layer.restype = ctypes.c_int64
    _lib = lib
    return lib


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:  # bf16 bit patterns
        return BF16
    raise TypeError(f"oracle takes float32 or bf16-as-uint16 arrays, got {a.dtype}")


def _c(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _seq_start(lens) -> np.ndarray:
    lens = np.asarray(lens, dtype=np.int64)
    st = np.zeros(len(lens) + 1, dtype=np.int64)
    np.cumsum(lens, out=st[1:])
    return st


def decode(q, k, v, lens, scale, pairs=None, threads: int = 0) -> np.ndarray:
    """Decode attention over logically contiguous K/V.

    Follows the "LLM Inference: KV Cache, Batching & Scheduling" page, section
    "The KV cache": the query attends the keys and values of all prior
    positions of its sequence (the token appended this step included).

    q: [B][Hq][D]; k, v: [sum(lens)][Hkv][D] (rows of sequence b contiguous,
    in append order); float32 or bf16 bit patterns (uint16).  Returns float64
    [B][Hq][D].  ``pairs`` (array of (b, h)) restricts the rows computed; the
    others stay NaN.
    """
    lib = _load()
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share one dtype")
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    st = _seq_start(lens)
    if st[-1] != k.shape[0] or k.shape != v.shape or k.shape[2] != D:
        raise ValueError("k/v rows do not match lens")
    out = np.full((B, Hq, D), np.nan, dtype=np.float64)
    pr = None
    n = 0
    if pairs is not None:
        pr = _c(np.asarray(pairs, dtype=np.int32).reshape(-1, 2))
        n = pr.shape[0]
    rc = lib.oracle_decode(B, Hq, Hkv, D, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(st), float(scale),
                           _ptr(out), _ptr(pr), n, int(threads))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return out


def decode_weights(q, k, v, lens, scale, b: int, h: int):
    """Softmax weights and output row of one decode row (b, h)."""
    lib = _load()
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    B, Hq, D = q.shape
    st = _seq_start(lens)
    L = int(st[b + 1] - st[b])
    w = np.zeros(max(L, 1), dtype=np.float64)
    row = np.zeros(D, dtype=np.float64)
    rc = lib.oracle_decode_weights(B, Hq, k.shape[1], D, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(st),
                                   float(scale), int(b), int(h), _ptr(w), _ptr(row))
    if rc != 0:
        raise ValueError("oracle_decode_weights rejected its arguments")
    return w[:L], row


def prefill(q, query_start, k, v, lens, scale, rows=None, threads: int = 0) -> np.ndarray:
    """Causal chunked-prefill attention.

    Follows the "LLM Inference: KV Cache, Batching & Scheduling" page, section
    "Chunked prefill": a prompt split into chunks attends exactly what the
    unsplit prompt would.  Row i of sequence b's chunk (C_b rows) attends keys
    0 .. lens[b] - C_b + i (the chunk is already in the sequence's K/V).

    q: [sum C][Hq][D]; query_start: [S+1] int; k, v as in ``decode``.
    Returns float64 [sum C][Hq][D]; ``rows`` (array of (token row, h))
    restricts the rows computed, the others stay NaN.
    """
    lib = _load()
    q, k, v = _c(q), _c(k), _c(v)
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k, v must share one dtype")
    T, Hq, D = q.shape
    Hkv = k.shape[1]
    qs = _c(np.asarray(query_start, dtype=np.int32))
    S = len(qs) - 1
    if qs[-1] != T:
        raise ValueError("query_start does not match q")
    st = _seq_start(lens)
    out = np.full((T, Hq, D), np.nan, dtype=np.float64)
    pr = None
    n = 0
    if rows is not None:
        pr = _c(np.asarray(rows, dtype=np.int32).reshape(-1, 2))
        n = pr.shape[0]
    rc = lib.oracle_prefill(S, Hq, Hkv, D, dt, _ptr(q), _ptr(qs), _ptr(k), _ptr(v), _ptr(st),
                            float(scale), _ptr(out), _ptr(pr), n, int(threads))
    if rc != 0:
        raise ValueError("oracle_prefill rejected its arguments")
    return out


def append(k, v, slots, k_cache: np.ndarray, v_cache: np.ndarray, block_size: int) -> None:
    """KV append into host copies of the caches, in place.

    Follows the "LLM Inference: KV Cache, Batching & Scheduling" page, section
    "The KV cache" (the new token's K and V are appended each step).  Caches
    are [num_blocks][Hkv] tiles of block_size x D elements; slot s -> block
    s // block_size, offset s % block_size; negative slots are skipped.
    Inside a tile (the layout is a reading: the pages fix none) K element
    (t, d) sits at ((d // E) * bs + t) * E + d % E, E = 16 // element size,
    and V element (t, d) at ((t // 4) * D + d) * 4 + t % 4.
    """
    lib = _load()
    k, v = _c(k), _c(v)
    slots = _c(np.asarray(slots, dtype=np.int32))
    T, Hkv, D = k.shape
    if not (k_cache.flags.c_contiguous and v_cache.flags.c_contiguous):
        raise ValueError("caches must be contiguous")
    nb = k_cache.shape[0]
    rc = lib.oracle_append(_ptr(k), _ptr(v), _ptr(slots), T, Hkv, D, k.dtype.itemsize,
                           int(block_size), nb, _ptr(k_cache), _ptr(v_cache))
    if rc != 0:
        raise ValueError("oracle_append: slot out of range or bad arguments")


def tile_index(t: int, d: int, block_size: int, head_dim: int, elem_size: int):
    """(K index, V index) of element (token offset t, dim d) inside one
    (block, head) tile, in elements -- the layout ``append`` writes."""
    E = 16 // elem_size
    return ((d // E) * block_size + t) * E + d % E, ((t // 4) * head_dim + d) * 4 + t % 4


def copy_blocks(src_k, src_v, dst_k: np.ndarray, dst_v: np.ndarray, src_ids, dst_ids) -> None:
    """Block copy between host copies of two caches (may be the same arrays),
    in place: block dst_ids[i] of dst receives block src_ids[i] of src, pairs
    in order, a pair with an id outside its cache skipped.

    Sequences with an identical prefix share its pages (the "LLM Inference
    Engineering" summary, section 2); copying a shared block before a sharer
    writes into it is the reading taken where the pages are silent.
    """
    lib = _load()
    src_ids = _c(np.asarray(src_ids, dtype=np.int32))
    dst_ids = _c(np.asarray(dst_ids, dtype=np.int32))
    if src_ids.shape != dst_ids.shape:
        raise ValueError("id lists differ in length")
    for a in (src_k, src_v, dst_k, dst_v):
        if not a.flags.c_contiguous or a.ndim != 4:
            raise ValueError("caches must be contiguous [num_blocks][Hkv][bs][D]")
    if src_k.shape[1:] != dst_k.shape[1:] or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination blocks differ")
    _, Hkv, bs, D = src_k.shape
    rc = lib.oracle_copy_blocks(_ptr(src_k), _ptr(src_v), src_k.shape[0], _ptr(dst_k),
                                _ptr(dst_v), dst_k.shape[0], _ptr(src_ids), _ptr(dst_ids),
                                len(src_ids), Hkv, bs, D, src_k.dtype.itemsize)
    if rc != 0:
        raise ValueError("oracle_copy_blocks rejected its arguments")


def reusable_prefix_tokens(prompt, cached_prompts, block_size: int) -> int:
    """Tokens of ``prompt`` a prefix cache can serve from earlier prompts.

    The "LLM Inference: KV Cache, Batching & Scheduling" page, section
    "Prefix caching": a prefix's KV is computed once and later requests pay
    only for the tokens after it.  Readings: KV is cached per whole block, a
    block is reusable only if every token up to its end matches (its KV
    depends on the whole prefix), and at least one prompt token is always
    left to compute.  So the answer is the longest common prefix with any
    earlier prompt, rounded down to whole blocks, capped at
    (len(prompt) - 1) // block_size blocks.
    """
    best = 0
    for c in cached_prompts:
        k = 0
        while k < min(len(prompt), len(c)) and prompt[k] == c[k]:
            k += 1
        best = max(best, k // block_size)
    cap = (len(prompt) - 1) // block_size if len(prompt) > 0 else 0
    return min(best, cap) * block_size


def kv_bytes_per_layer(seq_len: int, num_kv_heads: int, head_dim: int, elem_size: int) -> int:
    """Per-layer KV bytes, the memory-cost formula of the "LLM Inference: KV
    Cache, Batching & Scheduling" page, section "The KV cache"."""
    return int(_load().oracle_kv_bytes_per_layer(seq_len, num_kv_heads, head_dim, elem_size))
