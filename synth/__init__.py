"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This module draws random numbers and describes workload shapes; it holds none
of the method's arithmetic (no attention, no paging, no slot math).  Every
draw comes from ``numpy.random.default_rng([config_id, stream, *sub])`` so a
(config, stream) pair always reproduces the same values.

Streams: 0 lengths, 1 pool free-list seed, 2 queries, 3 keys, 4 values,
5 continuous-batching churn, 6 prefix rows (shared prefix of config 4).

Values are N(0, 1) float32; bf16 workloads round them to bf16 by
round-to-nearest-even on the host and carry the 16-bit patterns as uint16.

Workload shapes follow the pages: 8 KV heads x head_dim 128 x 2-byte values
("LLM Inference: KV Cache, Batching & Scheduling", "The KV cache" table),
16- or 32-token blocks (same page, "PagedAttention and vLLM"; the
"LLM Inference Engineering" summary, section 2), 512-token prefill chunks
("Chunked prefill"), a 2048-token shared prompt ("Prefix caching").
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np

S_LENS, S_POOL, S_Q, S_K, S_V, S_CHURN, S_PREFIX = range(7)


def rng(config_id: int, stream: int, *sub: int) -> np.random.Generator:
    return np.random.default_rng([int(config_id), int(stream), *[int(s) for s in sub]])


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest even.
    Inputs here are finite draws; NaN/inf are not expected."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(g: np.random.Generator, shape, dtype: str) -> np.ndarray:
    x = g.standard_normal(size=shape, dtype=np.float32)
    if dtype == "f32":
        return x
    if dtype == "bf16":
        return bf16_bits(x)
    raise ValueError(dtype)


def elem_size(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


# Poison written into every cache byte before any append (quiet NaN), so a
# read of an unused slot or block shows up in the output.
POISON_F32 = 0x7FC00000
POISON_BF16 = 0x7FC0


@dataclass
class Shape:
    """Attention shape of one workload."""
    Hq: int
    Hkv: int
    D: int
    dtype: str          # "f32" or "bf16"
    block_size: int
    scale: float

    @property
    def elem(self) -> int:
        return elem_size(self.dtype)


@dataclass
class DecodeBatch:
    """One decode step's logical inputs.

    ``lens[b]`` is the context the query of sequence b attends, the token
    appended this step included; ``k``/``v`` hold every sequence's rows in
    append order, concatenated ([sum lens][Hkv][D]); the last row of each
    sequence is the one appended in the step.
    """
    cfg_id: int
    name: str
    shape: Shape
    lens: np.ndarray            # int64 [B]
    q: np.ndarray               # [B][Hq][D]
    k: np.ndarray               # [sum lens][Hkv][D]
    v: np.ndarray
    pool_blocks: int
    pool_seed: int
    prefix_len: int = 0         # config 4: leading tokens shared by all sequences

    @property
    def B(self) -> int:
        return len(self.lens)

    def seq_start(self) -> np.ndarray:
        st = np.zeros(self.B + 1, dtype=np.int64)
        np.cumsum(self.lens, out=st[1:])
        return st


def _pool_seed(cfg_id: int) -> int:
    return int(rng(cfg_id, S_POOL).integers(1, 2**62))


def _uniform_int(g, lo, hi, n):
    """Inclusive integer uniform on [lo, hi]."""
    return g.integers(lo, hi + 1, size=n, dtype=np.int64)


def _pool_size(lens, bs, factor=1.2, extra=0, shared_blocks=0):
    need = int(np.sum((np.asarray(lens) + bs - 1) // bs)) + shared_blocks
    return int(np.ceil(factor * need)) + extra


def _draw_kv(cfg_id, rows, shape, sub=()):
    k = normal(rng(cfg_id, S_K, *sub), (rows, shape.Hkv, shape.D), shape.dtype)
    v = normal(rng(cfg_id, S_V, *sub), (rows, shape.Hkv, shape.D), shape.dtype)
    return k, v


def _draw_q(cfg_id, B, shape, sub=()):
    return normal(rng(cfg_id, S_Q, *sub), (B, shape.Hq, shape.D), shape.dtype)


# ---------------------------------------------------------------------------
# The five workloads.  ``batch`` shrinks B for fast parity runs while keeping
# the length distribution; None keeps the full size.

def cfg1(B: Optional[int] = None) -> DecodeBatch:
    """Tiny paged decode: 8 q heads = 8 KV heads, d64, fp32, 16-token blocks,
    128-block pool in a seeded order; pre-step lengths U[1,256], one token
    appended per sequence, so the step attends length + 1."""
    shape = Shape(Hq=8, Hkv=8, D=64, dtype="f32", block_size=16, scale=1.0 / 8.0)
    B = 4 if B is None else B
    lens = _uniform_int(rng(1, S_LENS), 1, 256, B) + 1
    k, v = _draw_kv(1, int(lens.sum()), shape)
    return DecodeBatch(1, "tiny-f32-d64", shape, lens, _draw_q(1, B, shape), k, v,
                       pool_blocks=128, pool_seed=_pool_seed(1))


def cfg2(B: Optional[int] = None) -> DecodeBatch:
    """Llama-70B-shaped layer: 64 q / 8 KV heads, d128, bf16, 16-token blocks,
    32 sequences, lengths U[512,4096], pool 1.2x need in shuffled order."""
    shape = Shape(Hq=64, Hkv=8, D=128, dtype="bf16", block_size=16,
                  scale=1.0 / np.sqrt(128.0))
    full = _uniform_int(rng(2, S_LENS), 512, 4096, 32)
    lens = full if B is None else full[:B]
    k, v = _draw_kv(2, int(lens.sum()), shape)
    return DecodeBatch(2, "llama70b-bf16-bs16", shape, lens, _draw_q(2, len(lens), shape), k, v,
                       pool_blocks=_pool_size(lens, 16), pool_seed=_pool_seed(2))


CFG3_SIGMA = 1.0          # log-normal sigma; the workload fixes only the median (1024)
CFG3_FINISH_FRAC = 0.10   # sequences finishing per step
CFG3_NEW_LO, CFG3_NEW_HI = 16, 128


def cfg3_initial(B: Optional[int] = None) -> DecodeBatch:
    """Continuous-batching step: 64/8 heads, d128, bf16, 32-token blocks,
    256 sequences, pre-step lengths log-normal (median 1024, sigma 1.0)
    clipped to [16, 8192], one token appended per step."""
    shape = Shape(Hq=64, Hkv=8, D=128, dtype="bf16", block_size=32,
                  scale=1.0 / np.sqrt(128.0))
    nb = 256 if B is None else B
    g = rng(3, S_LENS)
    raw = g.lognormal(mean=np.log(1024.0), sigma=CFG3_SIGMA, size=256)
    pre = np.clip(np.rint(raw), 16, 8192).astype(np.int64)[:nb]
    lens = pre + 1
    k, v = _draw_kv(3, int(lens.sum()), shape)
    return DecodeBatch(3, "contbatch-bf16-bs32", shape, lens, _draw_q(3, nb, shape), k, v,
                       pool_blocks=_pool_size(lens + 16, 32, extra=256),
                       pool_seed=_pool_seed(3))


@dataclass
class ChurnEvent:
    """Between step ``step`` and step+1: sequences at batch positions
    ``finished`` end; each is replaced in place by a new sequence with
    ``new_lens[i]`` tokens whose rows are ``new_k[i]``/``new_v[i]``."""
    step: int
    finished: np.ndarray
    new_lens: np.ndarray
    new_k: List[np.ndarray] = field(default_factory=list)
    new_v: List[np.ndarray] = field(default_factory=list)


def cfg3_step_rows(step: int, B: int, shape: Shape):
    """K/V rows appended by every sequence at decode step ``step`` (>= 1) and
    that step's queries."""
    k, v = _draw_kv(3, B, shape, sub=(step,))
    return k, v, _draw_q(3, B, shape, sub=(step,))


def cfg3_churn(step: int, B: int, shape: Shape) -> ChurnEvent:
    g = rng(3, S_CHURN, step)
    n = int(round(CFG3_FINISH_FRAC * B))
    fin = np.sort(g.choice(B, size=n, replace=False)).astype(np.int64)
    new = _uniform_int(g, CFG3_NEW_LO, CFG3_NEW_HI, n)
    ev = ChurnEvent(step, fin, new)
    for i, L in enumerate(new):
        k, v = _draw_kv(3, int(L), shape, sub=(1000 + step, i))
        ev.new_k.append(k)
        ev.new_v.append(v)
    return ev


CFG4_PREFIX = 2048


def cfg4(B: Optional[int] = None) -> DecodeBatch:
    """Prefix sharing: 128 sequences share one 2048-token prefix (the same
    physical blocks) followed by a private suffix of U[64,512] tokens; 64/8
    heads, d128, bf16, 16-token blocks.  ``k``/``v`` hold the fully duplicated
    logical rows (prefix rows repeated per sequence)."""
    shape = Shape(Hq=64, Hkv=8, D=128, dtype="bf16", block_size=16,
                  scale=1.0 / np.sqrt(128.0))
    nb = 128 if B is None else B
    suf = _uniform_int(rng(4, S_LENS), 64, 512, 128)[:nb]
    lens = suf + CFG4_PREFIX
    pk = normal(rng(4, S_PREFIX, 0), (CFG4_PREFIX, shape.Hkv, shape.D), shape.dtype)
    pv = normal(rng(4, S_PREFIX, 1), (CFG4_PREFIX, shape.Hkv, shape.D), shape.dtype)
    sk, sv = _draw_kv(4, int(suf.sum()), shape)
    ks, vs, o = [], [], 0
    for L in suf:
        ks += [pk, sk[o:o + L]]
        vs += [pv, sv[o:o + L]]
        o += int(L)
    k = np.concatenate(ks)
    v = np.concatenate(vs)
    pool = _pool_size(suf, 16, shared_blocks=CFG4_PREFIX // 16)
    return DecodeBatch(4, "prefix-share-bf16-bs16", shape, lens, _draw_q(4, nb, shape), k, v,
                       pool_blocks=pool, pool_seed=_pool_seed(4), prefix_len=CFG4_PREFIX)


@dataclass
class PrefillBatch:
    """Chunked-prefill inputs: sequence b holds ``prior[b]`` cached tokens and
    appends a chunk of ``chunk[b]`` tokens, whose queries are the rows
    ``query_start[b] .. query_start[b+1]`` of ``q``.  ``k``/``v`` hold every
    sequence's rows (prior + chunk) in order."""
    shape: Shape
    prior: np.ndarray           # int64 [S]
    chunk: np.ndarray           # int64 [S]
    q: np.ndarray               # [sum chunk][Hq][D]
    k: np.ndarray               # [sum(prior + chunk)][Hkv][D]
    v: np.ndarray
    pool_blocks: int
    pool_seed: int

    @property
    def lens(self) -> np.ndarray:
        return self.prior + self.chunk

    @property
    def query_start(self) -> np.ndarray:
        qs = np.zeros(len(self.chunk) + 1, dtype=np.int64)
        np.cumsum(self.chunk, out=qs[1:])
        return qs


CFG5_CHUNK = 512


def cfg5(S: Optional[int] = None, D: Optional[int] = None, n_decode: Optional[int] = None):
    """Chunked prefill mixed with decode: 4 sequences prefill a 512-token
    chunk over prior context U[0,7680] (causal), and 64 decode sequences with
    pre-step context U[256,8192] + 1 appended; 64/8 heads, d128, bf16,
    16-token blocks.  Returns (PrefillBatch, DecodeBatch)."""
    shape = Shape(Hq=64, Hkv=8, D=128, dtype="bf16", block_size=16,
                  scale=1.0 / np.sqrt(128.0))
    ns = 4 if S is None else S
    g = rng(5, S_LENS)
    prior = _uniform_int(g, 0, 7680, 4)[:ns]
    chunk = np.full(ns, CFG5_CHUNK, dtype=np.int64)
    dec_pre = _uniform_int(g, 256, 8192, 64)
    nd = 64 if n_decode is None else n_decode
    dec_lens = dec_pre[:nd] + 1
    lens = prior + chunk
    pk, pv = _draw_kv(5, int(lens.sum()), shape, sub=(0,))
    pq = normal(rng(5, S_Q, 0), (int(chunk.sum()), shape.Hq, shape.D), shape.dtype)
    pool_p = _pool_size(lens, 16)
    pre = PrefillBatch(shape, prior, chunk, pq, pk, pv, pool_blocks=pool_p,
                       pool_seed=_pool_seed(5))
    dk, dv = _draw_kv(5, int(dec_lens.sum()), shape, sub=(1,))
    dq = normal(rng(5, S_Q, 1), (nd, shape.Hq, shape.D), shape.dtype)
    dec = DecodeBatch(5, "mixed-decode-bf16-bs16", shape, dec_lens, dq, dk, dv,
                      pool_blocks=_pool_size(dec_lens, 16), pool_seed=_pool_seed(5) ^ 1)
    return pre, dec


def custom_decode(cfg_id: int, lens, Hq: int, Hkv: int, D: int, dtype: str, block_size: int,
                  scale: Optional[float] = None, pool_factor: float = 1.5,
                  pool_extra: int = 8) -> DecodeBatch:
    """A decode batch of arbitrary shape for edge cases (seeded by cfg_id)."""
    shape = Shape(Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, block_size=block_size,
                  scale=(1.0 / np.sqrt(D)) if scale is None else scale)
    lens = np.asarray(lens, dtype=np.int64)
    k, v = _draw_kv(cfg_id, int(lens.sum()), shape)
    return DecodeBatch(cfg_id, f"custom-{cfg_id}", shape, lens, _draw_q(cfg_id, len(lens), shape),
                       k, v, pool_blocks=_pool_size(lens, block_size, pool_factor, pool_extra),
                       pool_seed=_pool_seed(cfg_id))


def custom_prefill(cfg_id: int, prior, chunk, Hq: int, Hkv: int, D: int, block_size: int,
                   dtype: str = "bf16", scale: Optional[float] = None) -> PrefillBatch:
    shape = Shape(Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, block_size=block_size,
                  scale=(1.0 / np.sqrt(D)) if scale is None else scale)
    prior = np.asarray(prior, dtype=np.int64)
    chunk = np.asarray(chunk, dtype=np.int64)
    lens = prior + chunk
    k, v = _draw_kv(cfg_id, int(lens.sum()), shape, sub=(0,))
    q = normal(rng(cfg_id, S_Q, 0), (int(chunk.sum()), Hq, D), dtype)
    return PrefillBatch(shape, prior, chunk, q, k, v,
                        pool_blocks=_pool_size(lens, block_size, 1.5, 8),
                        pool_seed=_pool_seed(cfg_id))
