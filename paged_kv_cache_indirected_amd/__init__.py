"""Python binding of libpkv: paged-KV attention on AMD MI355X (gfx950).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libpkv.so`` behind the C ABI declared in ``include/pkv.h``;
torch supplies device memory and streams.  There is no fallback: if the
library is not built, importing this package fails.

Calls mirror the C ABI names: ``append`` (pkv_append), ``decode``
(pkv_decode), ``append_decode`` (pkv_append_decode), ``decode_cascade``
(pkv_decode_cascade), ``prefill_chunk``
(pkv_prefill_chunk), ``copy_blocks`` (pkv_copy_blocks), ``Pool``
(pkv_pool_*) and ``Seqs`` (pkv_seqs_*).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKV_DEBUG=1 selects the debug build of the same library: every call that
# enqueues device work synchronises and returns PKV_EINVAL when a kernel found
# a device precondition violated (block id, context length, slot), PKV_EHIP
# on a device error.
DEBUG = os.environ.get("PKV_DEBUG", "") == "1"
LIB_PATH = os.path.join(_HERE, "libpkv_debug.so" if DEBUG else "libpkv.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m paged_kv_cache_indirected_amd.build` "
        "(no CPU fallback exists)")

# One HIP runtime per process: torch ships its own libamdhip64, and a library
# loaded before it would bind the system runtime instead, leaving two runtimes
# that do not share devices, memory or streams.  Importing torch first makes
# libpkv resolve the HIP runtime torch already loaded.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

OK, EINVAL, EUNSUPPORTED, ENOBLOCKS, ESTATE, EHIP = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1

_P = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64
_sz = ctypes.c_size_t


class CacheDescC(ctypes.Structure):
    _fields_ = [("num_blocks", _i32), ("num_kv_heads", _i32), ("block_size", _i32),
                ("head_dim", _i32), ("dtype", _i32)]


class SeqsStatsC(ctypes.Structure):
    _fields_ = [("num_seqs", _i32), ("blocks_referenced", _i64), ("blocks_in_use", _i32),
                ("tokens", _i64), ("slots_unused", _i64)]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_DESC = ctypes.POINTER(CacheDescC)
_sig("pkv_strerror", ctypes.c_char_p, ctypes.c_int)
_sig("pkv_last_error", ctypes.c_char_p)
_sig("pkv_abi_version", ctypes.c_int)
_sig("pkv_append", ctypes.c_int, _P, _P, _P, _i32, _P, _P, _DESC, _P)
_sig("pkv_copy_blocks", ctypes.c_int, _P, _P, _DESC, _P, _P, _DESC, _P, _P, _i32, _P)
_sig("pkv_decode_num_splits", _i32, _i32, _i32, _i32, _DESC)
_sig("pkv_decode_workspace_bytes", _sz, _i32, _i32, _i32, _i32, _DESC)
_sig("pkv_decode", ctypes.c_int, _P, _P, _P, _P, _i32, _P, _i32, _i32, _i32, ctypes.c_float, _P,
     _i32, _i32, _P, _sz, _DESC, _P)
_sig("pkv_decode_noalloc", ctypes.c_int, _P, _P, _P, _P, _i32, _P, _i32, _i32, _i32,
     ctypes.c_float, _P, _i32, _i32, _DESC, _P)
_sig("pkv_append_decode", ctypes.c_int, _P, _P, _P, _P, _P, _P, _P, _i32, _P, _i32, _i32, _i32,
     ctypes.c_float, _P, _i32, _i32, _P, _sz, _DESC, _P)
_sig("pkv_prefill_workspace_bytes", _sz, _i32, _i32, _i32, _DESC)
_sig("pkv_decode_cascade_workspace_bytes", _sz, _i32, _i32, _i32, _i32, _DESC)
_sig("pkv_decode_cascade", ctypes.c_int, _P, _P, _P, _P, _i32, _P, _i32, _P, _i32, _i32, _i32,
     ctypes.c_float, _P, _i32, _P, _sz, _DESC, _P)
_sig("pkv_prefill_chunk", ctypes.c_int, _P, _P, _i32, _i32, _P, _P, _P, _i32, _P, _i32, _i32,
     ctypes.c_float, _P, _i32, _P, _sz, _DESC, _P)
_sig("pkv_pool_create", _P, _i32, _u64)
_sig("pkv_pool_destroy", None, _P)
_sig("pkv_pool_alloc", ctypes.c_int, _P, _i32, _P)
_sig("pkv_pool_share", ctypes.c_int, _P, _i32, _P)
_sig("pkv_pool_release", ctypes.c_int, _P, _i32, _P)
_sig("pkv_pool_num_free", _i32, _P)
_sig("pkv_pool_num_cached", _i32, _P)
_sig("pkv_pool_num_blocks", _i32, _P)
_sig("pkv_pool_refcount", _i32, _P, _i32)
_sig("pkv_seqs_create", _P, _P, _i32)
_sig("pkv_seqs_destroy", None, _P)
_sig("pkv_seqs_add", ctypes.c_int, _P, _i64)
_sig("pkv_seqs_add_shared", ctypes.c_int, _P, _i64, _i64, _i32)
_sig("pkv_seqs_append", ctypes.c_int, _P, _i64, _i32, _P)
_sig("pkv_seqs_append_batch", ctypes.c_int, _P, _i32, _P, _P)
_sig("pkv_seqs_fork", ctypes.c_int, _P, _i64, _i64)
_sig("pkv_seqs_append_cow", ctypes.c_int, _P, _i64, _i32, _P, _P, _P, _P)
_sig("pkv_seqs_append_batch_cow", ctypes.c_int, _P, _i32, _P, _P, _P, _P, _P)
_sig("pkv_seqs_add_cached", _i32, _P, _i64, _P, _i32)
_sig("pkv_seqs_cache", ctypes.c_int, _P, _i64, _P, _i32)
_sig("pkv_seqs_swap_out", ctypes.c_int, _P, _i64, _P, _i32, _P, _P, _P)
_sig("pkv_seqs_swap_in", ctypes.c_int, _P, _i64, _i32, _P, _P, _P)
_sig("pkv_seqs_is_swapped", ctypes.c_int, _P, _i64)
_sig("pkv_seqs_release", ctypes.c_int, _P, _i64)
_sig("pkv_seqs_len", _i32, _P, _i64)
_sig("pkv_seqs_block_ids", _i32, _P, _i64, _i32, _P)
_sig("pkv_seqs_fill", ctypes.c_int, _P, _i32, _P, _P, _i32, _P)
_sig("pkv_seqs_stats_get", ctypes.c_int, _P, ctypes.POINTER(SeqsStatsC))


class StepPlanC(ctypes.Structure):
    _fields_ = [("decode_ids", _P), ("decode_slots", _P), ("chunk_ids", _P),
                ("chunk_prior", _P), ("chunk_len", _P), ("chunk_slots", _P),
                ("first_ids", _P), ("finished_ids", _P), ("preempted_ids", _P),
                ("n_decode", _i32), ("n_chunks", _i32), ("n_chunk_tokens", _i32),
                ("n_first", _i32), ("n_finished", _i32), ("n_preempted", _i32)]


_sig("pkv_sched_create", _P, _P, _P, _i32, _i32, _i32, _i32)
_sig("pkv_sched_destroy", None, _P)
_sig("pkv_sched_submit", ctypes.c_int, _P, _i64, _i32, _i32)
_sig("pkv_sched_step", ctypes.c_int, _P, ctypes.POINTER(StepPlanC))
_sig("pkv_sched_num_waiting", _i32, _P)
_sig("pkv_sched_num_running", _i32, _P)


class PkvError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = _lib.pkv_last_error().decode() or _lib.pkv_strerror(code).decode()
        super().__init__(f"{where}: {_lib.pkv_strerror(code).decode()} ({code}): {msg}")


def _check(rc: int, where: str) -> None:
    if rc != OK:
        raise PkvError(rc, where)


def strerror(code: int) -> str:
    return _lib.pkv_strerror(code).decode()


def abi_version() -> int:
    return int(_lib.pkv_abi_version())


@dataclass(frozen=True)
class CacheDesc:
    """Shape of one layer's cache.

    k_cache / v_cache each hold num_blocks x num_kv_heads tiles of
    block_size * head_dim elements of ``dtype`` (allocated here as
    [num_blocks][num_kv_heads][block_size][head_dim] for the sizes only).
    Inside a tile the order is not row-major: with E = 16 // element size,
    K element (token t, dim d) sits at ((d // E) * block_size + t) * E + d % E
    and V element (t, d) at ((t // 4) * head_dim + d) * 4 + t % 4 (the C
    header's pkv_k_elem_offset / pkv_v_elem_offset).  pkv_append writes this
    layout; fill a cache any other way only by the same offsets."""
    num_blocks: int
    num_kv_heads: int
    block_size: int
    head_dim: int
    dtype: int  # F32 or BF16

    def c(self) -> CacheDescC:
        return CacheDescC(self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim,
                          self.dtype)

    def cache_shape(self):
        return (self.num_blocks, self.num_kv_heads, self.block_size, self.head_dim)


# ---------------------------------------------------------------------------
# Tensor marshalling.

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name: str, dtype=None):
    """Device pointer of a contiguous GPU tensor (None passes NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _need(cond: bool, what: str) -> None:
    if not cond:
        raise ValueError(what)


def _cache_ok(t, desc: "CacheDesc", name: str) -> None:
    _need(t.numel() == desc.num_blocks * desc.num_kv_heads * desc.block_size * desc.head_dim,
          f"{name} does not match the cache descriptor {desc}")
    _need(_dtype_code(t) == desc.dtype, f"{name} dtype does not match the descriptor")


def _stream(stream) -> Optional[int]:
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def append(k, v, slot_mapping, k_cache, v_cache, desc: CacheDesc, stream=None) -> None:
    """pkv_append: copy k/v rows ([T][Hkv][D]) into the cache slots
    ``slot_mapping`` (int32 [T]; negative = skip)."""
    torch = _torch()
    T = int(slot_mapping.numel())
    row = desc.num_kv_heads * desc.head_dim
    _need(k.numel() == T * row and v.numel() == T * row, "k/v must be [T][Hkv][D]")
    _need(_dtype_code(k) == desc.dtype and _dtype_code(v) == desc.dtype, "k/v dtype")
    _cache_ok(k_cache, desc, "k_cache")
    _cache_ok(v_cache, desc, "v_cache")
    rc = _lib.pkv_append(_dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping", torch.int32),
                         T, _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                         ctypes.byref(desc.c()), _stream(stream))
    _check(rc, "pkv_append")


def copy_blocks(src_k, src_v, src_desc: CacheDesc, dst_k, dst_v, dst_desc: CacheDesc,
                src_ids, dst_ids, stream=None) -> None:
    """pkv_copy_blocks: block dst_ids[i] of (dst_k, dst_v) receives block
    src_ids[i] of (src_k, src_v).  The caches may be GPU tensors or pinned
    host tensors (device-accessible); the id lists are int32 GPU tensors."""
    torch = _torch()
    n = int(src_ids.numel())
    _need(int(dst_ids.numel()) == n, "src_ids and dst_ids differ in length")
    for t, d, name in ((src_k, src_desc, "src_k"), (src_v, src_desc, "src_v"),
                       (dst_k, dst_desc, "dst_k"), (dst_v, dst_desc, "dst_v")):
        _cache_ok(t, d, name)
        _need(t.is_contiguous() and (t.is_cuda or t.is_pinned()),
              f"{name} must be a contiguous GPU or pinned host tensor")
    rc = _lib.pkv_copy_blocks(src_k.data_ptr(), src_v.data_ptr(), ctypes.byref(src_desc.c()),
                              dst_k.data_ptr(), dst_v.data_ptr(), ctypes.byref(dst_desc.c()),
                              _dev(src_ids, "src_ids", torch.int32),
                              _dev(dst_ids, "dst_ids", torch.int32), n, _stream(stream))
    _check(rc, "pkv_copy_blocks")


def decode_num_splits(num_seqs: int, num_q_heads: int, max_context_len: int,
                      desc: CacheDesc) -> int:
    """pkv_decode_num_splits: the library's workgroups per KV head."""
    return int(_lib.pkv_decode_num_splits(num_seqs, num_q_heads, max_context_len,
                                          ctypes.byref(desc.c())))


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, max_context_len: int,
                           desc: CacheDesc, num_splits: int = 0) -> int:
    return int(_lib.pkv_decode_workspace_bytes(num_seqs, num_q_heads, max_context_len,
                                               num_splits, ctypes.byref(desc.c())))


def decode(q, k_cache, v_cache, block_tables, context_lens, scale: float, out, desc: CacheDesc,
           max_context_len: int, workspace=None, num_splits: int = 0, stream=None) -> None:
    """pkv_decode: out[b][h] = softmax(scale q[b][h] K^T) V over the paged
    context of sequence b.  ``workspace`` is a uint8 GPU tensor of at least
    ``decode_workspace_bytes(...)`` bytes."""
    torch = _torch()
    B, Hq, D = q.shape
    _need(D == desc.head_dim and _dtype_code(q) == desc.dtype, "q must be [B][Hq][head_dim]")
    _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    _need(block_tables.dim() == 2 and block_tables.shape[0] >= B, "block_tables must be [B][W]")
    _need(context_lens.numel() >= B, "context_lens must hold B entries")
    _cache_ok(k_cache, desc, "k_cache")
    _cache_ok(v_cache, desc, "v_cache")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.pkv_decode(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                         _dev(block_tables, "block_tables", torch.int32),
                         int(block_tables.shape[1]) if block_tables.dim() == 2 else 0,
                         _dev(context_lens, "context_lens", torch.int32), B, Hq,
                         int(max_context_len), float(scale), _dev(out, "out"), _dtype_code(out),
                         int(num_splits), _dev(workspace, "workspace"), ws_bytes,
                         ctypes.byref(desc.c()), _stream(stream))
    _check(rc, "pkv_decode")


# Bytes of partials pkv_decode_noalloc can hold (PKV_DECODE_NOALLOC_SCRATCH_BYTES).
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale: float, out,
                   desc: CacheDesc, max_context_len: int, num_splits: int = 0,
                   stream=None) -> None:
    """pkv_decode_noalloc: pkv_decode without a workspace, for callers
    that cannot allocate; the split partials live in the library's per-GPU
    scratch (calls that overlap on one GPU race)."""
    torch = _torch()
    B, Hq, D = q.shape
    _need(D == desc.head_dim and _dtype_code(q) == desc.dtype, "q must be [B][Hq][head_dim]")
    _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    _need(block_tables.dim() == 2 and block_tables.shape[0] >= B, "block_tables must be [B][W]")
    _need(context_lens.numel() >= B, "context_lens must hold B entries")
    _cache_ok(k_cache, desc, "k_cache")
    _cache_ok(v_cache, desc, "v_cache")
    rc = _lib.pkv_decode_noalloc(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                 _dev(block_tables, "block_tables", torch.int32),
                                 int(block_tables.shape[1]),
                                 _dev(context_lens, "context_lens", torch.int32), B, Hq,
                                 int(max_context_len), float(scale), _dev(out, "out"),
                                 _dtype_code(out), int(num_splits), ctypes.byref(desc.c()),
                                 _stream(stream))
    _check(rc, "pkv_decode_noalloc")


def append_decode(k_new, v_new, slot_mapping, q, k_cache, v_cache, block_tables, context_lens,
                  scale: float, out, desc: CacheDesc, max_context_len: int, workspace=None,
                  num_splits: int = 0, stream=None) -> None:
    """pkv_append_decode: a decode step's append (one row per sequence) and
    the decode, in one launch (plus the merge pass)."""
    torch = _torch()
    B, Hq, D = q.shape
    _need(D == desc.head_dim and _dtype_code(q) == desc.dtype, "q must be [B][Hq][head_dim]")
    _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    row = desc.num_kv_heads * desc.head_dim
    _need(k_new.numel() == B * row and v_new.numel() == B * row, "k_new/v_new must be [B][Hkv][D]")
    _need(_dtype_code(k_new) == desc.dtype and _dtype_code(v_new) == desc.dtype, "k_new/v_new dtype")
    _need(slot_mapping.numel() >= B, "slot_mapping must hold B entries")
    _need(block_tables.dim() == 2 and block_tables.shape[0] >= B, "block_tables must be [B][W]")
    _need(context_lens.numel() >= B, "context_lens must hold B entries")
    _cache_ok(k_cache, desc, "k_cache")
    _cache_ok(v_cache, desc, "v_cache")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.pkv_append_decode(_dev(k_new, "k_new"), _dev(v_new, "v_new"),
                                _dev(slot_mapping, "slot_mapping", torch.int32), _dev(q, "q"),
                                _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                                _dev(block_tables, "block_tables", torch.int32),
                                int(block_tables.shape[1]),
                                _dev(context_lens, "context_lens", torch.int32), B, Hq,
                                int(max_context_len), float(scale), _dev(out, "out"),
                                _dtype_code(out), int(num_splits), _dev(workspace, "workspace"),
                                ws_bytes, ctypes.byref(desc.c()), _stream(stream))
    _check(rc, "pkv_append_decode")


def decode_cascade_workspace_bytes(num_seqs: int, num_q_heads: int, prefix_len: int,
                                   max_context_len: int, desc: CacheDesc) -> int:
    return int(_lib.pkv_decode_cascade_workspace_bytes(int(num_seqs), int(num_q_heads),
                                                       int(prefix_len), int(max_context_len),
                                                       ctypes.byref(desc.c())))


def decode_cascade(q, k_cache, v_cache, prefix_blocks, prefix_len: int, block_tables,
                   context_lens, scale: float, out, desc: CacheDesc,
                   max_context_len: Optional[int] = None, workspace=None, stream=None) -> None:
    """pkv_decode_cascade: decode over a shared prefix (prefix_blocks, int32
    [prefix_len / block_size]) followed by each sequence's own blocks
    (block_tables [B][stride], context_lens [B] = own tokens)."""
    torch = _torch()
    B, Hq, D = (int(x) for x in q.shape)
    _need(D == desc.head_dim, "q head_dim does not match the descriptor")
    _cache_ok(k_cache, desc, "k_cache")
    _cache_ok(v_cache, desc, "v_cache")
    _need(block_tables.dim() == 2 and int(block_tables.shape[0]) == B, "block_tables must be [B][stride]")
    stride = int(block_tables.shape[1])
    if max_context_len is None:
        max_context_len = stride * desc.block_size
    nbytes = decode_cascade_workspace_bytes(B, Hq, prefix_len, max_context_len, desc)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    pb = _dev(prefix_blocks, "prefix_blocks", torch.int32) if prefix_len > 0 else None
    rc = _lib.pkv_decode_cascade(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), pb, int(prefix_len),
        _dev(block_tables, "block_tables", torch.int32), stride,
        _dev(context_lens, "context_lens", torch.int32), B, Hq, int(max_context_len),
        float(scale), _dev(out, "out"), _dtype_code(out), _dev(workspace, "workspace"),
        int(workspace.numel() * workspace.element_size()), ctypes.byref(desc.c()),
        _stream(stream))
    _check(rc, "pkv_decode_cascade")


def prefill_workspace_bytes(num_seqs: int, num_q_heads: int, max_query_len: int,
                            desc: CacheDesc) -> int:
    return int(_lib.pkv_prefill_workspace_bytes(num_seqs, num_q_heads, max_query_len,
                                                ctypes.byref(desc.c())))


def prefill_chunk(q, query_start_loc, k_cache, v_cache, block_tables, context_lens, scale: float,
                  out, desc: CacheDesc, max_query_len: int, max_context_len: int, workspace=None,
                  stream=None) -> None:
    """pkv_prefill_chunk: causal attention of each sequence's chunk rows over
    its paged context (the chunk already appended).  ``workspace`` (a uint8
    GPU tensor of ``prefill_workspace_bytes(...)`` bytes, or None) lets the
    library split the keys of a grid smaller than the device."""
    torch = _torch()
    S = int(query_start_loc.numel()) - 1
    _need(q.dim() == 3 and q.shape[2] == desc.head_dim and _dtype_code(q) == desc.dtype,
          "q must be [T][Hq][head_dim]")
    _need(tuple(out.shape) == tuple(q.shape), "out must have q's shape")
    _need(block_tables.dim() == 2 and block_tables.shape[0] >= S, "block_tables must be [S][W]")
    _need(context_lens.numel() >= S, "context_lens must hold S entries")
    _cache_ok(k_cache, desc, "k_cache")
    _cache_ok(v_cache, desc, "v_cache")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rc = _lib.pkv_prefill_chunk(_dev(q, "q"), _dev(query_start_loc, "query_start_loc", torch.int32),
                                S, int(max_query_len), _dev(k_cache, "k_cache"),
                                _dev(v_cache, "v_cache"),
                                _dev(block_tables, "block_tables", torch.int32),
                                int(block_tables.shape[1]) if block_tables.dim() == 2 else 0,
                                _dev(context_lens, "context_lens", torch.int32),
                                int(max_context_len), int(q.shape[1]), float(scale),
                                _dev(out, "out"), _dtype_code(out), _dev(workspace, "workspace"),
                                ws_bytes, ctypes.byref(desc.c()), _stream(stream))
    _check(rc, "pkv_prefill_chunk")


# ---------------------------------------------------------------------------
# Host pool and sequences.

def _i32buf(n: int):
    return (ctypes.c_int32 * max(n, 1))()


class Pool:
    """pkv_pool_*: physical block ids with reference counts."""

    def __init__(self, num_blocks: int, seed: int = 0):
        self._h = _lib.pkv_pool_create(int(num_blocks), int(seed) & (2**64 - 1))
        if not self._h:
            raise PkvError(EINVAL, "pkv_pool_create")

    def close(self) -> None:
        if self._h and _lib is not None:   # _lib is None during interpreter shutdown
            _lib.pkv_pool_destroy(self._h)
        self._h = None

    def __del__(self):
        self.close()

    @property
    def handle(self):
        return self._h

    def alloc(self, n: int):
        buf = _i32buf(n)
        _check(_lib.pkv_pool_alloc(self._h, int(n), buf), "pkv_pool_alloc")
        return list(buf[:n])

    def share(self, ids: Sequence[int]) -> None:
        buf = (ctypes.c_int32 * max(len(ids), 1))(*ids)
        _check(_lib.pkv_pool_share(self._h, len(ids), buf), "pkv_pool_share")

    def release(self, ids: Sequence[int]) -> None:
        buf = (ctypes.c_int32 * max(len(ids), 1))(*ids)
        _check(_lib.pkv_pool_release(self._h, len(ids), buf), "pkv_pool_release")

    @property
    def num_free(self) -> int:
        return int(_lib.pkv_pool_num_free(self._h))

    @property
    def num_cached(self) -> int:
        return int(_lib.pkv_pool_num_cached(self._h))

    @property
    def num_blocks(self) -> int:
        return int(_lib.pkv_pool_num_blocks(self._h))

    def refcount(self, block_id: int) -> int:
        return int(_lib.pkv_pool_refcount(self._h, int(block_id)))


class Seqs:
    """pkv_seqs_*: per-sequence lengths and block lists over a Pool."""

    def __init__(self, pool: Pool, block_size: int):
        self.pool = pool  # keeps the pool alive
        self.block_size = int(block_size)
        self._h = _lib.pkv_seqs_create(pool.handle, int(block_size))
        if not self._h:
            raise PkvError(EINVAL, "pkv_seqs_create")

    def close(self) -> None:
        if self._h and _lib is not None:
            _lib.pkv_seqs_destroy(self._h)
        self._h = None

    def __del__(self):
        self.close()

    def add(self, seq_id: int) -> None:
        _check(_lib.pkv_seqs_add(self._h, int(seq_id)), "pkv_seqs_add")

    def add_shared(self, seq_id: int, src_id: int, num_tokens: int) -> None:
        _check(_lib.pkv_seqs_add_shared(self._h, int(seq_id), int(src_id), int(num_tokens)),
               "pkv_seqs_add_shared")

    def append(self, seq_id: int, n: int):
        """Extend by n tokens; returns their slots (a numpy int32 array)."""
        import numpy as np
        out = np.empty(max(int(n), 1), dtype=np.int32)
        _check(_lib.pkv_seqs_append(self._h, int(seq_id), int(n), out.ctypes.data),
               "pkv_seqs_append")
        return out[:n]

    def append_batch(self, seq_ids, out=None):
        """One token for each listed sequence; returns the slots.  ``out``:
        an optional contiguous int32 array of at least len(seq_ids) entries
        (e.g. a view of pinned host memory) that receives them."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        if out is None:
            out = np.empty(max(len(ids), 1), dtype=np.int32)
        _need(out.dtype == np.int32 and out.flags.c_contiguous and out.size >= len(ids),
              "out must be a contiguous int32 array of len(seq_ids) entries")
        _check(_lib.pkv_seqs_append_batch(self._h, len(ids), ids.ctypes.data, out.ctypes.data),
               "pkv_seqs_append_batch")
        return out[:len(ids)]

    def fork(self, seq_id: int, src_id: int) -> None:
        _check(_lib.pkv_seqs_fork(self._h, int(seq_id), int(src_id)), "pkv_seqs_fork")

    def append_cow(self, seq_id: int, n: int):
        """Extend by n tokens with copy-on-write; returns (slots, copies),
        copies a list of (src_block, dst_block) pairs to copy first."""
        import numpy as np
        out = np.empty(max(int(n), 1), dtype=np.int32)
        cs, cd, nc = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        _check(_lib.pkv_seqs_append_cow(self._h, int(seq_id), int(n), out.ctypes.data,
                                        ctypes.byref(cs), ctypes.byref(cd), ctypes.byref(nc)),
               "pkv_seqs_append_cow")
        return out[:n], [(cs.value, cd.value)] if nc.value else []

    def append_batch_cow(self, seq_ids):
        """One token for each listed sequence with copy-on-write; returns
        (slots, copies)."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        n = len(ids)
        out = np.empty(max(n, 1), dtype=np.int32)
        cs = np.empty(max(n, 1), dtype=np.int32)
        cd = np.empty(max(n, 1), dtype=np.int32)
        nc = ctypes.c_int32()
        _check(_lib.pkv_seqs_append_batch_cow(self._h, n, ids.ctypes.data, out.ctypes.data,
                                              cs.ctypes.data, cd.ctypes.data, ctypes.byref(nc)),
               "pkv_seqs_append_batch_cow")
        return out[:n], list(zip(cs[:nc.value].tolist(), cd[:nc.value].tolist()))

    def add_cached(self, seq_id: int, tokens) -> int:
        """New sequence reusing the longest cached whole-block prefix of the
        prompt ``tokens``; returns the number of tokens reused."""
        import numpy as np
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        r = int(_lib.pkv_seqs_add_cached(self._h, int(seq_id), t.ctypes.data if len(t) else None,
                                         len(t)))
        if r < 0:
            raise PkvError(r, "pkv_seqs_add_cached")
        return r

    def cache(self, seq_id: int, tokens) -> None:
        """Register the sequence's full blocks as holding ``tokens``."""
        import numpy as np
        t = np.ascontiguousarray(tokens, dtype=np.int32)
        _check(_lib.pkv_seqs_cache(self._h, int(seq_id), t.ctypes.data if len(t) else None,
                                   len(t)), "pkv_seqs_cache")

    def swap_out(self, seq_id: int, host: Pool):
        """Move the blocks the sequence holds alone to slots of ``host``;
        returns the (device_block, host_slot) pairs to copy."""
        import numpy as np
        cap = max(len(self.block_ids(seq_id)), 1)
        dev = np.empty(cap, dtype=np.int32)
        hst = np.empty(cap, dtype=np.int32)
        n = ctypes.c_int32()
        _check(_lib.pkv_seqs_swap_out(self._h, int(seq_id), host.handle, cap, dev.ctypes.data,
                                      hst.ctypes.data, ctypes.byref(n)), "pkv_seqs_swap_out")
        # The host pool must outlive the swapped sequences: keep it referenced.
        self._host_pools = getattr(self, "_host_pools", {})
        self._host_pools[id(host)] = host
        return list(zip(dev[:n.value].tolist(), hst[:n.value].tolist()))

    def swap_in(self, seq_id: int):
        """Bring a swapped sequence back; returns the (host_slot,
        device_block) pairs to copy."""
        import numpy as np
        cap = max(len(self.block_ids(seq_id)), 1)
        dev = np.empty(cap, dtype=np.int32)
        hst = np.empty(cap, dtype=np.int32)
        n = ctypes.c_int32()
        _check(_lib.pkv_seqs_swap_in(self._h, int(seq_id), cap, hst.ctypes.data, dev.ctypes.data,
                                     ctypes.byref(n)), "pkv_seqs_swap_in")
        return list(zip(hst[:n.value].tolist(), dev[:n.value].tolist()))

    def is_swapped(self, seq_id: int) -> bool:
        r = int(_lib.pkv_seqs_is_swapped(self._h, int(seq_id)))
        if r < 0:
            raise PkvError(ESTATE, "pkv_seqs_is_swapped")
        return bool(r)

    def release(self, seq_id: int) -> None:
        _check(_lib.pkv_seqs_release(self._h, int(seq_id)), "pkv_seqs_release")

    def length(self, seq_id: int) -> int:
        return int(_lib.pkv_seqs_len(self._h, int(seq_id)))

    def block_ids(self, seq_id: int):
        n = int(_lib.pkv_seqs_block_ids(self._h, int(seq_id), 0, None))
        if n < 0:
            raise PkvError(n, "pkv_seqs_block_ids")
        buf = _i32buf(n)
        _lib.pkv_seqs_block_ids(self._h, int(seq_id), n, buf)
        return list(buf[:n])

    def fill(self, seq_ids, stride: int, out=None):
        """Block tables [n][stride] (padding -1) and context lengths [n], int32.
        ``out``: optional (tables, lens) contiguous int32 arrays to fill
        (e.g. views of pinned host memory)."""
        import numpy as np
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        if out is None:
            tables = np.empty((len(ids), int(stride)), dtype=np.int32)
            lens = np.empty(max(len(ids), 1), dtype=np.int32)
        else:
            tables, lens = out
            _need(tables.dtype == np.int32 and lens.dtype == np.int32 and
                  tables.flags.c_contiguous and lens.flags.c_contiguous and
                  tables.size >= len(ids) * int(stride) and lens.size >= len(ids),
                  "out must be contiguous int32 (tables [n][stride], lens [n]) arrays")
        _check(_lib.pkv_seqs_fill(self._h, len(ids), ids.ctypes.data, tables.ctypes.data,
                                  int(stride), lens.ctypes.data), "pkv_seqs_fill")
        return tables, lens[:len(ids)]

    def stats(self) -> dict:
        st = SeqsStatsC()
        _check(_lib.pkv_seqs_stats_get(self._h, ctypes.byref(st)), "pkv_seqs_stats_get")
        return {f: getattr(st, f) for f, _ in SeqsStatsC._fields_}


class Sched:
    """pkv_sched_*: token-budget step scheduler over a Pool and Seqs."""

    def __init__(self, pool: Pool, seqs: Seqs, token_budget: int, chunk_tokens: int,
                 max_running: int):
        import numpy as np
        self.pool, self.seqs = pool, seqs   # keep them alive
        self._h = _lib.pkv_sched_create(pool.handle, seqs._h, seqs.block_size, int(token_budget),
                                        int(chunk_tokens), int(max_running))
        if not self._h:
            raise PkvError(EINVAL, "pkv_sched_create")
        R, T = max(int(max_running), 1), max(int(token_budget), 1)
        self._a = {
            "decode_ids": np.empty(R, np.int64), "decode_slots": np.empty(R, np.int32),
            "chunk_ids": np.empty(R, np.int64), "chunk_prior": np.empty(R, np.int32),
            "chunk_len": np.empty(R, np.int32), "chunk_slots": np.empty(T, np.int32),
            "first_ids": np.empty(R, np.int64), "finished_ids": np.empty(R, np.int64),
            "preempted_ids": np.empty(R, np.int64),
        }
        self._plan = StepPlanC(*[self._a[f].ctypes.data for f, _ in StepPlanC._fields_[:9]])

    def close(self) -> None:
        if self._h and _lib is not None:
            _lib.pkv_sched_destroy(self._h)
        self._h = None

    def __del__(self):
        self.close()

    def submit(self, req_id: int, prompt_len: int, max_new_tokens: int) -> None:
        _check(_lib.pkv_sched_submit(self._h, int(req_id), int(prompt_len), int(max_new_tokens)),
               "pkv_sched_submit")

    def step(self) -> dict:
        """Plan one step; returns copies of the plan's arrays."""
        p = self._plan
        _check(_lib.pkv_sched_step(self._h, ctypes.byref(p)), "pkv_sched_step")
        a = self._a
        return {
            "decode_ids": a["decode_ids"][:p.n_decode].copy(),
            "decode_slots": a["decode_slots"][:p.n_decode].copy(),
            "chunk_ids": a["chunk_ids"][:p.n_chunks].copy(),
            "chunk_prior": a["chunk_prior"][:p.n_chunks].copy(),
            "chunk_len": a["chunk_len"][:p.n_chunks].copy(),
            "chunk_slots": a["chunk_slots"][:p.n_chunk_tokens].copy(),
            "first_ids": a["first_ids"][:p.n_first].copy(),
            "finished_ids": a["finished_ids"][:p.n_finished].copy(),
            "preempted_ids": a["preempted_ids"][:p.n_preempted].copy(),
        }

    @property
    def num_waiting(self) -> int:
        return int(_lib.pkv_sched_num_waiting(self._h))

    @property
    def num_running(self) -> int:
        return int(_lib.pkv_sched_num_running(self._h))
