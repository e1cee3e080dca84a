"""Paged-cache state on the GPU, driven only through the libpkv C ABI.

``PagedCache`` owns one layer's k_cache / v_cache tensors, a host block
pool and the sequence bookkeeping, and loads K/V rows into the cache with
``pkv_append`` at the slots the pool hands out.  It is the host side of a
serving step ("LLM Inference: KV Cache, Batching & Scheduling", sections
"PagedAttention and vLLM", "Continuous batching (Orca)" and "Prefix
caching"): sequences are added, grow by appends, share prefix blocks (by
explicit sharing, by forking, or through the prefix cache), and are
released, their blocks returning to the pool at once.  A write into a
shared, partially filled block first copies it (pkv_copy_blocks).
"""
from __future__ import annotations

from typing import Iterable, Optional

import numpy as np
import torch

from . import BF16, F32, CacheDesc, Pool, Seqs, append, copy_blocks  # noqa: F401

# Quiet-NaN bit patterns written into every cache element before any append,
# so a read of an unused slot or block would surface in the output.
POISON_BITS = {F32: 0x7FC00000, BF16: 0x7FC0}


def torch_dtype(code: int):
    return torch.float32 if code == F32 else torch.bfloat16


def to_device_rows(rows: np.ndarray, code: int, device) -> torch.Tensor:
    """Host rows (float32, or bf16 bit patterns as uint16) -> device tensor."""
    if code == F32:
        t = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.float32))
    else:
        t = torch.from_numpy(np.ascontiguousarray(rows, dtype=np.uint16).view(np.int16))
        t = t.view(torch.bfloat16)
    return t.to(device, non_blocking=False)


class StepMetadata:
    """A decode step's metadata -- block tables, context lengths and the
    slots of the step's new tokens -- written by the host bookkeeping straight
    into pinned host memory and copied to the device with one asynchronous
    copy on the caller's stream ("LLM Inference: KV Cache, Batching &
    Scheduling", "PagedAttention and vLLM": the logical-to-physical map is
    kept by a host memory manager and changes every step).

    A ring of ``depth`` pinned buffers, each with its own device buffer: a
    pinned buffer is refilled only once the copy that last read it has
    completed (an event per buffer), so the host may run up to ``depth``
    steps ahead of the GPU.  A device buffer is overwritten only by a copy
    enqueued on the same stream after the kernels of the step that used it
    (stream order); steps staged with one StepMetadata must use one stream.
    """

    def __init__(self, max_seqs: int, stride: int, depth: int = 4, device="cuda"):
        self.max_seqs, self.stride = int(max_seqs), int(stride)
        n = self.max_seqs * (self.stride + 2)
        self.device = torch.device(device)
        self.host = [torch.empty(n, dtype=torch.int32).pin_memory() for _ in range(depth)]
        self.hostv = [h.numpy() for h in self.host]
        self.dev = [torch.empty(n, dtype=torch.int32, device=self.device) for _ in range(depth)]
        self.events = [torch.cuda.Event() for _ in range(depth)]
        self.pending = [False] * depth
        self.i = 0
        # One copy from every pinned buffer now: the first transfer out of a
        # freshly pinned buffer pays a one-time mapping cost that would
        # otherwise land on the first steps.
        for h, d in zip(self.host, self.dev):
            d.copy_(h, non_blocking=True)
        torch.cuda.current_stream(self.device).synchronize()

    def fill(self, seqs, seq_ids, append: bool = True):
        """Host part: the step's bookkeeping for ``seq_ids`` (one new token
        per sequence when ``append``: pkv_seqs_append_batch), then its block
        tables and lengths (pkv_seqs_fill), written into the next pinned
        buffer.  Returns a handle for upload()."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        B, W = len(ids), self.stride
        if B > self.max_seqs:
            raise ValueError(f"{B} sequences, room for {self.max_seqs}")
        k = self.i
        self.i = (self.i + 1) % len(self.host)
        if self.pending[k]:
            self.events[k].synchronize()
        hv = self.hostv[k]
        lens = hv[B:2 * B]
        if append:
            seqs.append_batch(ids, out=hv[:B])
        seqs.fill(ids, W, out=(hv[2 * B:2 * B + B * W], lens))
        return (k, B, append, int(lens.max()) if B else 0)

    def upload(self, handle, stream=None, timing=None):
        """Device part: one non-blocking copy of the filled buffer on
        ``stream`` (default: the current stream).  ``timing``: an optional
        pair of timing events recorded right before and after the copy.
        Returns device (tables [B][stride], lens [B], slots [B] or None) and
        the host maximum length."""
        k, B, append, max_len = handle
        W = self.stride
        used = 2 * B + B * W
        st = stream if stream is not None else torch.cuda.current_stream(self.device)
        with torch.cuda.stream(st):
            if timing:
                timing[0].record(st)
            self.dev[k][:used].copy_(self.host[k][:used], non_blocking=True)
            if timing:
                timing[1].record(st)
            self.events[k].record(st)
        self.pending[k] = True
        d = self.dev[k]
        return (d[2 * B:used].view(B, W), d[B:2 * B], d[:B] if append else None, max_len)

    def stage(self, seqs, seq_ids, append: bool = True, stream=None):
        """fill() then upload()."""
        return self.upload(self.fill(seqs, seq_ids, append), stream)


class PagedCache:
    """One layer's paged K/V cache plus its host-side block bookkeeping."""

    def __init__(self, num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                 dtype: int, device="cuda", pool_seed: int = 0, poison: Optional[int] = None):
        self.desc = CacheDesc(int(num_blocks), int(num_kv_heads), int(block_size), int(head_dim),
                              int(dtype))
        self.device = torch.device(device)
        shape = self.desc.cache_shape()
        bits = POISON_BITS[dtype] if poison is None else poison
        if dtype == F32:
            fill = torch.tensor(bits, dtype=torch.int64).to(torch.int32)
            self.k_cache = torch.full(shape, int(fill), dtype=torch.int32, device=self.device)
            self.k_cache = self.k_cache.view(torch.float32)
        else:
            v16 = bits - 0x10000 if bits >= 0x8000 else bits
            self.k_cache = torch.full(shape, v16, dtype=torch.int16, device=self.device)
            self.k_cache = self.k_cache.view(torch.bfloat16)
        self.v_cache = self.k_cache.clone()
        self.pool = Pool(num_blocks, pool_seed)
        self.seqs = Seqs(self.pool, block_size)
        self.stream = None

    @property
    def dtype(self) -> int:
        return self.desc.dtype

    def write(self, slots: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray) -> None:
        """pkv_append of host rows [T][Hkv][D] into the given slots."""
        if len(slots) == 0:
            return
        s = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int32)).to(self.device)
        k = to_device_rows(k_rows, self.dtype, self.device)
        v = to_device_rows(v_rows, self.dtype, self.device)
        append(k, v, s, self.k_cache, self.v_cache, self.desc)

    def add_sequences(self, seq_ids: Iterable[int], lens, k_rows: np.ndarray,
                      v_rows: np.ndarray) -> np.ndarray:
        """Add sequences holding lens[i] rows each (rows concatenated in
        k_rows / v_rows); returns the slots the rows were written to."""
        slots = []
        for sid, L in zip(seq_ids, lens):
            self.seqs.add(int(sid))
            slots.append(self.seqs.append(int(sid), int(L)))
        slots = np.concatenate(slots) if slots else np.zeros(0, dtype=np.int32)
        self.write(slots, k_rows, v_rows)
        return slots

    def add_shared(self, seq_id: int, src_id: int, num_tokens: int) -> None:
        self.seqs.add_shared(int(seq_id), int(src_id), int(num_tokens))

    def extend(self, seq_id: int, k_rows: np.ndarray, v_rows: np.ndarray) -> np.ndarray:
        slots = self.seqs.append(int(seq_id), len(k_rows))
        self.write(slots, k_rows, v_rows)
        return slots

    def copy(self, copies) -> None:
        """pkv_copy_blocks for a list of (src_block, dst_block) pairs."""
        if not copies:
            return
        ids = torch.tensor(np.asarray(copies, dtype=np.int32).T.copy(), device=self.device)
        copy_blocks(self.k_cache, self.v_cache, self.desc, self.k_cache, self.v_cache, self.desc,
                    ids[0].contiguous(), ids[1].contiguous())

    def fork(self, seq_id: int, src_id: int) -> None:
        self.seqs.fork(int(seq_id), int(src_id))

    def extend_cow(self, seq_id: int, k_rows: np.ndarray, v_rows: np.ndarray) -> np.ndarray:
        """Append rows with copy-on-write of a shared partial last block."""
        slots, copies = self.seqs.append_cow(int(seq_id), len(k_rows))
        self.copy(copies)
        self.write(slots, k_rows, v_rows)
        return slots

    def step_cow(self, seq_ids, k_rows: np.ndarray, v_rows: np.ndarray):
        """One token for each sequence (a decode step) with copy-on-write.
        Returns (slots, copies)."""
        slots, copies = self.seqs.append_batch_cow(list(seq_ids))
        self.copy(copies)
        self.write(slots, k_rows, v_rows)
        return slots, copies

    def attach_swap(self, num_blocks: int) -> None:
        """A pinned-host swap area of num_blocks blocks (same block shape)
        with its own pool of slots."""
        d = self.desc
        self.swap_desc = CacheDesc(int(num_blocks), d.num_kv_heads, d.block_size, d.head_dim,
                                   d.dtype)
        shape = self.swap_desc.cache_shape()
        self.swap_k = torch.zeros(shape, dtype=torch_dtype(d.dtype)).pin_memory()
        self.swap_v = torch.zeros(shape, dtype=torch_dtype(d.dtype)).pin_memory()
        self.swap_pool = Pool(int(num_blocks), 0)

    def _copy_pairs(self, pairs, to_host: bool) -> None:
        if not pairs:
            return
        ids = torch.tensor(np.asarray(pairs, dtype=np.int32).T.copy(), device=self.device)
        if to_host:
            copy_blocks(self.k_cache, self.v_cache, self.desc, self.swap_k, self.swap_v,
                        self.swap_desc, ids[0].contiguous(), ids[1].contiguous())
        else:
            copy_blocks(self.swap_k, self.swap_v, self.swap_desc, self.k_cache, self.v_cache,
                        self.desc, ids[0].contiguous(), ids[1].contiguous())

    def swap_out(self, seq_id: int):
        """Preempt a sequence by moving its private blocks to the swap area."""
        pairs = self.seqs.swap_out(int(seq_id), self.swap_pool)
        self._copy_pairs(pairs, to_host=True)
        return pairs

    def swap_in(self, seq_id: int):
        pairs = self.seqs.swap_in(int(seq_id))
        self._copy_pairs(pairs, to_host=False)
        return pairs

    def admit_cached(self, seq_id: int, tokens) -> int:
        """New sequence for a prompt, reusing cached prefix blocks; returns
        the number of prompt tokens whose KV is already in the cache."""
        return self.seqs.add_cached(int(seq_id), tokens)

    def register(self, seq_id: int, tokens) -> None:
        """Record in the prefix cache that the sequence holds these tokens."""
        self.seqs.cache(int(seq_id), tokens)

    def release(self, seq_id: int) -> None:
        self.seqs.release(int(seq_id))

    def tables(self, seq_ids, stride: Optional[int] = None):
        """Device block tables [n][stride] and context lengths [n] (int32),
        and the host maximum length."""
        ids = list(seq_ids)
        if stride is None:
            stride = max(1, max((len(self.seqs.block_ids(i)) for i in ids), default=1))
        tab, lens = self.seqs.fill(ids, stride)
        max_len = int(lens.max()) if len(lens) else 0
        return (torch.from_numpy(tab).to(self.device), torch.from_numpy(lens.copy()).to(self.device),
                max_len)
