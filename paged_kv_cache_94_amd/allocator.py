"""Python binding of the host block allocator (include/pa_alloc.h).

Argument marshalling only: the allocator itself is C++ in libpa.so. Inputs
and outputs are numpy arrays; slot ids feed ``cache_write`` and block tables
and lengths feed ``decode`` / ``verify`` once copied to the GPU.
"""

from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _lib


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class BlockAllocator:
    """Blocks on demand, release at the end of a sequence, prefix caching of complete blocks."""

    def __init__(self, num_blocks: int, block_size: int = 16, prefix_cache: bool = True, lib=None):
        # lib: libpa.so (default), or another build of the allocator's host sources with the same
        # signatures bound (_lib.bind_host); the host-sanitizer test passes one.
        self._lib = lib or _lib.load()
        h = ctypes.c_void_p()
        self._check(self._lib.pa_alloc_create(int(num_blocks), int(block_size), int(bool(prefix_cache)),
                                             ctypes.byref(h)))
        self._h = h
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)

    def _check(self, rc: int) -> None:
        _lib.check(rc, self._lib)

    def close(self) -> None:
        if getattr(self, "_h", None):
            self._lib.pa_alloc_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()

    def add(self, seq_id: int, ring_blocks: int = 0) -> None:
        """Start a sequence; ring_blocks > 0 makes it a ring of that many blocks (window layers)."""
        if ring_blocks:
            self._check(self._lib.pa_alloc_add_ring(self._h, int(seq_id), int(ring_blocks)))
        else:
            self._check(self._lib.pa_alloc_add(self._h, int(seq_id)))

    def append(self, seq_id: int, n: int, tokens: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, int]:
        """Grow a sequence by n tokens: (slot ids, -1 where cached; number of cached leading tokens)."""
        toks = None if tokens is None else _i32(tokens)
        if toks is not None and toks.size != n:
            raise ValueError("tokens must hold n ids")
        slots = np.empty(max(n, 0), dtype=np.int64)
        cached = ctypes.c_int32(0)
        self._check(self._lib.pa_alloc_append(self._h, int(seq_id), int(n), _p(toks), _p(slots),
                                             ctypes.byref(cached)))
        return slots, cached.value

    def append_batch(self, seq_ids: Sequence[int], counts: Sequence[int],
                     tokens: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
        """Grow several sequences in order: (concatenated slot ids, cached count per sequence)."""
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        cnt = _i32(counts)
        total = int(cnt.sum()) if cnt.size else 0
        toks = None if tokens is None else _i32(tokens)
        if toks is not None and toks.size != total:
            raise ValueError("tokens must hold sum(counts) ids")
        slots = np.empty(total, dtype=np.int64)
        cached = np.zeros(ids.size, dtype=np.int32)
        done = ctypes.c_int32(0)
        rc = self._lib.pa_alloc_append_batch(self._h, int(ids.size), _p(ids), _p(cnt), _p(toks), _p(slots),
                                             _p(cached), ctypes.byref(done))
        if rc != _lib.PA_OK:
            err = _lib.PaError(rc, self._lib.pa_last_error().decode())
            err.done = done.value
            raise err
        return slots, cached

    def release(self, seq_id: int) -> None:
        self._check(self._lib.pa_alloc_release(self._h, int(seq_id)))

    def num_free(self) -> int:
        return int(self._lib.pa_alloc_num_free(self._h))

    def block_table(self, seq_ids: Sequence[int], max_blocks: int) -> Tuple[np.ndarray, np.ndarray]:
        ids = np.ascontiguousarray(seq_ids, dtype=np.int64)
        table = np.empty((ids.size, max_blocks), dtype=np.int32)
        lens = np.empty(ids.size, dtype=np.int32)
        self._check(self._lib.pa_alloc_block_table(self._h, int(ids.size), _p(ids), int(max_blocks), _p(table),
                                                  _p(lens)))
        return table, lens

    def stats(self) -> Tuple[int, int]:
        q, h = ctypes.c_int64(0), ctypes.c_int64(0)
        self._check(self._lib.pa_alloc_stats(self._h, ctypes.byref(q), ctypes.byref(h)))
        return q.value, h.value

    def free_queue(self) -> np.ndarray:
        out = np.empty(self.num_blocks, dtype=np.int32)
        n = ctypes.c_int32(0)
        self._check(self._lib.pa_alloc_free_queue(self._h, _p(out), int(out.size), ctypes.byref(n)))
        return out[:n.value].copy()
