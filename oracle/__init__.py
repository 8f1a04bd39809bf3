"""fp64 CPU oracle for one paged decode-attention step (test infrastructure).

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP library and never reads
its results. ``oracle.c`` holds the arithmetic; this module builds it with
gcc and marshals numpy arrays into it.

Dtype codes follow the storage: float32 arrays are fp32, uint16 arrays are
bf16 bit patterns, int8 arrays are int8 codes (with float32 scales).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

ORC_F32, ORC_BF16, ORC_I8 = 0, 1, 2
_ERRORS = {1: "invalid argument", 2: "sequence length or block id out of range", 3: "out of memory"}


class OracleError(RuntimeError):
    pass


class _Problem(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("B", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("Hq", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("scale", ctypes.c_double),
        ("ring_blocks", ctypes.c_int32),
        ("head_scales", ctypes.c_int32),
        ("q_start", ctypes.c_void_p),
    ]


class _Write(ctypes.Structure):
    _fields_ = [
        ("k_new", ctypes.c_void_p),
        ("v_new", ctypes.c_void_p),
        ("slot_ids", ctypes.c_void_p),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("src_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("T", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("head_scales", ctypes.c_int32),
    ]


def build(force: bool = False, extra_flags: Optional[list] = None, out: Optional[str] = None) -> str:
    """Compile oracle.c into a shared library with gcc (-O2, OpenMP)."""
    target = out or _LIB_PATH
    if not force and out is None and os.path.exists(target) and \
            os.path.getmtime(target) >= os.path.getmtime(_SRC):
        return target
    tmp = target + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"] + list(extra_flags or [])
    subprocess.run(cmd, check=True)
    os.replace(tmp, target)
    return target


def _bind(path: str):
    lib = ctypes.CDLL(path)
    lib.oracle_attention.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_int]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_visited_blocks.argtypes = [ctypes.POINTER(_Problem), ctypes.c_void_p]
    lib.oracle_visited_blocks.restype = ctypes.c_int
    lib.oracle_gather.argtypes = [ctypes.POINTER(_Problem), ctypes.c_int, ctypes.c_void_p,
                                  ctypes.c_int64]
    lib.oracle_gather.restype = ctypes.c_int
    lib.oracle_default_threads.restype = ctypes.c_int
    lib.oracle_cache_write.argtypes = [ctypes.POINTER(_Write)]
    lib.oracle_cache_write.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            _lib = _bind(build())
    return _lib


_override = threading.local()


def _current():
    lib = getattr(_override, "lib", None)
    return lib if lib is not None else _load()


class use_variant:
    """Context manager: route this thread's oracle calls to another build of oracle.c.

    Only the tests use it, to run the pins against copies built with a
    planted mistake (``-DORC_MUTANT=n``).
    """

    def __init__(self, path: str):
        self.lib = _bind(path)

    def __enter__(self):
        self.prev = getattr(_override, "lib", None)
        _override.lib = self.lib
        return self

    def __exit__(self, *exc):
        _override.lib = self.prev
        return False


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return ORC_F32
    if a.dtype == np.uint16:
        return ORC_BF16
    if a.dtype == np.int8:
        return ORC_I8
    raise TypeError(f"unsupported storage dtype {a.dtype}")


class Problem:
    """Keeps the numpy arrays alive while the C struct points into them."""

    def __init__(self, q, k_pool, v_pool, block_table, seq_lens, *, q_len, window, scale,
                 k_scale=None, v_scale=None, block_size=16, ring_blocks=0, q_start=None):
        """q_start: None (q is [B, q_len, Hq, D]) or [B+1] offsets of packed queries (q is [total, Hq, D])."""
        self.q_start = None if q_start is None else np.ascontiguousarray(q_start, dtype=np.int32)
        q = np.asarray(q)
        if self.q_start is not None:
            if q.ndim != 3 or q.shape[0] != int(self.q_start[-1]):
                raise ValueError("packed queries must be [q_start[-1], Hq, D]")
            q = q.reshape(q.shape[0], 1, q.shape[1], q.shape[2])
            q_len = 1
        self.q = np.ascontiguousarray(q)
        self.k_pool = np.ascontiguousarray(k_pool)
        self.v_pool = self.k_pool if v_pool is k_pool else np.ascontiguousarray(v_pool)
        self.block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        self.seq_lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
        self.k_scale = None if k_scale is None else np.ascontiguousarray(k_scale, dtype=np.float32)
        self.v_scale = None if v_scale is None else np.ascontiguousarray(v_scale, dtype=np.float32)
        if self.q.ndim != 4 or self.k_pool.ndim != 4 or self.k_pool.shape != self.v_pool.shape:
            raise ValueError("q must be [B,q_len,Hq,D]; pools [num_blocks,block_size,Hkv,D]")
        B, ql, Hq, D = self.q.shape
        nb, bs, Hkv, Dk = self.k_pool.shape
        if ql != q_len or Dk != D or bs != block_size:
            raise ValueError("shape mismatch")
        kv_code = _dtype_code(self.k_pool)
        if _dtype_code(self.v_pool) != kv_code:
            raise ValueError("k and v pools differ in dtype")
        head_scales = 0
        for sc in (self.k_scale, self.v_scale):
            if sc is not None and sc.shape == (Hkv,):
                head_scales = 1
            elif sc is not None and sc.shape != (nb, Hkv, bs):
                raise ValueError("scales must be [num_blocks, Hkv, block_size] (per token) or [Hkv] (per head)")
        if self.k_scale is not None and self.v_scale is not None and self.k_scale.shape != self.v_scale.shape:
            raise ValueError("k and v scales must have the same granularity")
        s = _Problem()
        s.q = self.q.ctypes.data
        s.k_pool = self.k_pool.ctypes.data
        s.v_pool = self.v_pool.ctypes.data
        s.k_scale = self.k_scale.ctypes.data if self.k_scale is not None else None
        s.v_scale = self.v_scale.ctypes.data if self.v_scale is not None else None
        s.block_table = self.block_table.ctypes.data
        s.seq_lens = self.seq_lens.ctypes.data
        s.q_dtype = _dtype_code(self.q)
        s.kv_dtype = kv_code
        s.B, s.q_len, s.Hq, s.Hkv, s.D = B, q_len, Hq, Hkv, D
        s.block_size, s.num_blocks = bs, nb
        s.max_blocks = self.block_table.shape[1]
        s.window = int(window)
        s.scale = float(scale)
        s.ring_blocks = int(ring_blocks)
        s.head_scales = head_scales
        if self.q_start is not None:
            if self.q_start.shape != (self.seq_lens.size + 1,):
                raise ValueError("q_start must be [B+1]")
            s.q_start = self.q_start.ctypes.data
            s.B = self.seq_lens.size
            self.shape = (int(self.q_start[-1]), Hq, D)
        else:
            self.shape = (B, q_len, Hq, D)
        self.struct = s

    @classmethod
    def from_inputs(cls, x) -> "Problem":
        """Build from any object with the paged-input attribute names."""
        return cls(x.q, x.k_pool, x.v_pool, x.block_table, x.seq_lens, q_len=x.q_len,
                   window=x.window, scale=x.scale, k_scale=x.k_scale, v_scale=x.v_scale,
                   block_size=x.block_size, ring_blocks=getattr(x, "ring_blocks", 0),
                   q_start=getattr(x, "q_start", None))


def _check(rc: int) -> None:
    if rc != 0:
        raise OracleError(_ERRORS.get(rc, f"error {rc}"))


def attention(p: Problem, rows: Optional[np.ndarray] = None, threads: int = 0) -> np.ndarray:
    """fp64 attention. All rows -> [B,q_len,Hq,D] ([total,Hq,D] packed); listed rows -> [n_rows, D]."""
    lib = _current()
    D = p.shape[-1]
    if rows is None:
        out = np.empty(p.shape, dtype=np.float64)
        _check(lib.oracle_attention(ctypes.byref(p.struct), None, 0, out.ctypes.data, threads))
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        out = np.empty((r.size, D), dtype=np.float64)
        _check(lib.oracle_attention(ctypes.byref(p.struct), r.ctypes.data, r.size, out.ctypes.data, threads))
    return out


def visited_blocks(p: Problem) -> np.ndarray:
    """[B, max_blocks] int32: per table entry, the logical blocks it holds with a key some query row sees.

    A linear table gives 1 for such blocks and 0 elsewhere; in a ring the entry
    holding both the oldest and the newest keys of the window counts 2.
    """
    lib = _current()
    vis = np.empty((p.seq_lens.size, p.block_table.shape[1]), dtype=np.int32)
    _check(lib.oracle_visited_blocks(ctypes.byref(p.struct), vis.ctypes.data))
    return vis


def gather(p: Problem, which: int, dst_tokens: int, fill: int = 0) -> np.ndarray:
    """Raw K (which=0) or V (which=1) rows of the visible key range, [B, dst_tokens, Hkv, D]."""
    lib = _current()
    B = p.seq_lens.size
    _, _, Hkv, D = p.k_pool.shape
    dst = np.full((B, dst_tokens, Hkv, D), fill, dtype=p.k_pool.dtype)
    _check(lib.oracle_gather(ctypes.byref(p.struct), which, dst.ctypes.data, dst_tokens))
    return dst


def default_threads() -> int:
    return int(_current().oracle_default_threads())


def cache_write(k_new: np.ndarray, v_new: np.ndarray, slot_ids: np.ndarray, k_pool: np.ndarray,
                v_pool: np.ndarray, k_scale: Optional[np.ndarray] = None, v_scale: Optional[np.ndarray] = None,
                block_size: int = 16) -> None:
    """Write this step's rows [T, Hkv, D] into the pools in place (int8 pools: quantize).

    int8 pools take scales [num_blocks, Hkv, block_size] (per token: computed
    and written) or [Hkv] (per head: given, read only). Every array is
    modified in place and must be C-contiguous of its declared dtype.
    """
    lib = _current()
    arrays = [k_new, v_new, slot_ids, k_pool, v_pool] + [a for a in (k_scale, v_scale) if a is not None]
    for a in arrays:
        if not a.flags.c_contiguous:
            raise ValueError("cache_write needs C-contiguous arrays")
    if slot_ids.dtype != np.int64 or k_new.shape != v_new.shape or k_new.ndim != 3:
        raise ValueError("slot_ids must be int64 [T]; k_new, v_new [T, Hkv, D]")
    T, Hkv, D = k_new.shape
    nb, bs, hkv2, d2 = k_pool.shape
    if (bs, hkv2, d2) != (block_size, Hkv, D) or v_pool.shape != k_pool.shape or slot_ids.shape != (T,):
        raise ValueError("shape mismatch")
    kv = _dtype_code(k_pool)
    head_scales = 0
    if kv == ORC_I8:
        for sc in (k_scale, v_scale):
            if sc is None or sc.dtype != np.float32 or sc.shape not in ((nb, Hkv, bs), (Hkv,)):
                raise ValueError("int8 pools need float32 scales [num_blocks, Hkv, block_size] or [Hkv]")
        if k_scale.shape != v_scale.shape:
            raise ValueError("k and v scales must have the same granularity")
        head_scales = int(k_scale.shape == (Hkv,))
    w = _Write()
    w.k_new, w.v_new, w.slot_ids = k_new.ctypes.data, v_new.ctypes.data, slot_ids.ctypes.data
    w.k_pool, w.v_pool = k_pool.ctypes.data, v_pool.ctypes.data
    w.k_scale = k_scale.ctypes.data if k_scale is not None else None
    w.v_scale = v_scale.ctypes.data if v_scale is not None else None
    w.src_dtype, w.kv_dtype = _dtype_code(k_new), kv
    w.T, w.Hkv, w.D, w.block_size, w.num_blocks = T, Hkv, D, bs, nb
    w.head_scales = head_scales
    _check(lib.oracle_cache_write(ctypes.byref(w)))

