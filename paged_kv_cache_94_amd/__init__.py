"""Paged decode attention for AMD Instinct MI355X (gfx950).

A thin binding over libpa.so (the C ABI in include/pa.h). Every step of the
attention runs in the library's HIP kernels; this module only checks tensor
shapes, dtypes and devices, passes raw pointers plus the HIP stream, and
allocates the split workspace through PyTorch's caching allocator -- on the
stream the kernels are launched on, so its zero-fill is ordered before them
and the block is not handed out again before they finish.

``tuning`` (decode / verify / plan): a dict of pa_tuning fields (waves,
blocks_per_wave, partition, pieces_per_wg, oversub, segment_blocks) overriding the launch
plan for tests and experiments; ``partition`` takes "aligned", "list",
"pieces" or "queue".

Layouts (row-major, all tensors on the same GPU):
    q, out       [B, q_len, Hq, D]            float32 or bfloat16
    k_pool, v_pool [num_blocks, 16, Hkv, D]   same dtype as q, or int8
    k_scale, v_scale [num_blocks, Hkv, 16]    float32 (int8 caches, one scale per token and head)
                     or [Hkv]                 float32 (int8 caches, one scale per head)
    k_new, v_new [T, Hkv, D]                  float32 or bfloat16 (cache_write)
    slot_ids     [T]                          int64, block * 16 + slot (cache_write)
    q, out       [total, Hq, D] with q_start [B+1] int32 (prefill: packed per-sequence queries)
    block_table  [B, max_blocks_per_seq]      int32 (ring_blocks > 0: each row's first
                                              ring_blocks entries are the sequence's ring)
    seq_lens     [B]                          int32, this step's tokens included
"""

from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib
from ._lib import PaError  # noqa: F401

__all__ = ["decode", "decode_int8", "verify", "verify_noalloc", "prefill", "cache_write", "debug_gather", "validate", "plan",
           "workspace_size", "PaError", "library_path"]

# Status bits of validate() (include/pa.h).
BAD_LEN_SHORT, BAD_LEN_LONG, BAD_BLOCK, BAD_SCALE, BIG_V_SCALE, BAD_WORKSPACE = 1, 2, 4, 8, 16, 32


def library_path() -> str:
    return _lib.LIB_PATH


def _torch():
    import torch
    return torch


def _dtype_code(t, allow_int8: bool) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return _lib.PA_F32
    if t.dtype == torch.bfloat16:
        return _lib.PA_BF16
    if allow_int8 and t.dtype == torch.int8:
        return _lib.PA_INT8
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


PARTITIONS = {"auto": _lib.PA_PART_AUTO, "aligned": _lib.PA_PART_ALIGNED, "list": _lib.PA_PART_LIST,
              "pieces": _lib.PA_PART_PIECES, "queue": _lib.PA_PART_QUEUE}


def _tuning(tuning) -> Optional[_lib.PaTuning]:
    if tuning is None:
        return None
    t = _lib.PaTuning()
    for key, value in dict(tuning).items():
        if key == "partition" and isinstance(value, str):
            value = PARTITIONS[value]
        _require(key in dict(t._fields_), f"unknown tuning field {key!r}")
        setattr(t, key, int(value))
    return t


def _build_args(out, q, k_pool, v_pool, block_table, seq_lens, *, window: int, scale: Optional[float],
                max_seq_len: Optional[int], k_scale, v_scale, num_splits: int, debug_visits,
                ring_blocks: int = 0, tuning=None) -> _lib.PaArgs:
    torch = _torch()
    tensors = [t for t in (out, q, k_pool, v_pool, block_table, seq_lens, k_scale, v_scale, debug_visits)
               if t is not None]
    dev = q.device
    for t in tensors:
        _require(t.is_cuda and t.device == dev, "all tensors must be on the same GPU")
        _require(t.is_contiguous(), "all tensors must be contiguous")
    _require(q.dim() == 4 and out.shape == q.shape and out.dtype == q.dtype, "q/out must be [B, q_len, Hq, D]")
    _require(k_pool.dim() == 4 and v_pool.shape == k_pool.shape and v_pool.dtype == k_pool.dtype,
             "k_pool/v_pool must be [num_blocks, block_size, Hkv, D] of one dtype")
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2, "block_table must be int32 [B, max_blocks]")
    _require(seq_lens.dtype == torch.int32 and seq_lens.dim() == 1, "seq_lens must be int32 [B]")
    B, q_len, Hq, D = q.shape
    nb, bs, Hkv, Dk = k_pool.shape
    _require(Dk == D, "head_dim mismatch between q and the cache")
    _require(block_table.shape[0] == B and seq_lens.shape[0] == B, "batch mismatch")
    per_head = 0
    for s in (k_scale, v_scale):
        if s is not None:
            _require(s.dtype == torch.float32 and tuple(s.shape) in ((nb, Hkv, bs), (Hkv,)),
                     "scales must be float32 [nb, Hkv, bs] (per token) or [Hkv] (per head)")
            per_head = int(tuple(s.shape) == (Hkv,))
    if k_scale is not None and v_scale is not None:
        _require(k_scale.shape == v_scale.shape, "k_scale and v_scale must have one granularity")
    if debug_visits is not None:
        _require(debug_visits.dtype == torch.int32 and tuple(debug_visits.shape) == (B, Hkv, block_table.shape[1]),
                 "debug_visits must be int32 [B, Hkv, max_blocks]")
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B > 0 else q_len   # host sync; pass it to avoid one
    if scale is None:
        scale = D ** -0.5
    a = _lib.PaArgs()
    a.out, a.q, a.k_pool, a.v_pool = _ptr(out), _ptr(q), _ptr(k_pool), _ptr(v_pool)
    a.k_scale, a.v_scale = _ptr(k_scale) or None, _ptr(v_scale) or None
    a.block_table, a.seq_lens = _ptr(block_table), _ptr(seq_lens)
    a.num_seqs, a.q_len, a.num_q_heads, a.num_kv_heads, a.head_dim = B, q_len, Hq, Hkv, D
    a.block_size, a.num_blocks, a.max_blocks_per_seq = bs, nb, block_table.shape[1]
    a.max_seq_len = int(max_seq_len)
    a.window = int(window)
    a.scale = float(scale)
    a.q_dtype = _dtype_code(q, allow_int8=False)
    a.kv_dtype = _dtype_code(k_pool, allow_int8=True)
    a.num_splits = int(num_splits)
    a.debug_visits = _ptr(debug_visits) or None
    a.ring_blocks = int(ring_blocks)
    a.scale_per_head = per_head
    t = _tuning(tuning)
    a._tuning_ref = t   # keeps the struct alive as long as the args
    a.tuning = ctypes.addressof(t) if t is not None else None
    return a


def _stream(stream, device=None):
    torch = _torch()
    return stream if stream is not None else torch.cuda.current_stream(device)


def _stream_handle(stream) -> int:
    return _stream(stream).cuda_stream


def _attach_workspace(a: _lib.PaArgs, workspace, device, stream) -> object:
    """Attach the caller's workspace, or allocate one on `stream` (the launch stream).

    A new workspace is allocated and zero-filled under `stream`: the fill is
    ordered before the kernels launched on it, and when the tensor is
    released the caching allocator hands the block out again only to later
    work on that same stream. A caller's own workspace is the caller's to
    order (its first 4096 bytes must be zero before the first call).
    """
    lib = _lib.load()
    need = lib.pa_workspace_size(ctypes.byref(a))
    if need == ctypes.c_size_t(-1).value:
        _lib.check(_lib.PA_ERR_INVALID_ARG)
    if need == 0:
        return None
    if workspace is None:
        torch = _torch()
        # Zero-filled: the library keeps the header words of the piece queue
        # at zero between calls but needs them zero before the first one.
        with torch.cuda.stream(stream):
            workspace = torch.zeros(need, dtype=torch.uint8, device=device)
    _require(workspace.numel() * workspace.element_size() >= need, f"workspace needs {need} bytes")
    a.workspace = workspace.data_ptr()
    a.workspace_bytes = workspace.numel() * workspace.element_size()
    return workspace


def _run(entry: str, out, q, k_pool, v_pool, block_table, seq_lens, *, window=0, scale=None, max_seq_len=None,
         k_scale=None, v_scale=None, num_splits=0, workspace=None, debug_visits=None, stream=None,
         timing=None, ring_blocks=0, tuning=None):
    lib = _lib.load()
    a = _build_args(out, q, k_pool, v_pool, block_table, seq_lens, window=window, scale=scale,
                    max_seq_len=max_seq_len, k_scale=k_scale, v_scale=v_scale, num_splits=num_splits,
                    debug_visits=debug_visits, ring_blocks=ring_blocks, tuning=tuning)
    s = _stream(stream, q.device)
    ws = _attach_workspace(a, workspace, q.device, s)
    if timing is not None:
        a.timing_start = ctypes.c_void_p(timing[0].cuda_event if hasattr(timing[0], "cuda_event") else timing[0])
        a.timing_stop = ctypes.c_void_p(timing[1].cuda_event if hasattr(timing[1], "cuda_event") else timing[1])
    rc = getattr(lib, entry)(ctypes.byref(a), ctypes.c_void_p(s.cuda_stream))
    _lib.check(rc)
    del ws  # allocated on s: reused only by later work on s, after these kernels
    return out


def decode(out, q, k_pool, v_pool, block_table, seq_lens, **kw):
    """Single-token decode (q_len == 1) over an fp32 or bf16 cache. Writes and returns ``out``."""
    return _run("pa_decode", out, q, k_pool, v_pool, block_table, seq_lens, **kw)


def decode_int8(out, q, k_pool, v_pool, block_table, seq_lens, k_scale, v_scale, **kw):
    """Single-token decode over an int8 cache with per-token, per-KV-head fp32 scales."""
    return _run("pa_decode_int8", out, q, k_pool, v_pool, block_table, seq_lens, k_scale=k_scale,
                v_scale=v_scale, **kw)


def verify(out, q, k_pool, v_pool, block_table, seq_lens, **kw):
    """q_len >= 1 query tokens per sequence, causal among themselves."""
    return _run("pa_verify", out, q, k_pool, v_pool, block_table, seq_lens, **kw)


def verify_noalloc(out, q, k_pool, v_pool, block_table, seq_lens, *, window=0, scale=None, max_seq_len=None,
                   k_scale=None, v_scale=None, num_splits=0, debug_visits=None, stream=None, timing=None,
                   ring_blocks=0, tuning=None):
    """pa_verify with the library's static scratch array as the workspace (pa_verify_noalloc).

    Nothing is allocated on this path, here or in the library; calls that
    overlap on one GPU share its scratch array and race.
    """
    lib = _lib.load()
    a = _build_args(out, q, k_pool, v_pool, block_table, seq_lens, window=window, scale=scale,
                    max_seq_len=max_seq_len, k_scale=k_scale, v_scale=v_scale, num_splits=num_splits,
                    debug_visits=debug_visits, ring_blocks=ring_blocks, tuning=tuning)
    if timing is not None:
        a.timing_start = ctypes.c_void_p(getattr(timing[0], "cuda_event", timing[0]))
        a.timing_stop = ctypes.c_void_p(getattr(timing[1], "cuda_event", timing[1]))
    _lib.check(lib.pa_verify_noalloc(ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream))))
    return out


def cache_write(k_new, v_new, slot_ids, k_pool, v_pool, k_scale=None, v_scale=None, *, stream=None,
                timing=None):
    """Append this step's K/V rows to the pools at ``slot_ids`` (int8 pools: quantize per token and head).

    Negative slot ids skip their token. Pass the same tensor as ``k_pool`` and
    ``v_pool`` (and as ``k_new`` and ``v_new``) for a cache whose values are
    its keys. Asynchronous on ``stream``. ``timing``: optional pair of
    recorded timing events that the kernel's own dispatch stamps.
    """
    torch = _torch()
    tensors = [t for t in (k_new, v_new, slot_ids, k_pool, v_pool, k_scale, v_scale) if t is not None]
    dev = k_new.device
    for t in tensors:
        _require(t.is_cuda and t.device == dev, "all tensors must be on the same GPU")
        _require(t.is_contiguous(), "all tensors must be contiguous")
    _require(k_new.dim() == 3 and v_new.shape == k_new.shape and v_new.dtype == k_new.dtype,
             "k_new/v_new must be [T, Hkv, D] of one dtype")
    _require(k_pool.dim() == 4 and v_pool.shape == k_pool.shape and v_pool.dtype == k_pool.dtype,
             "k_pool/v_pool must be [num_blocks, block_size, Hkv, D] of one dtype")
    T, Hkv, D = k_new.shape
    nb, bs, hkv2, d2 = k_pool.shape
    _require((hkv2, d2) == (Hkv, D), "k_new and the pools disagree on Hkv or D")
    _require(slot_ids.dtype == torch.int64 and tuple(slot_ids.shape) == (T,), "slot_ids must be int64 [T]")
    per_head = 0
    for sc in (k_scale, v_scale):
        if sc is not None:
            _require(sc.dtype == torch.float32 and tuple(sc.shape) in ((nb, Hkv, bs), (Hkv,)),
                     "scales must be float32 [nb, Hkv, bs] (per token) or [Hkv] (per head)")
            per_head = int(tuple(sc.shape) == (Hkv,))
    w = _lib.PaWriteArgs()
    w.k_new, w.v_new, w.slot_ids = _ptr(k_new), _ptr(v_new), _ptr(slot_ids)
    w.k_pool, w.v_pool = _ptr(k_pool), _ptr(v_pool)
    w.k_scale, w.v_scale = _ptr(k_scale) or None, _ptr(v_scale) or None
    w.num_tokens, w.num_kv_heads, w.head_dim = T, Hkv, D
    w.block_size, w.num_blocks = bs, nb
    w.src_dtype = _dtype_code(k_new, allow_int8=False)
    w.kv_dtype = _dtype_code(k_pool, allow_int8=True)
    w.scale_per_head = per_head
    if timing is not None:
        w.timing_start = getattr(timing[0], "cuda_event", timing[0])
        w.timing_stop = getattr(timing[1], "cuda_event", timing[1])
    lib = _lib.load()
    _lib.check(lib.pa_cache_write(ctypes.byref(w), ctypes.c_void_p(_stream_handle(stream))))
    return k_pool


def prefill(out, q, q_start, k_pool, v_pool, block_table, seq_lens, *, max_q_len: int, window=0, scale=None,
            max_seq_len: Optional[int] = None, k_scale=None, v_scale=None, ring_blocks=0, stream=None,
            timing=None):
    """Causal attention of packed query chunks over their sequences' paged caches. Writes and returns ``out``.

    Sequence b's queries are rows q_start[b] .. q_start[b+1]-1 of q; the chunk's own
    keys and values must already be in the cache. ``max_q_len`` (a host integer, no
    device read) bounds every sequence's query count and sizes the launch.
    """
    torch = _torch()
    tensors = [t for t in (out, q, q_start, k_pool, v_pool, block_table, seq_lens, k_scale, v_scale) if t is not None]
    dev = q.device
    for t in tensors:
        _require(t.is_cuda and t.device == dev, "all tensors must be on the same GPU")
        _require(t.is_contiguous(), "all tensors must be contiguous")
    _require(q.dim() == 3 and out.shape == q.shape and out.dtype == q.dtype, "q/out must be [total, Hq, D]")
    _require(k_pool.dim() == 4 and v_pool.shape == k_pool.shape and v_pool.dtype == k_pool.dtype,
             "k_pool/v_pool must be [num_blocks, block_size, Hkv, D] of one dtype")
    _require(q_start.dtype == torch.int32 and q_start.dim() == 1, "q_start must be int32 [B+1]")
    _require(block_table.dtype == torch.int32 and block_table.dim() == 2, "block_table must be int32 [B, max_blocks]")
    _require(seq_lens.dtype == torch.int32 and seq_lens.dim() == 1, "seq_lens must be int32 [B]")
    total, Hq, D = q.shape
    nb, bs, Hkv, Dk = k_pool.shape
    B = seq_lens.shape[0]
    _require(Dk == D and q_start.shape[0] == B + 1 and block_table.shape[0] == B, "shape mismatch")
    per_head = 0
    for sc in (k_scale, v_scale):
        if sc is not None:
            _require(sc.dtype == torch.float32 and tuple(sc.shape) in ((nb, Hkv, bs), (Hkv,)),
                     "scales must be float32 [nb, Hkv, bs] (per token) or [Hkv] (per head)")
            per_head = int(tuple(sc.shape) == (Hkv,))
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B > 0 else 1   # host sync; pass it to avoid one
    a = _lib.PaPrefillArgs()
    a.out, a.q, a.q_start = _ptr(out), _ptr(q), _ptr(q_start)
    a.k_pool, a.v_pool = _ptr(k_pool), _ptr(v_pool)
    a.k_scale, a.v_scale = _ptr(k_scale) or None, _ptr(v_scale) or None
    a.block_table, a.seq_lens = _ptr(block_table), _ptr(seq_lens)
    a.num_seqs, a.total_q, a.max_q_len = B, total, int(max_q_len)
    a.num_q_heads, a.num_kv_heads, a.head_dim = Hq, Hkv, D
    a.block_size, a.num_blocks, a.max_blocks_per_seq = bs, nb, block_table.shape[1]
    a.max_seq_len = int(max_seq_len)
    a.window = int(window)
    a.scale = float(D ** -0.5 if scale is None else scale)
    a.q_dtype = _dtype_code(q, allow_int8=False)
    a.kv_dtype = _dtype_code(k_pool, allow_int8=True)
    a.ring_blocks = int(ring_blocks)
    a.scale_per_head = per_head
    if timing is not None:
        a.timing_start = getattr(timing[0], "cuda_event", timing[0])
        a.timing_stop = getattr(timing[1], "cuda_event", timing[1])
    lib = _lib.load()
    _lib.check(lib.pa_prefill(ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream))))
    return out


def plan(q, k_pool, v_pool, block_table, seq_lens, *, window=0, scale=None, max_seq_len=None, k_scale=None,
         v_scale=None, num_splits=0, ring_blocks=0, tuning=None) -> dict:
    """The launch plan libpa would use for these tensors (no launch)."""
    lib = _lib.load()
    a = _build_args(q, q, k_pool, v_pool, block_table, seq_lens, window=window, scale=scale,
                    max_seq_len=max_seq_len, k_scale=k_scale, v_scale=v_scale, num_splits=num_splits,
                    debug_visits=None, ring_blocks=ring_blocks, tuning=tuning)
    info = _lib.PaPlanInfo()
    _lib.check(lib.pa_plan(ctypes.byref(a), ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in info._fields_}


def workspace_size(q, k_pool, v_pool, block_table, seq_lens, **kw) -> int:
    return plan(q, k_pool, v_pool, block_table, seq_lens, **kw)["workspace_bytes"]


def debug_gather(which: int, dst, q, k_pool, v_pool, block_table, seq_lens, *, window=0, max_seq_len=None,
                 stream=None, ring_blocks=0):
    """Raw cache rows the kernels load, in logical key order: dst [B, dst_tokens, Hkv, D]."""
    lib = _lib.load()
    _require(dst.is_cuda and dst.is_contiguous() and dst.dtype == k_pool.dtype and dst.dim() == 4,
             "dst must be a contiguous [B, dst_tokens, Hkv, D] tensor of the cache dtype")
    a = _build_args(q, q, k_pool, v_pool, block_table, seq_lens, window=window, scale=1.0,
                    max_seq_len=max_seq_len, k_scale=None, v_scale=None, num_splits=0, debug_visits=None,
                    ring_blocks=ring_blocks)
    rc = lib.pa_debug_gather(ctypes.byref(a), int(which), ctypes.c_void_p(dst.data_ptr()), dst.shape[1],
                             ctypes.c_void_p(_stream_handle(stream)))
    _lib.check(rc)
    return dst


def validate(q, k_pool, v_pool, block_table, seq_lens, *, window=0, max_seq_len=None, ring_blocks=0,
             k_scale=None, v_scale=None, stream=None, workspace=None, num_splits=0, tuning=None):
    """Device check of the lengths, table entries and (int8, given both scales) scales a step would use.

    Returns int32 [B+1]: entry 1+b holds sequence b's BAD_* / BIG_V_SCALE
    bits (0 when fine), entry 0 their OR. With ``workspace`` (and the plan
    that ``num_splits`` / ``tuning`` give), entry 0 also gets BAD_WORKSPACE
    if the call would use the piece queue and the workspace's queue counters
    are not zero.
    """
    torch = _torch()
    lib = _lib.load()
    a = _build_args(q, q, k_pool, v_pool, block_table, seq_lens, window=window, scale=1.0,
                    max_seq_len=max_seq_len, k_scale=k_scale, v_scale=v_scale, num_splits=num_splits,
                    debug_visits=None, ring_blocks=ring_blocks, tuning=tuning)
    if workspace is not None:
        a.workspace = workspace.data_ptr()
        a.workspace_bytes = workspace.numel() * workspace.element_size()
    s = _stream(stream, q.device)
    with torch.cuda.stream(s):   # zero-filled on the stream the check runs on
        status = torch.zeros(seq_lens.shape[0] + 1, dtype=torch.int32, device=q.device)
    _lib.check(lib.pa_validate(ctypes.byref(a), ctypes.c_void_p(status.data_ptr()), ctypes.c_void_p(s.cuda_stream)))
    return status


class Prepared:
    """A call whose arguments are marshalled once and launched many times.

    Pointers, shapes and the workspace are fixed at construction (the
    tiniestgpt notes' rule for replaying a decode step: static buffers, no
    host sync per step); ``launch`` only enqueues the kernels on a stream.
    The tensors must stay alive and keep their storage while this object is
    used. A workspace the object allocates is zero-filled at construction,
    which waits for the fill, so launches on any stream find it ready; every
    other stream a launch uses is recorded on it, so the caching allocator
    does not hand the block out again while that stream's kernels may still
    use it.
    """

    def __init__(self, entry: str, out, q, k_pool, v_pool, block_table, seq_lens, *, window=0, scale=None,
                 max_seq_len=None, k_scale=None, v_scale=None, num_splits=0, workspace=None, ring_blocks=0,
                 tuning=None, entry_point: Optional[str] = None):
        self._lib = _lib.load()
        self._fn = getattr(self._lib, entry_point or {"decode": "pa_decode", "decode_int8": "pa_decode_int8",
                                                      "verify": "pa_verify"}[entry])
        self.args = _build_args(out, q, k_pool, v_pool, block_table, seq_lens, window=window, scale=scale,
                                max_seq_len=max_seq_len, k_scale=k_scale, v_scale=v_scale,
                                num_splits=num_splits, debug_visits=None, ring_blocks=ring_blocks, tuning=tuning)
        home = _stream(None, q.device)
        owned = workspace is None
        self.workspace = _attach_workspace(self.args, workspace, q.device, home)
        if owned and self.workspace is not None:
            home.synchronize()   # the zero-fill is done before any stream launches
        self._home = home.cuda_stream
        self._recorded = set()
        self._keep = (out, q, k_pool, v_pool, block_table, seq_lens, k_scale, v_scale)

    def launch(self, stream=None, timing=None) -> None:
        if timing is not None:
            self.args.timing_start = ctypes.c_void_p(timing[0].cuda_event)
            self.args.timing_stop = ctypes.c_void_p(timing[1].cuda_event)
        else:
            self.args.timing_start = None
            self.args.timing_stop = None
        s = _stream(stream)
        if self.workspace is not None and s.cuda_stream != self._home and s.cuda_stream not in self._recorded:
            self.workspace.record_stream(s)
            self._recorded.add(s.cuda_stream)
        _lib.check(self._fn(ctypes.byref(self.args), ctypes.c_void_p(s.cuda_stream)))


__all__.append("Prepared")
