"""ctypes view of libpa.so (include/pa.h). Marshalling only, no compute.

load() refuses a library whose build id (pa_build_id: a hash of the sources
it was compiled from) differs from the hash of the sources beside it, so a
stale binary is never run in place of the code in the tree.
"""

from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_F32, PA_BF16, PA_INT8 = 0, 1, 2
PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP, PA_ERR_NO_BLOCKS = 0, 1, 2, 3, 4, 5
PA_PART_AUTO, PA_PART_ALIGNED, PA_PART_LIST, PA_PART_PIECES, PA_PART_QUEUE = 0, 1, 2, 3, 4

EXPORTED = ("pa_workspace_size", "pa_plan", "pa_decode", "pa_decode_int8", "pa_verify", "pa_cache_write", "pa_prefill",
            "pa_verify_noalloc", "pa_debug_gather", "pa_validate", "pa_strerror", "pa_last_error", "pa_version",
            "pa_build_id",
            "pa_alloc_create", "pa_alloc_destroy", "pa_alloc_add", "pa_alloc_add_ring", "pa_alloc_append",
            "pa_alloc_append_batch",
            "pa_alloc_release", "pa_alloc_num_free", "pa_alloc_block_table", "pa_alloc_stats",
            "pa_alloc_free_queue")


class PaTuning(ctypes.Structure):
    _fields_ = [
        ("waves", ctypes.c_int32),
        ("blocks_per_wave", ctypes.c_int32),
        ("partition", ctypes.c_int32),
        ("pieces_per_wg", ctypes.c_int32),
        ("oversub", ctypes.c_int32),
        ("segment_blocks", ctypes.c_int32),
    ]


class PaArgs(ctypes.Structure):
    _fields_ = [
        ("out", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("num_seqs", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("debug_visits", ctypes.c_void_p),
        ("timing_start", ctypes.c_void_p),
        ("timing_stop", ctypes.c_void_p),
        ("ring_blocks", ctypes.c_int32),
        ("scale_per_head", ctypes.c_int32),
        ("tuning", ctypes.c_void_p),
        ("debug_stamps", ctypes.c_void_p),
    ]


class PaPlanInfo(ctypes.Structure):
    _fields_ = [
        ("kernel", ctypes.c_int32),
        ("rows", ctypes.c_int32),
        ("waves_per_group", ctypes.c_int32),
        ("splits", ctypes.c_int32),
        ("blocks_per_split", ctypes.c_int32),
        ("grid", ctypes.c_int32),
        ("balanced", ctypes.c_int32),
        ("pieces", ctypes.c_int32),
        ("queue", ctypes.c_int32),
        ("segment_blocks", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class PaWriteArgs(ctypes.Structure):
    _fields_ = [
        ("k_new", ctypes.c_void_p),
        ("v_new", ctypes.c_void_p),
        ("slot_ids", ctypes.c_void_p),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("num_tokens", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("src_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("timing_start", ctypes.c_void_p),
        ("timing_stop", ctypes.c_void_p),
        ("scale_per_head", ctypes.c_int32),
    ]


class PaPrefillArgs(ctypes.Structure):
    _fields_ = [
        ("out", ctypes.c_void_p),
        ("q", ctypes.c_void_p),
        ("q_start", ctypes.c_void_p),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("seq_lens", ctypes.c_void_p),
        ("num_seqs", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("ring_blocks", ctypes.c_int32),
        ("scale_per_head", ctypes.c_int32),
        ("timing_start", ctypes.c_void_p),
        ("timing_stop", ctypes.c_void_p),
    ]


class PaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_lock = threading.Lock()
_lib = None


def check_build_id(lib, root=None) -> None:
    """Raise unless lib was built from the sources under root (default: this checkout).

    Without the sources (an installed copy) there is nothing to compare with
    and the library is taken as it is.
    """
    from . import build
    root = root or build.ROOT
    if not os.path.isdir(os.path.join(root, "paged_kv_cache_94_amd", "csrc")):
        return
    lib.pa_build_id.restype = ctypes.c_char_p
    have = lib.pa_build_id().decode()
    want = build.source_hash(root)
    if have != want:
        raise RuntimeError(f"libpa.so was built from other sources (build id {have}, sources {want}): "
                           "rebuild it with `python -m paged_kv_cache_94_amd.build`")


def load(path: str = LIB_PATH):
    """Load libpa.so. Raises if it has not been built, or was built from other
    sources: there is no fallback."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_94_amd.build` "
                               "(the paged-attention kernels have no CPU or PyTorch fallback)")
        lib = ctypes.CDLL(path)
        check_build_id(lib)
        P = ctypes.POINTER(PaArgs)
        lib.pa_workspace_size.argtypes = [P]
        lib.pa_workspace_size.restype = ctypes.c_size_t
        lib.pa_plan.argtypes = [P, ctypes.POINTER(PaPlanInfo)]
        lib.pa_plan.restype = ctypes.c_int
        for name in ("pa_decode", "pa_decode_int8", "pa_verify", "pa_verify_noalloc"):
            fn = getattr(lib, name)
            fn.argtypes = [P, ctypes.c_void_p]
            fn.restype = ctypes.c_int
        lib.pa_prefill.argtypes = [ctypes.POINTER(PaPrefillArgs), ctypes.c_void_p]
        lib.pa_prefill.restype = ctypes.c_int
        lib.pa_cache_write.argtypes = [ctypes.POINTER(PaWriteArgs), ctypes.c_void_p]
        lib.pa_cache_write.restype = ctypes.c_int
        lib.pa_debug_gather.argtypes = [P, ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.pa_debug_gather.restype = ctypes.c_int
        lib.pa_validate.argtypes = [P, ctypes.c_void_p, ctypes.c_void_p]
        lib.pa_validate.restype = ctypes.c_int
        lib.pa_version.restype = ctypes.c_int
        lib.pa_build_id.restype = ctypes.c_char_p
        bind_host(lib)
        _lib = lib
        return lib


def bind_host(lib):
    """Declare the signatures of the host-only calls (error strings, block
    allocator) on lib: libpa.so, or a separate host build of those sources."""
    lib.pa_strerror.argtypes = [ctypes.c_int]
    lib.pa_strerror.restype = ctypes.c_char_p
    lib.pa_last_error.restype = ctypes.c_char_p
    V, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    alloc_sigs = {
        "pa_alloc_create": ([I32, I32, I32, ctypes.POINTER(V)], ctypes.c_int),
        "pa_alloc_destroy": ([V], None),
        "pa_alloc_add": ([V, I64], ctypes.c_int),
        "pa_alloc_add_ring": ([V, I64, I32], ctypes.c_int),
        "pa_alloc_append": ([V, I64, I32, V, V, V], ctypes.c_int),
        "pa_alloc_append_batch": ([V, I32, V, V, V, V, V, V], ctypes.c_int),
        "pa_alloc_release": ([V, I64], ctypes.c_int),
        "pa_alloc_num_free": ([V], I32),
        "pa_alloc_block_table": ([V, I32, V, I32, V, V], ctypes.c_int),
        "pa_alloc_stats": ([V, V, V], ctypes.c_int),
        "pa_alloc_free_queue": ([V, V, I32, V], ctypes.c_int),
    }
    for name, (args, res) in alloc_sigs.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


def check(rc: int, lib=None) -> None:
    """Raise PaError for a failed call; lib is the library that made it (default libpa.so)."""
    if rc != PA_OK:
        lib = lib or load()
        detail = lib.pa_last_error().decode() or lib.pa_strerror(rc).decode()
        raise PaError(rc, detail)
