"""ctypes loader for libpagedkv.so (the C ABI declared in include/pa.h and
include/pa_block_manager.h)."""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# PAGEDKV_LIB names another build of the same ABI (e.g. the host sanitizer build)
LIB_PATH = os.environ.get("PAGEDKV_LIB") or os.path.join(HERE, "libpagedkv.so")
CHECKED_LIB_PATH = os.path.join(HERE, "libpagedkv_checked.so")   # PA_DEBUG_CHECKS=1 build

PA_OK = 0
PA_F32, PA_F16, PA_BF16 = 0, 1, 2
PA_STREAM_READ_PARTIALS = 16384   # include/pa.h
PA_DECODE_SCRATCH_BYTES = 64 << 20   # include/pa.h
PA_PARTITION_BALANCED = -1
STATUS_NAMES = {0: "PA_OK", 1: "PA_ERR_NULL", 2: "PA_ERR_SHAPE", 3: "PA_ERR_BLOCK_SIZE",
                4: "PA_ERR_DTYPE", 5: "PA_ERR_PARTITION", 6: "PA_ERR_WORKSPACE", 7: "PA_ERR_HIP",
                8: "PA_ERR_ALIGN", 9: "PA_ERR_NO_BLOCKS", 10: "PA_ERR_SEQUENCE", 11: "PA_ERR_CAPACITY",
                12: "PA_ERR_HOST_MEMORY", 13: "PA_ERR_UNSUPPORTED"}
PA_VIOLATION_TABLE_ID, PA_VIOLATION_LENGTH, PA_VIOLATION_SLOT, PA_VIOLATION_BLOCK_ID = 1, 2, 4, 8   # include/pa.h

_c_i32, _c_i64, _c_size, _c_f32, _vp = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                        ctypes.c_float, ctypes.c_void_p)

# name -> (restype, argtypes), mirroring include/pa.h
SIGNATURES = {
    "pa_kv_append": (_c_i32, [_vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                              _c_i32, _vp]),
    "pa_decode_workspace_bytes": (_c_size, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_decode_choose_partition": (_c_i32, [_c_i32, _c_i32, _c_i32, _c_i32]),
    "pa_decode_attention": (_c_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                     _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _c_i32, _c_i32, _vp,
                                     _c_size, _vp]),
    "pa_decode_attention_grouped": (_c_i32, [_vp] * 8 + [_c_i32] * 11 + [_c_f32, _c_i32, _c_i32, _vp, _c_size, _vp]),
    "pa_decode_attention_noalloc": (_c_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                             _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _c_i32, _c_i32, _vp]),
    "pa_prefill_attention": (_c_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32,
                                      _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32, _c_i32, _vp]),
    "pa_decode_attention_hier": (_c_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                                          _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_f32,
                                          _c_i32, _c_i32, _vp, _c_size, _vp]),
    "pa_prefill_attention_hier": (_c_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32,
                                           _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                           _c_f32, _c_i32, _vp]),
    "pa_block_copy": (_c_i32, [_vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp]),
    "pa_swap_out": (_c_i32, [_vp, _vp, _vp, _c_i32, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp]),
    "pa_swap_in": (_c_i32, [_vp, _vp, _vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp]),
    "pa_stream_read": (_c_i32, [_vp, ctypes.c_uint64, _vp, _vp]),
    "pa_status_string": (ctypes.c_char_p, [_c_i32]),
    "pa_debug_violations": (_c_i32, [ctypes.POINTER(ctypes.c_uint32), _c_i32]),
    # include/pa_block_manager.h (host only)
    "pa_bm_create": (_c_i32, [_c_i32, _c_i32, ctypes.POINTER(_vp)]),
    "pa_bm_destroy": (None, [_vp]),
    "pa_bm_add_sequence": (_c_i32, [_vp, ctypes.POINTER(_c_i64)]),
    "pa_bm_fork": (_c_i32, [_vp, _c_i64, ctypes.POINTER(_c_i64)]),
    "pa_bm_free_sequence": (_c_i32, [_vp, _c_i64]),
    "pa_bm_append_slots": (_c_i32, [_vp, _vp, _vp, _c_i32, _vp, _c_i64, _vp, _c_i32,
                                    ctypes.POINTER(_c_i32)]),
    "pa_bm_block_tables": (_c_i32, [_vp, _vp, _c_i32, _c_i32, _vp, _vp]),
    "pa_bm_append_prompt_large": (_c_i32, [_vp, _c_i64, _c_i32, _c_i32, _vp, _c_i64]),
    "pa_bm_block_tables_hier": (_c_i32, [_vp, _vp, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp]),
    "pa_bm_swap_out": (_c_i32, [_vp, _c_i64, _vp, _c_i32, ctypes.POINTER(_c_i32)]),
    "pa_bm_swap_in": (_c_i32, [_vp, _c_i64, _vp, _c_i32, ctypes.POINTER(_c_i32)]),
    "pa_bm_num_free_blocks": (_c_i32, [_vp]),
    "pa_bm_sequence_length": (_c_i32, [_vp, _c_i64, ctypes.POINTER(_c_i64)]),
    "pa_bm_utilisation": (_c_i32, [_vp, ctypes.POINTER(_c_i64), ctypes.POINTER(_c_i64)]),
    "pa_bm_refcounts": (_c_i32, [_vp, _vp, _c_i32]),
    "pa_last_hip_error": (ctypes.c_int, []),
}

_LIB = None


class PagedKVError(RuntimeError):
    """A libpagedkv call returned a non-OK status."""

    def __init__(self, fn: str, status: int, lib=None):
        self.status = status
        msg = STATUS_NAMES.get(status, str(status))
        if lib is not None:
            try:
                msg = lib.pa_status_string(status).decode()
            except Exception:  # pragma: no cover
                pass
            if status == 7:
                msg += f" (hipError_t {lib.pa_last_hip_error()})"
        super().__init__(f"{fn}: {msg}")


def load(path: str = LIB_PATH):
    """Load libpagedkv.so.  There is no fallback: a missing library is an error."""
    global _LIB
    if _LIB is not None and path == LIB_PATH:
        return _LIB
    if not os.path.exists(path):
        raise ImportError(f"libpagedkv.so not built at {path}; run "
                          "`python -m paged_kv_cache_313_amd._build` (needs hipcc)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIB_PATH:
        _LIB = lib
    return lib


def check(fn: str, status: int) -> None:
    if status != PA_OK:
        raise PagedKVError(fn, status, _LIB)
