"""ctypes loader for ``libpagedkv.so`` (the C ABI of ``include/pa.h``).

Argument marshalling only.  The library must have been built in-tree (see
``__graft_entry__.build()``); if it is missing, every call raises: there is no
fallback implementation.
"""

from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpagedkv.so")

PA_F16, PA_BF16, PA_F8E4M3, PA_I8 = 0, 1, 2, 3
PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_HIP = range(5)
# Scratch of pa_decode_noalloc (PA_DECODE_SCRATCH_BYTES in include/pa.h).
PA_DECODE_SCRATCH_BYTES = 64 << 20
STATUS_NAMES = {
    PA_OK: "PA_OK",
    PA_ERR_INVALID: "PA_ERR_INVALID",
    PA_ERR_UNSUPPORTED: "PA_ERR_UNSUPPORTED",
    PA_ERR_WORKSPACE: "PA_ERR_WORKSPACE",
    PA_ERR_HIP: "PA_ERR_HIP",
}

# Exported entry points and their C signatures (names as in include/pa.h).
_i32, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
SIGNATURES = {
    "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_reshape_and_cache": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, ctypes.c_int,
        _f32, _f32, _vp]),
    "pa_reshape_and_cache_i8": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _vp]),
    "pa_copy_blocks": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _vp]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_decode_workspace_bytes_for": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                            ctypes.c_int]),
    "pa_decode": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
        ctypes.c_int, ctypes.c_int, _f32, _f32, _i32, _i32, _vp, _sz, _vp]),
    "pa_decode_noalloc": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
        ctypes.c_int, ctypes.c_int, _f32, _f32, _i32, _i32, _vp]),
    "pa_decode_append": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
        ctypes.c_int, ctypes.c_int, _f32, _f32, _i32, _i32, _vp, _sz, _vp]),
    "pa_decode_i8": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
        ctypes.c_int, _i32, _i32, _vp, _sz, _vp]),
    "pa_decode_append_i8": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
        _i32, _f32, ctypes.c_int, _i32, _i32, _vp, _sz, _vp]),
    "pa_prefill_chunk_i8": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
        _f32, ctypes.c_int, _vp]),
    "pa_prefill_chunk": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32,
        ctypes.c_int, ctypes.c_int, _f32, _f32, _vp]),
    "pa_prefill_chunk_window": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
        _f32, ctypes.c_int, _i32, _vp]),
    "pa_prefill_chunk_window_quant": (ctypes.c_int, [
        _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
        _i32, _i32, _f32, ctypes.c_int, ctypes.c_int, _f32, _f32, _i32, _vp]),
}

_lock = threading.Lock()
_lib = None


class PagedKVError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library once and declare its signatures."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build the HIP library first "
                "(python -c 'import __graft_entry__ as g; g.build()')")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def check(status: int) -> None:
    if status != PA_OK:
        msg = load().pa_last_error().decode(errors="replace")
        raise PagedKVError(status, msg)
