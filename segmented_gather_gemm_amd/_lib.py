"""Views of libsgg_lora.so (the C ABI declared in include/sgg_lora.h).

``lib()`` is a ctypes handle with every entry point; ``calls()`` is the
CPython module ``_sggcall`` with the hot entry points (plan upload, shrink,
expand, qkv, embedding), which take integer arguments and cost far less per
call than ctypes.
"""

import ctypes
import os

from .build import CALLMOD, LIB

_i32, _i64, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
_pi32, _pi64 = ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)

SIGNATURES = {
    "lora_last_error": (ctypes.c_char_p, []),
    "lora_plan_segments": (ctypes.c_int, [
        _pi32, _pi32, _i32, _i32, _i32, _i32, _i32,
        _pi32, _i64, _pi32, _pi32, _i32, _pi32, _pi32, _pi32, _pi64]),
    "lora_plan_lm_head": (ctypes.c_int, [
        _pi32, _pi32, _i32, _i32, _i32, _i32,
        _pi32, _i64, _pi32, _pi32, _i32, _pi32, _pi32, _pi64]),
    "lora_plan_max_segments": (_i64, [_i64, _i32, _i32]),
    "lora_plan_layout": (_i64, [_i64, _i32, _i32, _i32, _pi64]),
    # host arrays are passed as addresses (NumPy .ctypes.data) on this hot call
    "lora_plan_upload": (ctypes.c_int, [
        _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
        _i64, _i32, _i32, _vp, _vp, _i64, _vp, _vp, _i32, _vp]),
    "lora_plan_upload_embedding": (ctypes.c_int, [
        _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
        _i64, _i32, _i32, _vp, _vp, _i64, _vp, _vp, _i32,
        _vp, _vp, _i64, _vp, _i64, _i32, _i64, _vp]),
    "lora_plan_device": (ctypes.c_int, [
        _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
        _i64, _i32, _i32, _vp, _i64, _vp, _vp]),
    "lora_plan_lm_head_upload": (ctypes.c_int, [
        _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32,
        _i64, _i32, _i32, _vp, _vp, _i64, _vp, _vp, _i32, _vp]),
    "lora_shrink_workspace_bytes": (_i64, [_i64, _i64, _i32, _i32, _i32, _i32]),
    "lora_shrink": (ctypes.c_int, [
        _vp, _i64, _vp, _vp, _i64, _i64, _i64, _i32, _i32, _i32,
        _vp, _vp, _i32, _vp, _vp, _i32, _vp, _i64, _vp]),
    "lora_expand": (ctypes.c_int, [
        _vp, _i64, _vp, _i64, _vp, _i64, _i64, _i32, _i32, _pi32, _i32, _i32,
        _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp]),
    "lora_qkv_workspace_bytes": (_i64, [_i64, _i64, _i32, _i32, _i32, _i32]),
    "lora_qkv": (ctypes.c_int, [
        _vp, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _pi32, _i32, _i32,
        _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i64, _vp]),
    "lora_qkv_noalloc": (ctypes.c_int, [
        _vp, _i64, _vp, _vp, _i64, _vp, _i64, _i64, _i64, _i32, _i32, _pi32, _i32, _i32,
        _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp]),
    "lora_set_option": (_i64, [ctypes.c_char_p, _i64]),
    "lora_moe_route": (ctypes.c_int, [
        _vp, _vp, _i32, _vp, _i64, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp]),
    "lora_moe_plan": (ctypes.c_int, [
        _vp, _vp, _i32, _vp, _i64, _i32, _i32, _vp, _vp, _i32, _i32, _i32, _vp, _i64, _vp, _vp]),
    "lora_moe_add": (ctypes.c_int, [
        _vp, _i64, _i64, _i32, _vp, _vp, _i64, _vp, _i64, _i64, _i32, _i32,
        _vp, _vp, _i32, _vp, _vp, _vp, _i32, _vp, _i64, _vp]),
    "lora_a_embedding": (ctypes.c_int, [
        _vp, _vp, _i64, _vp, _i64, _i64, _i32, _i32, _i64, _vp, _vp, _i32, _vp, _vp, _i32, _vp]),
}

STATUS = {0: "ok", -1: "invalid argument", -2: "unsupported", -3: "capacity", -4: "HIP error"}


class SggError(RuntimeError):
    """A non-zero status from libsgg_lora; `.code` holds the status."""

    def __init__(self, code, message):
        super().__init__(f"{STATUS.get(code, code)} ({code}): {message}")
        self.code = code


_lib = None


def lib():
    """Load the library once.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise ImportError(
                f"{LIB} is missing: build it with `python segmented_gather_gemm_amd/build.py`")
        handle = ctypes.CDLL(LIB)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


_calls = None


def calls():
    """The CPython call module over the library.  Raises if it has not been built."""
    global _calls
    if _calls is None:
        if not os.path.exists(CALLMOD):
            raise ImportError(
                f"{CALLMOD} is missing: build it with `python segmented_gather_gemm_amd/build.py`")
        lib()
        from . import _sggcall
        _calls = _sggcall
    return _calls


def check(rc):
    if rc != 0:
        raise SggError(rc, lib().lora_last_error().decode(errors="replace"))
