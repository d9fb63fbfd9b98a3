"""ctypes loader for libspecverify.so: argument and return types of every exported symbol.

The library must have been built in-tree (python -m speculative_decoding_decode_amd.build);
there is no fallback of any kind: a missing library raises.  SPEC_VERIFY_LIB may name another
build of the same sources (a timing variant, see build.py) to load instead.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.environ.get("SPEC_VERIFY_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")

c_int, c_float, c_size_t, c_void_p = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p
c_char_p, c_uint64 = ctypes.c_char_p, ctypes.c_uint64

# name -> (restype, argtypes), in the order of include/spec_verify.h
SIGNATURES = {
    "spec_version": (c_int, []),
    "spec_last_error": (c_char_p, []),
    "spec_verify_attn_workspace": (c_size_t, [c_int] * 8),
    "spec_verify_attn": (c_int, [c_void_p] * 6 + [c_int] * 9 + [c_float, c_int, c_void_p,
                                                                    c_size_t, c_void_p]),
    "spec_lm_head_workspace": (c_size_t, [c_int] * 3),
    "spec_lm_head": (c_int, [c_void_p] * 5 + [c_int] * 4 + [c_void_p, c_size_t, c_void_p]),
    "spec_lm_head_noalloc": (c_int, [c_void_p] * 5 + [c_int] * 4 + [c_void_p]),
    "spec_profile_lm_head": (c_int, [c_void_p, c_void_p]),
    "spec_accept_workspace": (c_size_t, [c_int] * 3),
    "spec_accept": (c_int, [c_void_p] * 6 + [c_int] * 3 + [c_void_p, c_size_t, c_void_p]),
    "spec_accept_philox": (c_int, [c_void_p] * 3 + [c_uint64, c_uint64] + [c_void_p] * 3
                           + [c_int] * 3 + [c_void_p, c_size_t, c_void_p]),
    "spec_lm_head_accept_workspace": (c_size_t, [c_int] * 4),
    "spec_lm_head_accept": (c_int, [c_void_p] * 6 + [c_uint64, c_uint64] + [c_void_p] * 3
                            + [c_int] * 5 + [c_void_p, c_size_t, c_void_p]),
    "spec_kv_append": (c_int, [c_void_p] * 6 + [c_int] * 7 + [c_int, c_void_p]),
    "spec_kv_commit": (c_int, [c_void_p, c_void_p, c_int, c_int, c_void_p]),
    "spec_hbm_probe_grid": (c_int, []),
    "spec_hbm_probe": (c_int, [c_int, c_void_p, c_void_p, c_size_t, c_void_p]),
}

_lib = None


class SpecError(RuntimeError):
    """A negative status from the library, with its spec_last_error() message."""

    def __init__(self, fn: str, code: int, msg: str):
        super().__init__(f"{fn} failed ({code}): {msg}")
        self.code = code


def load() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m speculative_decoding_decode_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def last_error() -> str:
    return (load().spec_last_error() or b"").decode()


def check(fn: str, code: int) -> None:
    if code != 0:
        raise SpecError(fn, code, last_error())
