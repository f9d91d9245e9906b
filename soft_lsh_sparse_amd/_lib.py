"""ctypes loader for libsocket_lsh.so (the C ABI in include/socket_lsh.h).

The shared library is built in-tree by soft_lsh_sparse_amd.build. There is
no fallback: if it is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

from ctypes import c_float, c_int, c_int32, c_int64, c_size_t, c_void_p, c_char_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsocket_lsh.so")

SOCKET_OK = 0
SOCKET_ERR_INVALID_ARGUMENT = 1
SOCKET_ERR_UNSUPPORTED = 2
SOCKET_ERR_WORKSPACE = 3
SOCKET_ERR_HIP = 4

DTYPE_F32 = 0
DTYPE_BF16 = 1

# size of the library's device array behind socket_decode_noalloc
DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20

# name -> (restype, argtypes); mirrors include/socket_lsh.h
SIGNATURES = {
    "socket_version": (c_int32, []),
    "socket_status_string": (c_char_p, [c_int]),
    "socket_last_error": (c_char_p, []),
    "socket_hash_keys_workspace_bytes": (c_size_t, [c_int, c_int64, c_int64, c_int32,
                                                    c_int32, c_int32]),
    "socket_hash_keys": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int64,
                                 c_int64, c_int64, c_int32, c_int32, c_int32,
                                 c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "socket_bucket_probs": (c_int, [c_void_p, c_void_p, c_int, c_int32, c_int32,
                                    c_int32, c_int32, c_int32, c_int32, c_float,
                                    c_void_p, c_void_p]),
    "socket_hard_bucket_table": (c_int, [c_void_p, c_void_p, c_int, c_int32, c_int32, c_int32,
                                         c_int32, c_int32, c_int32, c_void_p, c_void_p]),
    "socket_score": (c_int, [c_void_p, c_void_p, c_void_p, c_int32, c_int32,
                             c_int32, c_int64, c_int64, c_int32, c_int32,
                             c_void_p, c_void_p]),
    "socket_topk_workspace_bytes": (c_size_t, [c_int32, c_int64, c_int64]),
    "socket_topk": (c_int, [c_void_p, c_int32, c_int64, c_int64, c_void_p,
                            c_void_p, c_size_t, c_void_p]),
    "socket_sparse_attn_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32,
                                                      c_int64]),
    "socket_sparse_attn": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int32,
                                   c_int32, c_int32, c_int32, c_int64, c_void_p,
                                   c_int64, c_void_p, c_void_p, c_size_t,
                                   c_void_p]),
    "socket_dense_attn_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32, c_int64]),
    "socket_dense_attn": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int32, c_int32,
                                  c_int32, c_int32, c_int64, c_int64, c_void_p, c_void_p,
                                  c_size_t, c_void_p]),
    "socket_decode_group_shared_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32,
                                                             c_int32, c_int64, c_int32,
                                                             c_int32, c_int64]),
    "socket_decode_group_shared": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_int, c_int32, c_int32, c_int32,
                                           c_int32, c_int64, c_int64, c_int32, c_int32,
                                           c_float, c_int64, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_size_t, c_void_p]),
    "socket_decode_workspace_bytes": (c_size_t, [c_int32, c_int32, c_int32,
                                                 c_int32, c_int64, c_int32,
                                                 c_int32, c_int64]),
    "socket_decode": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_int, c_int32, c_int32, c_int32,
                              c_int32, c_int64, c_int64, c_int32, c_int32,
                              c_float, c_int64, c_void_p, c_void_p, c_void_p,
                              c_void_p, c_size_t, c_void_p]),
}
SIGNATURES["socket_decode_noalloc"] = (
    c_int, SIGNATURES["socket_decode"][1][:20] + [c_void_p])
SIGNATURES["socket_decode_profiled"] = (
    c_int, SIGNATURES["socket_decode"][1] + [c_void_p, c_int32])
SIGNATURES["socket_decode_kernels"] = (
    c_int32, [c_void_p, c_int, c_int32, c_int32, c_int32, c_int32, c_int64, c_int64,
              c_int32, c_int32, c_int64, c_int32, c_char_p, c_size_t])

_lock = threading.Lock()
_lib = None


class SocketError(RuntimeError):
    """A non-OK status from the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


def load() -> ctypes.CDLL:
    """Load (once) and return the library with typed entry points."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m soft_lsh_sparse_amd.build` (hipcc, gfx950)")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


def check(status: int, what: str) -> None:
    if status == SOCKET_OK:
        return
    lib = load()
    detail = lib.socket_last_error().decode(errors="replace")
    kind = lib.socket_status_string(status).decode(errors="replace")
    raise SocketError(status, f"{what}: {kind}: {detail}")
