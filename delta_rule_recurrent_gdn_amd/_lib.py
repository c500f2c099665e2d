"""ctypes loader for libgdn2.so (the C ABI declared in include/gdn2.h).

The library is built in-tree by ``delta_rule_recurrent_gdn_amd.build``. There
is no fallback: if it is missing or cannot be loaded, importing the binding
raises with the reason.
"""

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgdn2.so")

GDN2_OK = 0
GDN2_ERR_NULL = -1
GDN2_ERR_SHAPE = -2
GDN2_ERR_DTYPE = -3
GDN2_ERR_ALIGN = -4
GDN2_ERR_UNSUPPORTED = -5
GDN2_ERR_WORKSPACE = -6
GDN2_ERR_HIP = -7

GDN2_F32 = 0
GDN2_BF16 = 1

GDN2_OP_FWD = 0
GDN2_OP_DECODE = 1
GDN2_OP_BWD = 2
GDN2_OP_BWD_RECORDS = 3

GDN2_FLAG_RAW_GATES = 1
GDN2_FLAG_SCALAR_B = 2
GDN2_FLAG_SCALAR_W = 4
GDN2_FLAG_SCALAR_DECAY = 8

GDN2_NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024  # the device array of gdn2_fwd_chunked_noalloc

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_U = ctypes.c_uint

# name -> (restype, argtypes), in the order of include/gdn2.h
SIGNATURES = {
    "gdn2_fwd_chunked": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I, _I, _I, _I, _I, _I, _I, _P]),
    "gdn2_fwd_chunked_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _I, _I, _I, _I, _I, _I, _I, _U,
                                 _P]),
    "gdn2_decode_step": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "gdn2_decode_step_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _U, _P]),
    "gdn2_bwd_chunked": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                              _I, _I, _I, _I, _I, _I, _I, _P]),
    "gdn2_bwd_chunked_ex": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                 _I, _I, _I, _I, _I, _I, _I, _U, _P]),
    "gdn2_records_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "gdn2_fwd_chunked_train": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _SZ, _I, _I, _I, _I, _I, _I,
                                    _I, _U, _P]),
    "gdn2_bwd_chunked_records": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                      _I, _I, _I, _I, _I, _I, _I, _U, _P]),
    "gdn2_varlen_max_chunks": (_I, [_I, _I, _I]),
    "gdn2_varlen_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "gdn2_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _SZ, _I, _I, _I, _I, _I, _I, _U,
                             _P]),
    "gdn2_bwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ,
                             _I, _I, _I, _I, _I, _I, _U, _P]),
    "gdn2_varlen_records_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "gdn2_fwd_varlen_train": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _P, _SZ, _P, _SZ, _I, _I, _I, _I, _I,
                                   _I, _U, _P]),
    "gdn2_bwd_varlen_records": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _P, _P, _SZ, _P, _P, _P, _P, _P, _P, _P, _P,
                                     _SZ, _I, _I, _I, _I, _I, _I, _U, _P]),
    "gdn2_decode_step_slots": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _U, _P]),
    "gdn2_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "gdn2_fwd_chunked_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P]),
    "gdn2_status_string": (ctypes.c_char_p, [_I]),
    "gdn2_version": (_I, []),
}

_lib = None


def load():
    """Load libgdn2.so once and set the C signatures. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built: run `python -m delta_rule_recurrent_gdn_amd.build` "
            "(or __graft_entry__.build()) first; there is no non-HIP fallback")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class GDN2Error(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = load().gdn2_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def check(status, where):
    if status != GDN2_OK:
        raise GDN2Error(status, where)
