"""ctypes view of the C ABI declared in include/csa.h (argument marshalling only)."""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa.so")

c_void_p = ctypes.c_void_p
c_int = ctypes.c_int
c_int32 = ctypes.c_int32
c_int64 = ctypes.c_int64
c_uint64 = ctypes.c_uint64
c_size_t = ctypes.c_size_t
c_double = ctypes.c_double


class Shape(ctypes.Structure):
    _fields_ = [("num_kv_heads", c_int32), ("group_size", c_int32), ("head_dim", c_int32),
                ("n_cap", c_int64)]


class Packed(ctypes.Structure):
    _fields_ = [("codes", c_void_p), ("kscale", c_void_p), ("zq", c_void_p), ("bmeta", c_void_p),
                ("kerr", c_void_p), ("vnorm", c_void_p), ("codes8", c_void_p), ("scale8", c_void_p),
                ("kerr8", c_void_p)]


class Params(ctypes.Structure):
    _fields_ = [("eps", c_double), ("delta", c_double), ("r", c_int32), ("J", c_int32),
                ("window", c_int32), ("measure", c_int32), ("seed", c_uint64), ("step", c_uint64),
                ("layer", c_int32), ("cand_budget", c_int32), ("cand_budget2", c_int32)]


class Item(ctypes.Structure):
    _fields_ = [("n", c_int64), ("slot", c_int32), ("layer", c_int32), ("eps", c_double),
                ("seed", c_uint64), ("step", c_uint64)]


class Trace(ctypes.Structure):
    _fields_ = [("c_R", c_void_p), ("c_lo", c_void_p), ("c_star", c_void_p),
                ("bucket_count", c_void_p), ("lub", c_void_p), ("cmax_count", c_void_p),
                ("cand_count", c_void_p), ("beta_level", c_void_p), ("dhat_level", c_void_p),
                ("k_level", c_void_p), ("logtau", c_void_p), ("ev_scan_begin", c_void_p),
                ("ev_scan_end", c_void_p), ("cand_pos", c_void_p), ("cand_hl", c_void_p),
                ("rescored_count", c_void_p), ("cand_l8", c_void_p)]


SYMBOLS = {
    "csa_pack_kv_4bit": (c_int, [ctypes.POINTER(Shape), c_void_p, c_void_p, c_int64, c_int64,
                                 ctypes.POINTER(Packed), c_void_p]),
    "csa_workspace_bytes": (c_size_t, [ctypes.POINTER(Shape), ctypes.POINTER(Params), c_int64]),
    "csa_certified_decode_attention": (c_int, [ctypes.POINTER(Shape), ctypes.POINTER(Params), c_void_p,
                                               c_void_p, c_void_p, ctypes.POINTER(Packed), c_int64,
                                               c_void_p, c_size_t, c_void_p, c_void_p, c_void_p,
                                               c_void_p, ctypes.POINTER(Trace), c_void_p]),
    "csa_certified_decode_attention_noalloc": (c_int, [ctypes.POINTER(Shape), ctypes.POINTER(Params), c_void_p,
                                                       c_void_p, c_void_p, ctypes.POINTER(Packed), c_int64,
                                                       c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "csa_workspace_bytes_batch": (c_size_t, [ctypes.POINTER(Shape), ctypes.POINTER(Params), c_int32, c_int64]),
    "csa_certified_decode_attention_batch": (c_int, [ctypes.POINTER(Shape), ctypes.POINTER(Params), c_int32,
                                                     c_int32, ctypes.POINTER(Item), c_void_p, c_void_p, c_void_p,
                                                     ctypes.POINTER(Packed), c_void_p, c_size_t, c_void_p,
                                                     c_void_p, c_void_p, c_void_p, c_void_p]),
    "csa_scan_bounds": (c_int, [ctypes.POINTER(Shape), ctypes.POINTER(Params), c_void_p, c_void_p,
                                ctypes.POINTER(Packed), c_int64, c_void_p, c_size_t, c_void_p,
                                c_void_p, c_void_p, c_void_p]),
    "csa_dense_workspace_bytes": (c_size_t, [ctypes.POINTER(Shape), c_int64]),
    "csa_dense_decode_attention": (c_int, [ctypes.POINTER(Shape), c_void_p, c_void_p, c_void_p, c_int64,
                                           c_void_p, c_size_t, c_void_p, c_void_p]),
    "csa_status_string": (ctypes.c_char_p, [c_int]),
    "csa_last_error": (ctypes.c_char_p, []),
    "csa_stream_read": (c_int, [c_void_p, ctypes.c_int64, c_int, c_void_p, c_void_p, c_void_p, c_void_p]),
    "csa_event_create": (c_int, [ctypes.POINTER(c_void_p)]),
    "csa_event_destroy": (c_int, [c_void_p]),
    "csa_event_elapsed_ms": (c_int, [c_void_p, c_void_p, ctypes.POINTER(ctypes.c_float)]),
}

_lib = None


class CsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


def load():
    """Load libcsa.so from the package directory; raise loudly when it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with certified_sparse_attention_amd._build.build() "
                           "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SYMBOLS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int, what: str):
    if status != 0:
        lib = load()
        raise CsaError(status, f"{what}: {lib.csa_status_string(status).decode()}: "
                               f"{lib.csa_last_error().decode()}")
