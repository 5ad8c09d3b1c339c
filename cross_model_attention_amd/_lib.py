"""ctypes declarations of libmapflow's C ABI (include/mapflow.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_int64, c_size_t, c_uint16, c_uint64, c_void_p

# MAPFLOW_LIB names another build of the library (for example one compiled with different flags)
LIB_PATH = os.environ.get("MAPFLOW_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib",
                                                          "libmapflow.so")
HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "mapflow.h")

MF_OK, MF_ERR_INVALID, MF_ERR_UNSUPPORTED, MF_ERR_OOM, MF_ERR_HIP, MF_ERR_CAPACITY = range(6)
MF_F32, MF_BF16 = 0, 1
STATUS_NAMES = {0: "MF_OK", 1: "MF_ERR_INVALID", 2: "MF_ERR_UNSUPPORTED", 3: "MF_ERR_OOM",
                4: "MF_ERR_HIP", 5: "MF_ERR_CAPACITY"}


class MfBsr(ctypes.Structure):
    _fields_ = [
        ("B", c_int32), ("H_s", c_int32), ("n_seq", c_int32), ("n_brow", c_int32),
        ("nb_max", c_int32), ("n_order", c_int32), ("T", c_int64), ("n_causal", c_int64),
        ("capacity", c_int64), ("nnzb", c_int64),
        ("brow_info", c_void_p), ("brow_order", c_void_p), ("brow_coff", c_void_p),
        ("block_ptr", c_void_p),
        ("block_idx", c_void_p), ("block_row", c_void_p), ("probs", c_void_p),
        ("row_kept_mass", c_void_p), ("counters", c_void_p), ("_owner", c_void_p),
    ]


class MfVfrag(ctypes.Structure):
    _fields_ = [
        ("B", c_int32), ("d", c_int32), ("H_kv", c_int32), ("n_brow", c_int32), ("T", c_int64),
        ("frag", c_void_p), ("exps", c_void_p), ("_owner", c_void_p),
    ]


class MfRecvLayer(ctypes.Structure):
    _fields_ = [("Q", c_void_p), ("K", c_void_p), ("V", c_void_p), ("W", c_void_p), ("O", c_void_p)]


class MfSendLayer(ctypes.Structure):
    _fields_ = [("Q", c_void_p), ("K", c_void_p)]


# mf_alloc_fn / mf_free_fn
ALLOC_FN = ctypes.CFUNCTYPE(c_void_p, c_size_t, c_void_p, c_void_p)
FREE_FN = ctypes.CFUNCTYPE(None, c_void_p, c_size_t, c_void_p, c_void_p)
MF_PREFILL_ISOLATE, MF_PREFILL_TIMING = 1, 2

_P_I32 = POINTER(c_int32)
_P_F32 = POINTER(c_float)
_SIGNATURES = {
    "mf_version": (c_char_p, []),
    "mf_last_error": (c_char_p, []),
    "mf_create": (c_int, [c_int, ALLOC_FN, FREE_FN, c_void_p, POINTER(c_void_p)]),
    "mf_destroy": (c_int, [c_void_p]),
    "mf_map_layers": (c_int, [c_void_p, _P_I32, c_int32, c_int32, c_int32]),
    "mf_layer_map_uniform": (c_int, [c_int32, c_int32, c_int32, _P_I32]),
    "mf_check_layer_map": (c_int, [_P_I32, c_int32, c_int32, c_int32]),
    "mf_bsr_create": (c_int, [c_void_p, c_int32, c_int32, _P_I32, c_int32, c_int64, POINTER(MfBsr)]),
    "mf_bsr_create_range": (c_int, [c_void_p, c_int32, c_int32, _P_I32, c_int32, _P_I32, c_int64, POINTER(MfBsr)]),
    "mf_bsr_download": (c_int, [c_void_p, POINTER(MfBsr), _P_I32, _P_I32, POINTER(c_uint16),
                                POINTER(c_float)]),
    "mf_bsr_download_blocks": (c_int, [c_void_p, POINTER(MfBsr), c_int64, c_int64, _P_I32, POINTER(c_uint16)]),
    "mf_bsr_upload": (c_int, [c_void_p, POINTER(MfBsr), _P_I32, _P_I32, POINTER(c_uint16),
                              POINTER(c_float)]),
    "mf_bsr_free": (c_int, [c_void_p, POINTER(MfBsr)]),
    "mf_compress_into": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int32, c_float,
                                 POINTER(MfBsr), c_void_p]),
    "mf_compress_prefill_into": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int32, c_float,
                                         POINTER(MfBsr), c_void_p, c_void_p]),
    "mf_compress_into_ex": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int32, c_float, ctypes.c_uint32,
                                    POINTER(MfBsr), c_void_p]),
    "mf_bsr_sync": (c_int, [c_void_p, POINTER(MfBsr), c_void_p]),
    "mf_compress": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_int32, c_int32, _P_I32, c_int32,
                            c_float, c_int32, c_void_p, POINTER(MfBsr)]),
    "mf_v_prepare": (c_int, [c_void_p, _P_I32, c_int32, c_int32, c_void_p, c_int, c_int32, c_int32,
                             c_void_p, c_int32, c_int32, POINTER(MfVfrag), c_void_p]),
    "mf_vfrag_free": (c_int, [c_void_p, POINTER(MfVfrag)]),
    "mf_retrieve_prepared": (c_int, [c_void_p, POINTER(MfBsr), c_void_p, c_int32, POINTER(MfVfrag),
                                     _P_I32, c_void_p, c_void_p]),
    "mf_retrieve_layers": (c_int, [c_void_p, c_int32, POINTER(MfBsr), POINTER(c_void_p), c_int32, POINTER(MfVfrag),
                                   _P_I32, c_void_p, c_void_p]),
    "mf_retrieve_multi": (c_int, [c_void_p, POINTER(MfBsr), c_int32, POINTER(c_void_p), _P_I32,
                                  POINTER(POINTER(MfVfrag)), POINTER(_P_I32), POINTER(c_void_p), c_void_p]),
    "mf_retrieve": (c_int, [c_void_p, POINTER(MfBsr), c_void_p, c_int32, c_void_p, c_int, c_int32,
                            c_int32, c_void_p, c_int32, c_int32, _P_I32, c_void_p, c_void_p]),
    "mf_retrieve_noalloc": (c_int, [c_void_p, POINTER(MfBsr), c_void_p, c_int32, c_void_p, c_int, c_int32,
                                    c_int32, c_void_p, c_int32, c_int32, _P_I32, c_void_p, c_void_p]),
    "mf_dense_attention": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int32, c_int32,
                                   c_int32, _P_I32, c_int32, _P_I32, c_void_p, c_void_p]),
    "mf_prefill_layers": (c_int, [c_void_p, POINTER(MfRecvLayer), POINTER(MfSendLayer), c_int, c_int32, c_int32,
                                  c_int32, _P_I32, c_float, c_int32, POINTER(MfBsr), ctypes.c_uint32, c_void_p,
                                  c_void_p]),
    "mf_prefill_timings": (c_int, [c_void_p, _P_F32, _P_F32, _P_F32, _P_F32]),
    "mf_copy_probe": (c_int, [c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "mf_read_probe": (c_int, [c_void_p, c_void_p, c_size_t, c_void_p, c_void_p]),
    "mf_write_probe": (c_int, [c_void_p, c_void_p, c_size_t, c_void_p, c_void_p]),
    "mf_fill_probe": (c_int, [c_void_p, c_void_p, c_size_t, ctypes.c_uint32, c_void_p]),
    "mf_prefix_hashes": (c_int, [_P_I32, c_int64, c_int32, POINTER(c_uint64)]),
    "mf_cache_create": (c_int, [c_void_p, c_int64, POINTER(c_void_p)]),
    "mf_cache_destroy": (c_int, [c_void_p]),
    "mf_cache_info": (c_int, [c_void_p, POINTER(c_int64), POINTER(c_int64)]),
    "mf_cache_insert": (c_int, [c_void_p, c_int32, _P_I32, c_int64, c_int32, POINTER(MfBsr), c_int32, c_void_p]),
    "mf_cache_lookup": (c_int, [c_void_p, c_int32, _P_I32, c_int64, c_int32, POINTER(c_int32), POINTER(MfBsr)]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree libmapflow.so; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmapflow.so is not built ({LIB_PATH}); run "
                          "`python cross_model_attention_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class MapflowError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def check(status: int) -> None:
    if status != MF_OK:
        raise MapflowError(status, load().mf_last_error().decode(errors="replace"))


def i32_array(values):
    arr = (c_int32 * len(values))(*[int(v) for v in values])
    return arr
