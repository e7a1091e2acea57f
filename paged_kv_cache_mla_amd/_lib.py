"""ctypes loader for libkvattn.so (the C ABI declared in include/kvattn.h).

Loading needs no GPU; it fails loudly if the library has not been built.
"""

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVATTN_LIB selects another build of the same sources (the sanitized host builds of
# build.py --sanitize); relative paths are taken from the repository root
LIB_PATH = os.environ.get("KVATTN_LIB") or os.path.join(_HERE, "libkvattn.so")
if not os.path.isabs(LIB_PATH):
    LIB_PATH = os.path.join(os.path.dirname(_HERE), LIB_PATH)

OK = 0
E_INVAL = -1
E_POOL_EXHAUSTED = -2
E_RANGE = -3
E_STATE = -4
E_UNSUPPORTED = -5
E_HIP = -6
F32 = 0
BF16 = 1
BLOCK_ABSENT = -1
MAX_REGIONS = 8
MAX_GROUP_PARTS = 16
ERR_BAD_BLOCK = 1
ERR_BAD_SEQ = 2
ERR_BAD_SELECT = 4

STATUS_NAMES = {OK: "OK", E_INVAL: "E_INVAL", E_POOL_EXHAUSTED: "E_POOL_EXHAUSTED",
                E_RANGE: "E_RANGE", E_STATE: "E_STATE", E_UNSUPPORTED: "E_UNSUPPORTED",
                E_HIP: "E_HIP"}


class Layout(ctypes.Structure):
    _fields_ = [("block_size", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim_k", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
                ("kv_dtype", ctypes.c_int32), ("latent", ctypes.c_int32)]


class Region(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("num_blocks", ctypes.c_int64)]


class ShareModel(ctypes.Structure):
    _fields_ = [("cpu_cost", ctypes.c_double), ("gpu_cost", ctypes.c_double),
                ("cpu_fixed", ctypes.c_double), ("gpu_fixed", ctypes.c_double)]


class ShareState(ctypes.Structure):
    _fields_ = [("placed_tokens", ctypes.c_int64), ("cpu_tokens", ctypes.c_int64),
                ("cpu_batches", ctypes.c_int64), ("batches", ctypes.c_int64),
                ("cpu_cost", ctypes.c_double), ("converged", ctypes.c_double),
                ("target_share", ctypes.c_double), ("samples", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_PI32 = ctypes.POINTER(ctypes.c_int32)
_PI64 = ctypes.POINTER(ctypes.c_int64)

_SIGNATURES = {
    "kvattn_block_bytes": (_I64, [ctypes.POINTER(Layout)]),
    "kvattn_choose_group_parts": (_I32, [_P, _I32, _I32, _PI32, _PI32, _PI32, _I32]),
    "kvattn_decode_plan": (_I32, [_P, _I32, _I32, _PI32, _I32, _PI32, _PI32, _PI32, _I32, _PI32,
                                   _I64, _PI64, _PI32, _PI32]),
    "kvattn_decode_partial_plan": (_I32, [_P, _P, _I32, _I32, _I32, ctypes.c_float, _P, _I32, _P,
                                           _I32, _P, _I32, _P, _P, _P, _P, _P]),
    "kvattn_decode_partial_plan_noalloc": (_I32, [_P, _P, _I32, _I32, _I32, ctypes.c_float, _P, _I32,
                                                   _P, _I32, _I32, _P, _P, _P, _P, _P]),
    "kvattn_pool_alloc": (_I32, [ctypes.POINTER(Layout), ctypes.POINTER(Region), _I32,
                                 ctypes.c_uint64, ctypes.POINTER(_P)]),
    "kvattn_pool_free": (None, [_P]),
    "kvattn_block_table": (_I32, [_P, _I32, _PI32, _PI32, _PI32, _PI32, _PI32, _I32, _PI32, _PI64]),
    "kvattn_block_release": (_I32, [_P, _PI32, _I32, _I32]),
    "kvattn_pool_num_free": (_I64, [_P]),
    "kvattn_pool_refcount": (_I32, [_P, _I32]),
    "kvattn_pool_shared_blocks": (_I64, [_P]),
    "kvattn_pool_add_region": (_I32, [_P, _P, _I64, _PI64]),
    "kvattn_pool_resize_last_region": (_I32, [_P, _I64]),
    "kvattn_pool_num_regions": (_I32, [_P]),
    "kvattn_vmm_create": (_I32, [_I32, ctypes.c_uint64, ctypes.c_uint64, ctypes.POINTER(_P)]),
    "kvattn_vmm_free": (None, [_P]),
    "kvattn_vmm_granularity": (ctypes.c_uint64, [_P]),
    "kvattn_vmm_base": (_P, [_P]),
    "kvattn_vmm_mapped_bytes": (ctypes.c_uint64, [_P]),
    "kvattn_vmm_map_new": (_I32, [_P, ctypes.c_uint64, ctypes.c_uint64]),
    "kvattn_vmm_move": (_I32, [_P, ctypes.c_uint64, _P, ctypes.c_uint64, ctypes.c_uint64, _I32]),
    "kvattn_partition_count": (_I32, [_I32, _I32, _I32]),
    "kvattn_decode_partial": (_I32, [_P, _P, _I32, _I32, _I32, ctypes.c_float, _P, _I32,
                                     _PI32, _PI32, _PI32, _P, _I32, _I32, _P, _P, _P, _P, _P]),
    "kvattn_merge_lse": (_I32, [_P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _P]),
    "kvattn_gather_probe": (_I32, [_P, _I32, _I32, _P, _I32, _PI32, _PI32, _PI32, _P, _I32, _P,
                                   _P, _P]),
    "kvattn_resolve_offsets": (_I32, [_P, _P, _I32, _I32, _P, _I32, _P, _P, _P]),
    "kvattn_select_blocks": (_I32, [_P, _I32, _P, _I32, _P, _I32, _I32, _P, _I32, _P, _P, _P]),
    "kvattn_append_kv": (_I32, [_P, _P, _P, _I32, _I32, _I32, _P, _I32, _P, _P, _P]),
    "kvattn_host_partial": (_I32, [ctypes.POINTER(Layout), ctypes.POINTER(Region), _I32, _P, _I32,
                                   _I32, _I32, ctypes.c_float, _PI32, _I32, _PI32, _P, _P, _I32]),
    "kvattn_share_optimum": (_I32, [ctypes.POINTER(ShareModel), ctypes.c_double,
                                    ctypes.POINTER(ctypes.c_double)]),
    "kvattn_share_fit": (_I32, [_P, _P, _I32, ctypes.POINTER(ctypes.c_double),
                                ctypes.POINTER(ctypes.c_double)]),
    "kvattn_share_ctl_create": (_I32, [ctypes.POINTER(ShareModel), _I32, ctypes.POINTER(_P)]),
    "kvattn_share_ctl_free": (None, [_P]),
    "kvattn_share_admit": (_I32, [_P, _I64, _I64, _PI64]),
    "kvattn_share_observe": (_I32, [_P, ctypes.c_double, ctypes.c_double]),
    "kvattn_share_route": (_I32, [_P, _I64, _PI32]),
    "kvattn_share_get_state": (_I32, [_P, ctypes.POINTER(ShareState)]),
    "kvattn_kvstore_create": (_I32, [_P, _P, _I32, _I32, _I32, ctypes.POINTER(_P),
                                     ctypes.POINTER(_P)]),
    "kvattn_kvstore_free": (None, [_P]),
    "kvattn_kvstore_reserve": (_I32, [_P, _PI32, _PI32]),
    "kvattn_kvstore_commit": (_I32, [_P, _PI32]),
    "kvattn_kvstore_place_prefill_plan": (_I32, [_P, _PI32, _I32, _PI32, _PI32]),
    "kvattn_kvstore_place_prefill": (_I32, [_P, _P, _PI32]),
    "kvattn_kvstore_flush_plan": (_I32, [_P, _PI32, _I32, _PI32, _PI32]),
    "kvattn_kvstore_flush": (_I32, [_P, _P, _PI32]),
    "kvattn_kvstore_views": (_I32, [_P, _PI32, _PI32, _PI32, _PI32]),
    "kvattn_last_error": (ctypes.c_char_p, []),
    "kvattn_version": (ctypes.c_char_p, []),
}

_lib = None


def load():
    """Load libkvattn.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m paged_kv_cache_mla_amd.build` "
            "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class KvattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.kvattn_last_error().decode()
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(status: int, where: str):
    if status != OK:
        raise KvattnError(status, where)
