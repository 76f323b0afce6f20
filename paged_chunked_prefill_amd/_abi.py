"""ctypes declarations of libpkv.so's C ABI (include/pkv.h)."""
from __future__ import annotations

import ctypes
import os

PKV_OK = 0
PKV_ERR_INVALID_ARGUMENT = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_WORKSPACE = -3
PKV_ERR_HIP = -4
PKV_DTYPE_BF16 = 0
PKV_DTYPE_FP32 = 1
PKV_STATUS_BAD_PAGE = 1
PKV_FLAG_NON_CAUSAL = 1
PKV_MAX_SPLITS = 32
PKV_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTS = ("pkv_extend_metadata_size", "build_extend_metadata", "pkv_extend_metadata_size_ex",
           "build_extend_metadata_ex", "pkv_append", "pkv_rope_append",
           "paged_extend_attn", "paged_extend_attn_masked", "paged_extend_attn_append", "paged_extend_attn_noalloc",
           "pkv_read_status",
           "pkv_last_error",
           "pkv_device_supported")

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")


class PkvShape(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class PkvPlan(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("total_q", ctypes.c_int32), ("max_q_len", ctypes.c_int32),
                ("max_kv_len", ctypes.c_int32), ("n_items", ctypes.c_int32), ("n_split_rows", ctypes.c_int32),
                ("max_splits", ctypes.c_int32), ("window", ctypes.c_int32), ("flags", ctypes.c_int32),
                ("slot_blocks", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("shape", PkvShape),
                ("workspace_bytes", ctypes.c_size_t),
                ("qo_indptr", ctypes.c_void_p), ("kv_indptr", ctypes.c_void_p),
                ("prefix_lens", ctypes.c_void_p), ("items", ctypes.c_void_p),
                ("split_rows", ctypes.c_void_p), ("status", ctypes.c_void_p)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_SZ = ctypes.c_size_t


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    # PyTorch ships its own HIP runtime (same soname as /opt/rocm's). Loading
    # torch first makes libpkv.so bind to that runtime instead of pulling in a
    # second one, which would not see the device torch has opened.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(path):
        raise ImportError(f"libpkv.so is not built ({path}); run __graft_entry__.build() or "
                          "python -m paged_chunked_prefill_amd.build_lib")
    lib = ctypes.CDLL(path)
    sig = {
        "pkv_extend_metadata_size": [_I32, _P, _P, ctypes.POINTER(PkvShape), _I32, _I32,
                                     ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)],
        "build_extend_metadata": [_I32, _P, _P, ctypes.POINTER(PkvShape), _I32, _I32, _P, _SZ, _P, _SZ,
                                  ctypes.POINTER(PkvPlan), _P],
        "pkv_extend_metadata_size_ex": [_I32, _P, _P, ctypes.POINTER(PkvShape), _I32, _I32, _I32, _I32,
                                        ctypes.POINTER(_SZ), ctypes.POINTER(_SZ)],
        "build_extend_metadata_ex": [_I32, _P, _P, ctypes.POINTER(PkvShape), _I32, _I32, _I32, _I32, _P, _SZ, _P,
                                     _SZ, ctypes.POINTER(PkvPlan), _P],
        "pkv_append": [_P, _P, _P, _P, _P, _I32, _P, ctypes.POINTER(PkvPlan), ctypes.POINTER(PkvShape), _P],
        "pkv_rope_append": [_P, _P, _P, _P, _P, _I32, _P, _P, _P, _I32, _P, ctypes.POINTER(PkvPlan),
                            ctypes.POINTER(PkvShape), _P],
        "paged_extend_attn": [_P, _P, _P, _P, _I32, _P, _P, _P, _P, _I32, ctypes.c_float,
                              ctypes.POINTER(PkvPlan), ctypes.POINTER(PkvShape), _P, _P, _SZ, _P],
        "paged_extend_attn_masked": [_P, _P, _P, _P, _I32, _P, _P, _P, _P, _I32, ctypes.c_float, _P, _I32, _I32,
                                     _I32, ctypes.POINTER(PkvPlan), ctypes.POINTER(PkvShape), _P, _P, _SZ, _P],
        "paged_extend_attn_append": [_P, _P, _P, _P, _P, _P, _I32, _P, _I32, ctypes.c_float,
                                     ctypes.POINTER(PkvPlan), ctypes.POINTER(PkvShape), _P, _P, _SZ, _P],
        "paged_extend_attn_noalloc": [_P, _P, _P, _P, _I32, _P, _P, _P, _P, _I32, ctypes.c_float,
                                      ctypes.POINTER(PkvPlan), ctypes.POINTER(PkvShape), _P, _P],
        "pkv_read_status": [ctypes.POINTER(PkvPlan), ctypes.POINTER(_I32), _P],
        "pkv_last_error": [],
        "pkv_device_supported": [ctypes.c_int],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_char_p if name == "pkv_last_error" else ctypes.c_int
    return lib
