"""ctypes view of ``include/nvfp4_attn.h``: struct layouts, signatures and errors.

Argument marshalling only; every computation happens in the HIP library.  The
library must have been built (``python attention_bit_paged_amd/build.py``); a missing
library, or one without every entry point, raises ImportError instead of falling
back to anything else.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# NVFP4_ATTN_LIB selects another build of the same library (for example a copy built
# with different compile flags); by default the in-tree build is loaded.
LIB_PATH = os.environ.get("NVFP4_ATTN_LIB") or os.path.join(_HERE, "libnvfp4_attn.so")

STATUS = {
    0: "NVFP4_OK", 1: "NVFP4_E_INVALID", 2: "NVFP4_E_SHAPE", 3: "NVFP4_E_UNSUPPORTED",
    4: "NVFP4_E_LDS_BUDGET", 5: "NVFP4_E_WORKSPACE", 6: "NVFP4_E_DEVICE", 7: "NVFP4_E_HIP",
}
STATUS_CODE = {v: k for k, v in STATUS.items()}

# Names declared in include/nvfp4_attn.h, in order.
EXPORTS = (
    "nvfp4_last_error", "nvfp4_version", "nvfp4_quantize_kv", "nvfp4_plan_create",
    "nvfp4_plan_create_ex",
    "nvfp4_plan_destroy", "nvfp4_plan_workspace_bytes", "nvfp4_plan_get_info",
    "nvfp4_plan_get_work", "nvfp4_plan_upload", "nvfp4_batch_decode",
    "nvfp4_batch_decode_noalloc",
    "nvfp4_batch_decode_append", "nvfp4_kv_checksum", "nvfp4_set_timing_events",
    "nvfp4_batch_prefill", "nvfp4_plan_mask_bytes", "nvfp4_batch_prefill_masked",
    "nvfp4_batch_prefill_ragged",
    "nvfp4_plan_set_deferred_merge", "nvfp4_merge_partials", "nvfp4_merge_states",
)

WORK_FIELDS = ("request", "kv_head", "row_begin", "row_count", "kv_begin", "kv_end",
               "partial_slot", "merge_index")


class KVPoolStruct(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("stride_page", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
        ("stride_token", ctypes.c_int64),
        ("sf", ctypes.c_void_p),
        ("sf_stride_page", ctypes.c_int64),
        ("sf_stride_head", ctypes.c_int64),
        ("sf_stride_token", ctypes.c_int64),
        ("num_pages", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("global_scale", ctypes.c_float),
        ("kv_dtype", ctypes.c_int32),
    ]


KV_DTYPES = {"nvfp4": 0, "fp8": 1}


class PlanOptionsStruct(ctypes.Structure):
    _fields_ = [("kv_dtype", ctypes.c_int32), ("kv_indptr", ctypes.c_void_p),
                ("custom_mask", ctypes.c_int32), ("pos_encoding", ctypes.c_int32),
                ("rope_theta", ctypes.c_float), ("rope_scale", ctypes.c_float)]


POS_ENCODINGS = {"none": 0, "rope": 1}  # nvfp4_pos_encoding


class KVRaggedStruct(ctypes.Structure):
    _fields_ = [
        ("data", ctypes.c_void_p),
        ("stride_row", ctypes.c_int64),
        ("stride_head", ctypes.c_int64),
        ("sf", ctypes.c_void_p),
        ("sf_stride_row", ctypes.c_int64),
        ("sf_stride_head", ctypes.c_int64),
        ("num_rows", ctypes.c_int64),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("global_scale", ctypes.c_float),
        ("kv_dtype", ctypes.c_int32),
    ]


class PlanInfoStruct(ctypes.Structure):
    _fields_ = [
        ("num_work_items", ctypes.c_int32),
        ("num_partials", ctypes.c_int32),
        ("num_merges", ctypes.c_int32),
        ("kv_chunk_tokens", ctypes.c_int32),
        ("rows_per_item", ctypes.c_int32),
        ("is_prefill", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_int64),
    ]


class NVFP4Error(RuntimeError):
    """A library call returned a status other than NVFP4_OK."""

    def __init__(self, status: int, message: str):
        self.status = STATUS.get(status, str(status))
        super().__init__(f"{self.status}: {message}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing; build it with `python attention_bit_paged_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                             ctypes.c_size_t)
    pool_p = ctypes.POINTER(KVPoolStruct)
    sig = {
        "nvfp4_last_error": (ctypes.c_char_p, []),
        "nvfp4_version": (ctypes.c_char_p, []),
        "nvfp4_quantize_kv": (ctypes.c_int, [vp, i64, i64, vp, i64, i64, i64, vp, pool_p, pool_p, vp]),
        "nvfp4_plan_create": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                             ctypes.POINTER(vp)]),
        "nvfp4_plan_create_ex": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, i32, i32, i32, i32,
                                                i32, ctypes.POINTER(PlanOptionsStruct),
                                                ctypes.POINTER(vp)]),
        "nvfp4_plan_destroy": (None, [vp]),
        "nvfp4_plan_workspace_bytes": (sz, [vp]),
        "nvfp4_plan_get_info": (ctypes.c_int, [vp, ctypes.POINTER(PlanInfoStruct)]),
        "nvfp4_plan_get_work": (ctypes.c_int, [vp, vp, i64]),
        "nvfp4_plan_upload": (ctypes.c_int, [vp, vp, sz, vp]),
        "nvfp4_batch_decode": (ctypes.c_int, [vp, vp, i64, i64, vp, i64, pool_p, pool_p, f32, vp, sz,
                                              vp, i64, i64, vp, vp]),
        "nvfp4_batch_decode_noalloc": (ctypes.c_int, [vp, vp, i64, i64, vp, i64, pool_p, pool_p,
                                                      f32, vp, i64, i64, vp, vp]),
        "nvfp4_batch_decode_append": (ctypes.c_int, [vp, vp, i64, i64, vp, i64, i64, vp, i64, i64,
                                                     vp, i64, pool_p, pool_p, f32, vp, sz,
                                                     vp, i64, i64, vp, vp]),
        "nvfp4_kv_checksum": (ctypes.c_int, [vp, vp, i64, pool_p, pool_p, vp, sz, vp, vp]),
        "nvfp4_set_timing_events": (ctypes.c_int, [vp, vp]),
        "nvfp4_batch_prefill": (ctypes.c_int, [vp, vp, i64, i64, vp, i64, pool_p, pool_p, f32, vp, sz,
                                               vp, i64, i64, vp, vp]),
        "nvfp4_plan_mask_bytes": (i64, [vp]),
        "nvfp4_batch_prefill_masked": (ctypes.c_int, [vp, vp, i64, i64, vp, i64, pool_p, pool_p,
                                                      vp, f32, vp, sz, vp, i64, i64, vp, vp]),
        "nvfp4_batch_prefill_ragged": (ctypes.c_int, [vp, vp, i64, i64,
                                                      ctypes.POINTER(KVRaggedStruct),
                                                      ctypes.POINTER(KVRaggedStruct), f32, vp, sz,
                                                      vp, i64, i64, vp, vp]),
        "nvfp4_plan_set_deferred_merge": (ctypes.c_int, [vp, i32]),
        "nvfp4_merge_partials": (ctypes.c_int, [vp, vp, sz, vp, i64, i64, vp, vp]),
        "nvfp4_merge_states": (ctypes.c_int, [vp, vp, i64, i32, i32, i32, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        if not hasattr(lib, name):
            raise ImportError(f"{LIB_PATH} does not export {name}; rebuild it with "
                              "`python attention_bit_paged_amd/build.py`")
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def check(status: int) -> None:
    if status != 0:
        raise NVFP4Error(status, lib.nvfp4_last_error().decode())
