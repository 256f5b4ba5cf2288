"""ctypes declarations of the C ABI in include/mok.h, and the library loader.

The loader fails loudly when ``libmok.so`` is missing: there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmok.so")

MOK_OK = 0
MOK_ERR_INVALID_ARGUMENT = 1
MOK_ERR_UNSUPPORTED = 2
MOK_ERR_CONFIG_MISMATCH = 3
MOK_ERR_BUFFER_TOO_SMALL = 4
MOK_ERR_HIP = 5

MOK_MODE_BF16 = 0
MOK_MODE_MXFP8 = 1

# Every symbol include/mok.h declares (checked by the CPU tests).
EXPORTS = (
    "mok_status_string", "mok_validate_config", "mok_schedule_bytes", "mok_schedule_layout_query",
    "mok_context_bytes", "mok_workspace_bytes", "mok_workspace_create", "mok_workspace_destroy",
    "mok_build_schedule", "mok_forward", "mok_forward_static", "mok_backward", "mok_mxfp8_quantize", "mok_mxfp8_quantize_transposed", "mok_kernel_name",
    "mok_workspace_set_timing", "mok_workspace_set_timing_mask", "mok_workspace_read_timing",
    "mok_workspace_read_status",
)

HDR_FIELDS = ("T", "k", "E", "C", "P", "rows_cap", "n_mb", "minibatch", "dropped", "invalid",
              "rows_total", "hash")
KERNEL_COUNT = 17
TILE_BMS = (32, 64, 128, 256)


class MokConfig(C.Structure):
    _fields_ = [
        ("struct_size", C.c_uint32),
        ("hidden", C.c_int32),
        ("intermediate", C.c_int32),
        ("num_experts", C.c_int32),
        ("topk", C.c_int32),
        ("shared_intermediate", C.c_int32),
        ("max_tokens", C.c_int64),
        ("capacity_multiplier", C.c_float),
        ("expert_pad", C.c_int32),
        ("minibatch_size", C.c_int32),
        ("num_mover_wgs", C.c_int32),
        ("swiglu_limit", C.c_float),
        ("macrobatch_size", C.c_int32),
        ("forward_only", C.c_int32),
    ]


class MokWeights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "routed_gate", "routed_up", "routed_down", "shared_gate", "shared_up", "shared_down",
        "routed_gate_scale", "routed_up_scale", "routed_down_scale",
        "shared_gate_scale", "shared_up_scale", "shared_down_scale")]


class MokGrads(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in (
        "dx", "d_router_weights", "d_routed_gate", "d_routed_up", "d_routed_down",
        "d_shared_gate", "d_shared_up", "d_shared_down")]


class MokScheduleLayout(C.Structure):
    _fields_ = [(n, C.c_size_t) for n in (
        "total_bytes", "header", "counts", "kept", "offsets", "mb_offsets", "row_src", "slot_row", "tiles")] + [
        ("rows_cap_max", C.c_int64), ("n_mb_max", C.c_int64)]


_lib = None


def load() -> C.CDLL:
    """Loads libmok.so once. Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mixture_experts_layer_build_amd.build` (there is no fallback path)")
    lib = C.CDLL(LIB_PATH)
    vp, sz, i64, i32 = C.c_void_p, C.c_size_t, C.c_int64, C.c_int
    cfgp = C.POINTER(MokConfig)
    sig = {
        "mok_status_string": (C.c_char_p, [i32]),
        "mok_validate_config": (i32, [cfgp]),
        "mok_schedule_bytes": (sz, [cfgp]),
        "mok_schedule_layout_query": (i32, [cfgp, C.POINTER(MokScheduleLayout)]),
        "mok_context_bytes": (sz, [cfgp, i32]),
        "mok_workspace_bytes": (sz, [cfgp]),
        "mok_workspace_create": (i32, [cfgp, i32, C.POINTER(vp)]),
        "mok_workspace_destroy": (i32, [vp]),
        "mok_build_schedule": (i32, [vp, vp, i64, vp, sz, vp]),
        "mok_forward": (i32, [vp, i32, vp, sz, vp, vp, C.POINTER(MokWeights), vp, vp, sz, vp]),
        "mok_forward_static": (i32, [cfgp, i32, vp, sz, vp, vp, C.POINTER(MokWeights), vp, vp]),
        "mok_backward": (i32, [vp, i32, vp, sz, vp, sz, vp, vp, vp, C.POINTER(MokWeights),
                               C.POINTER(MokGrads), vp]),
        "mok_mxfp8_quantize": (i32, [vp, i32, i64, i64, i64, i32, vp, i64, vp, vp]),
        "mok_mxfp8_quantize_transposed": (i32, [vp, i64, i64, i64, vp, vp, vp]),
        "mok_kernel_name": (C.c_char_p, [i32]),
        "mok_workspace_set_timing": (i32, [vp, i32]),
        "mok_workspace_set_timing_mask": (i32, [vp, C.c_uint32]),
        "mok_workspace_read_timing": (i32, [vp, C.POINTER(C.c_float), C.POINTER(i64), i32]),
        "mok_workspace_read_status": (i32, [vp, C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


class MokError(RuntimeError):
    def __init__(self, call: str, status: int):
        name = load().mok_status_string(status).decode()
        super().__init__(f"{call} failed: {name} ({status})")
        self.status = status


def check(call: str, status: int) -> None:
    if status != MOK_OK:
        raise MokError(call, status)
