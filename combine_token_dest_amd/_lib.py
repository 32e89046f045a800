"""ctypes binding of libmoe_ep.so: the C ABI of include/moe_ep.h, same names.

Argument marshalling only.  Every step of dispatch and combine runs in the
library's gfx950 kernels; when the library is missing, loading it raises.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import (POINTER, Structure, c_char_p, c_int, c_int32, c_int64, c_size_t, c_uint64,
                    c_void_p, byref)
from typing import List, Optional, Sequence

MOE_EP_MAX_RANKS = 64
MOE_EP_ALL_RANKS = (1 << 64) - 1

MOE_EP_OK = 0
MOE_EP_ERR_INVALID_ARG = -1
MOE_EP_ERR_STATE = -2
MOE_EP_ERR_CAPACITY = -3
MOE_EP_ERR_MASK = -4
MOE_EP_ERR_ALIGN = -5
MOE_EP_ERR_HIP = -6
MOE_EP_ERR_UNSUPPORTED = -7

MOE_EP_F32 = 0
MOE_EP_BF16 = 1
MOE_EP_F16 = 2

MOE_EP_ORDER_AUTO = 0
MOE_EP_ORDER_SOURCE_ROW = 1
MOE_EP_ORDER_DESTINATION = 2

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_ep.so")

# The exported symbols, in header order.
EXPORTS = [
    "moe_ep_is_platform_supported", "moe_ep_workspace_bytes", "moe_ep_create", "moe_ep_dispatch",
    "moe_ep_get_combine_input_buffer", "moe_ep_combine", "moe_ep_destroy",
    "moe_ep_create_vmm", "moe_ep_workspace", "moe_ep_checkpoint_prepare", "moe_ep_checkpoint_restore",
    "moe_ep_dispatch_noalloc", "moe_ep_active_rank_mask", "moe_ep_status_string", "moe_ep_last_error",
]

MOE_EP_NOALLOC_MAX_ROWS = 65536

R = MOE_EP_MAX_RANKS


class moe_ep_params(Structure):
    _fields_ = [
        ("ep_size", c_int32), ("num_experts", c_int32), ("top_k", c_int32),
        ("max_tokens_per_rank", c_int32), ("hidden_size", c_int32),
        ("combine_max_elem_bytes", c_int32), ("hidden_row_bytes", c_int64),
        ("scale_row_bytes", c_int64), ("invalid_expert_id", c_int32),
        ("enable_rank_mask", c_int32), ("eplb_stats_bytes", c_int64),
        ("dispatch_order", c_int32),
    ]


class moe_ep_dispatch_args(Structure):
    _fields_ = [
        ("hidden", c_void_p * R), ("hidden_scale", c_void_p * R), ("topk_ids", c_void_p * R),
        ("topk_weights", c_void_p * R), ("local_num_tokens", c_int32 * R),
        ("weights_present", c_uint64), ("scales_present", c_uint64),
        ("runtime_max_tokens_per_rank", c_int32), ("active_rank_mask", c_uint64),
        ("eplb_local_stats", c_void_p * R), ("eplb_present", c_uint64),
        ("local_num_tokens_device", c_void_p),
    ]


class moe_ep_dispatch_result(Structure):
    _fields_ = [
        ("hidden", c_void_p), ("hidden_scale", c_void_p), ("topk_ids", c_void_p),
        ("topk_weights", c_void_p), ("tokens_per_rank", c_int32), ("num_rows", c_int32),
        ("eplb_global_stats", c_void_p), ("dispatch_order", c_int32),
    ]


class moe_ep_combine_args(Structure):
    _fields_ = [
        ("expert_output", c_void_p * R), ("output", c_void_p * R), ("dtype", c_int32),
        ("active_rank_mask", c_uint64),
    ]


class MoeEpError(RuntimeError):
    """A non-zero status from the library."""

    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func}: {moe_ep_status_string(status)}: {detail}")
        self.status = status


_lib = None


def load(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libmoe_ep.so (built by combine_token_dest_amd.build).  Raises
    OSError when it is missing: there is no fallback path."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"{p} is missing; build it with `python -m combine_token_dest_amd.build`")
    lib = ctypes.CDLL(p)
    lib.moe_ep_is_platform_supported.argtypes = []
    lib.moe_ep_is_platform_supported.restype = c_int
    lib.moe_ep_workspace_bytes.argtypes = [POINTER(moe_ep_params), POINTER(c_size_t)]
    lib.moe_ep_workspace_bytes.restype = c_int
    lib.moe_ep_create.argtypes = [POINTER(moe_ep_params), c_void_p, c_size_t, POINTER(c_void_p)]
    lib.moe_ep_create.restype = c_int
    lib.moe_ep_dispatch.argtypes = [c_void_p, POINTER(moe_ep_dispatch_args),
                                    POINTER(moe_ep_dispatch_result), c_void_p]
    lib.moe_ep_dispatch.restype = c_int
    lib.moe_ep_get_combine_input_buffer.argtypes = [c_void_p, c_int32, c_int32, POINTER(c_void_p)]
    lib.moe_ep_get_combine_input_buffer.restype = c_int
    lib.moe_ep_combine.argtypes = [c_void_p, POINTER(moe_ep_combine_args), c_void_p]
    lib.moe_ep_combine.restype = c_int
    lib.moe_ep_destroy.argtypes = [c_void_p]
    lib.moe_ep_destroy.restype = c_int
    lib.moe_ep_create_vmm.argtypes = [POINTER(moe_ep_params), POINTER(c_void_p)]
    lib.moe_ep_create_vmm.restype = c_int
    lib.moe_ep_workspace.argtypes = [c_void_p, POINTER(c_void_p), POINTER(c_size_t)]
    lib.moe_ep_workspace.restype = c_int
    lib.moe_ep_checkpoint_prepare.argtypes = [c_void_p]
    lib.moe_ep_checkpoint_prepare.restype = c_int
    lib.moe_ep_checkpoint_restore.argtypes = [c_void_p]
    lib.moe_ep_checkpoint_restore.restype = c_int
    lib.moe_ep_dispatch_noalloc.argtypes = [c_void_p, POINTER(moe_ep_dispatch_args),
                                            POINTER(moe_ep_dispatch_result), c_void_p]
    lib.moe_ep_dispatch_noalloc.restype = c_int
    lib.moe_ep_active_rank_mask.argtypes = [POINTER(c_int32), c_int32, POINTER(c_uint64)]
    lib.moe_ep_active_rank_mask.restype = c_int
    lib.moe_ep_status_string.argtypes = [c_int]
    lib.moe_ep_status_string.restype = c_char_p
    lib.moe_ep_last_error.argtypes = []
    lib.moe_ep_last_error.restype = c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(status: int, func: str) -> None:
    if status != MOE_EP_OK:
        raise MoeEpError(status, func, moe_ep_last_error())


def moe_ep_status_string(status: int) -> str:
    return load().moe_ep_status_string(status).decode()


def moe_ep_last_error() -> str:
    return load().moe_ep_last_error().decode()


def moe_ep_is_platform_supported() -> bool:
    return bool(load().moe_ep_is_platform_supported())


def moe_ep_workspace_bytes(params: moe_ep_params) -> int:
    n = c_size_t(0)
    _check(load().moe_ep_workspace_bytes(byref(params), byref(n)), "moe_ep_workspace_bytes")
    return n.value


def moe_ep_create(params: moe_ep_params, workspace_ptr: int, workspace_bytes: int) -> int:
    h = c_void_p(0)
    _check(load().moe_ep_create(byref(params), c_void_p(workspace_ptr), workspace_bytes, byref(h)),
           "moe_ep_create")
    return h.value


def moe_ep_dispatch(handle: int, args: moe_ep_dispatch_args, ep_size: int,
                    stream: int) -> List[moe_ep_dispatch_result]:
    results = (moe_ep_dispatch_result * ep_size)()
    _check(load().moe_ep_dispatch(c_void_p(handle), byref(args), results, c_void_p(stream)),
           "moe_ep_dispatch")
    return list(results)


def moe_ep_dispatch_noalloc(handle: int, args: moe_ep_dispatch_args, ep_size: int,
                            stream: int) -> List[moe_ep_dispatch_result]:
    results = (moe_ep_dispatch_result * ep_size)()
    _check(load().moe_ep_dispatch_noalloc(c_void_p(handle), byref(args), results, c_void_p(stream)),
           "moe_ep_dispatch_noalloc")
    return list(results)


def moe_ep_get_combine_input_buffer(handle: int, rank: int, dtype: int) -> int:
    p = c_void_p(0)
    _check(load().moe_ep_get_combine_input_buffer(c_void_p(handle), rank, dtype, byref(p)),
           "moe_ep_get_combine_input_buffer")
    return p.value


def moe_ep_combine(handle: int, args: moe_ep_combine_args, stream: int) -> None:
    _check(load().moe_ep_combine(c_void_p(handle), byref(args), c_void_p(stream)), "moe_ep_combine")


def moe_ep_destroy(handle: Optional[int]) -> None:
    _check(load().moe_ep_destroy(c_void_p(handle or 0)), "moe_ep_destroy")


def moe_ep_create_vmm(params: moe_ep_params) -> int:
    h = c_void_p(0)
    _check(load().moe_ep_create_vmm(byref(params), byref(h)), "moe_ep_create_vmm")
    return h.value


def moe_ep_workspace(handle: int):
    p = c_void_p(0)
    n = c_size_t(0)
    _check(load().moe_ep_workspace(c_void_p(handle), byref(p), byref(n)), "moe_ep_workspace")
    return p.value, n.value


def moe_ep_checkpoint_prepare(handle: int) -> None:
    _check(load().moe_ep_checkpoint_prepare(c_void_p(handle)), "moe_ep_checkpoint_prepare")


def moe_ep_checkpoint_restore(handle: int) -> None:
    _check(load().moe_ep_checkpoint_restore(c_void_p(handle)), "moe_ep_checkpoint_restore")


def moe_ep_active_rank_mask(ranks: Sequence[int]) -> int:
    arr = (c_int32 * max(1, len(ranks)))(*[int(r) for r in ranks])
    out = c_uint64(0)
    _check(load().moe_ep_active_rank_mask(arr, len(ranks), byref(out)), "moe_ep_active_rank_mask")
    return out.value
