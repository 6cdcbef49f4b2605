"""ctypes declarations of the C ABI in include/moe.h (libmoe.so).

Loading fails loudly: there is no fallback implementation of any entry point.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH = range(5)
MOE_F32, MOE_BF16, MOE_MXFP8, MOE_FP8 = 0, 1, 2, 3
MOE_OP_PERMUTE, MOE_OP_MLP_FWD, MOE_OP_MLP_BWD, MOE_OP_GROUPED_GEMM, MOE_OP_ROUTER_BWD = 0, 1, 2, 3, 4
MOE_MAX_EXPERTS = 256

# every symbol include/moe.h declares
EXPORTS = (
    "moe_route_topk", "moe_router_logits", "moe_route_topk_bwd", "moe_router_bwd",
    "moe_permute", "moe_permute_noalloc", "moe_unpermute_combine", "mxfp8_quantize", "fp8_tensor_quantize", "mxfp8_quantize_colwise",
    "fp8_tensor_quantize_colwise", "fp8_tensor_pack_weight_bwd",
    "mxfp8_pack_weight_bwd", "mxfp8_quantize_weights", "fp8_tensor_quantize_weights",
    "moe_grouped_mlp_fwd", "moe_grouped_mlp_bwd", "moe_grouped_linear", "moe_grouped_gate_up_swiglu",
    "moe_workspace_size",
    "moe_status_str", "moe_last_error",
)


class MlpDesc(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int), ("H", ctypes.c_int), ("I", ctypes.c_int),
                ("compute", ctypes.c_int), ("act", ctypes.c_int), ("wt", ctypes.c_int),
                ("save_for_bwd", ctypes.c_int)]


class MoeError(RuntimeError):
    def __init__(self, fn, status, detail):
        super().__init__(f"{fn} failed: status {status} ({detail})")
        self.status = status


_lock = threading.Lock()
_lib = None

vp, i64, c_int, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
PP = ctypes.POINTER(ctypes.c_void_p)


def _declare(lib):
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_status_str.argtypes = [c_int]
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_last_error.argtypes = []
    sig = {
        "moe_route_topk": [vp, i64, c_int, c_int, c_int, vp, vp, vp],
        "moe_router_logits": [vp, vp, i64, c_int, c_int, vp, vp],
        "moe_route_topk_bwd": [vp, vp, vp, vp, i64, c_int, c_int, c_int, vp, vp],
        "moe_router_bwd": [vp, vp, vp, vp, i64, c_int, c_int, vp, vp, vp, sz, vp],
        "moe_permute": [vp, vp, c_int, i64, c_int, c_int, c_int, vp, vp, c_int, vp, vp, vp, vp, vp, vp, vp,
                        vp, sz, vp],
        "moe_permute_noalloc": [vp, vp, c_int, i64, c_int, c_int, c_int, vp, vp, c_int, vp, vp, vp, vp, vp, vp,
                                vp, vp],
        "moe_unpermute_combine": [vp, c_int, vp, vp, i64, c_int, c_int, vp, vp],
        "mxfp8_quantize": [vp, i64, i64, vp, vp, vp],
        "fp8_tensor_quantize": [vp, i64, vp, vp, vp],
        "mxfp8_quantize_colwise": [vp, i64, i64, c_int, vp, c_int, i64, vp, vp, vp, vp],
        "fp8_tensor_quantize_colwise": [vp, i64, i64, c_int, vp, c_int, i64, vp, vp, vp, vp],
        "fp8_tensor_pack_weight_bwd": [vp, i64, i64, vp, vp],
        "mxfp8_pack_weight_bwd": [vp, i64, i64, vp, vp],
        "mxfp8_quantize_weights": [c_int, PP, i64, i64, PP, PP, PP, vp],
        "fp8_tensor_quantize_weights": [c_int, PP, i64, i64, PP, vp, PP, vp],
        "moe_grouped_mlp_fwd": [ctypes.POINTER(MlpDesc), i64, vp, vp, PP, PP, PP, PP, vp, vp, vp, vp, vp, vp,
                                sz, vp],
        "moe_grouped_mlp_bwd": [ctypes.POINTER(MlpDesc), i64, vp, vp, vp, vp, vp, PP, PP, vp, vp, PP, PP, vp,
                                vp, sz, vp],
        "moe_grouped_linear": [c_int, i64, c_int, c_int, c_int, vp, PP, vp, vp, vp, sz, vp],
        "moe_grouped_gate_up_swiglu": [c_int, i64, c_int, c_int, c_int, vp, vp, PP, PP, vp, vp, vp, vp, vp, vp, sz,
                                       vp],
        "moe_workspace_size": [c_int, ctypes.POINTER(MlpDesc), i64, i64, c_int, c_int, ctypes.POINTER(sz)],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = c_int


def lib():
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m grouped_expert_gemm_amd.build` "
                    "(the MoE path has no fallback)")
            h = ctypes.CDLL(LIB_PATH)
            _declare(h)
            _lib = h
        return _lib


def check(fn_name: str, status: int):
    if status != MOE_OK:
        L = lib()
        raise MoeError(fn_name, status, f"{L.moe_status_str(status).decode()}: {L.moe_last_error().decode()}")


def ptr_table(ptrs):
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    return ctypes.cast(arr, PP), arr
