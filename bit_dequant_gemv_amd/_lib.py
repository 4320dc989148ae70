"""ctypes view of libbdg's C ABI (``include/bdg.h``).

Only argument marshalling lives here.  Loading fails loudly when the built
library is missing: there is no CPU fallback.
"""

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbdg.so")

BDG_OK = 0
BDG_E_INVALID = -1
BDG_E_ALIGN = -2
BDG_E_UNSUPPORTED = -3
BDG_E_HIP = -4
BDG_E_NOMEM = -5
BDG_E_TOO_LARGE = -6
BDG_E_WAIT = -7
BDG_ATTN_SCRATCH_BYTES = 8 * 1024 * 1024

BDG_F32 = 0
BDG_BF16 = 1
BDG_FMT_MXFP4 = 0
BDG_FMT_INT4G = 1
BDG_ROUTER_RMSNORM = 1
BDG_MOE_STACK = 1
BDG_MOE_NO_GRAPH = 2
BDG_MOE_ROUTE_EVERY_LAYER = 4
BDG_MOE_PER_TOKEN = 8
BDG_MOE_FUSED_LAYER = 16
BDG_MOE_MFMA = 32
BDG_MOE_ROUTE_KERNEL = 64
BDG_MAX_M = 16

# every symbol include/bdg.h declares
EXPORTED = (
    "mxfp4_dequant", "int4g_dequant", "qgemv", "moe_router_topk",
    "moe_plan_create", "moe_plan_destroy", "moe_plan_check", "moe_expert_decode", "moe_experts_routed",
    "moe_expert_decode_profiled", "moe_expert_decode_timeline", "mxfp8_quantize", "mx_scale_words_bytes",
    "mx_stage_scales", "mx_gemm_workspace", "mx_gemm",
    "moe_prefill_mx_workspace",
    "moe_prefill_mx", "attn_rope_table", "attn_decode_workspace", "attn_decode", "attn_decode_noalloc",
    "bdg_stream_read", "bdg_stream_copy", "bdg_strerror", "bdg_version",
)


class BdgError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


class QMat(ctypes.Structure):
    _fields_ = [
        ("fmt", ctypes.c_int32), ("group", ctypes.c_int32),
        ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
        ("expert_stride_codes", ctypes.c_int64), ("expert_stride_scales", ctypes.c_int64),
        ("expert_stride_zeros", ctypes.c_int64), ("mx_scale_words", ctypes.c_void_p),
    ]


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("w_router", ctypes.c_void_p), ("b_router", ctypes.c_void_p),
        ("gate_up", QMat), ("down", QMat),
    ]


class MoEDesc(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
        ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32), ("fmt", ctypes.c_int32),
        ("group", ctypes.c_int32), ("flags", ctypes.c_int32), ("norm_eps", ctypes.c_float),
        ("max_m", ctypes.c_int32), ("layers", ctypes.POINTER(LayerDesc)),
        ("wait_polls", ctypes.c_int32),
    ]


class Rope(ctypes.Structure):
    _fields_ = [
        ("theta", ctypes.c_double), ("factor", ctypes.c_double),
        ("beta_fast", ctypes.c_double), ("beta_slow", ctypes.c_double),
        ("orig_ctx", ctypes.c_int32), ("truncate", ctypes.c_int32),
    ]


_lib = None


def load():
    """The loaded libbdg (ctypes.CDLL) with argument types set."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(the HIP library is required; there is no CPU path)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sig = {
        "mxfp4_dequant": [vp, vp, i64, i64, vp, i32, vp],
        "int4g_dequant": [vp, vp, vp, i64, i64, i32, vp, vp],
        "qgemv": [ctypes.POINTER(QMat), vp, i32, i32, vp, vp],
        "moe_router_topk": [vp, i32, vp, vp, i32, i32, i32, i32, i32, f32, vp, vp, vp, vp],
        "moe_plan_create": [ctypes.POINTER(MoEDesc), ctypes.POINTER(vp)],
        "moe_plan_destroy": [vp],
        "moe_plan_check": [vp, vp],
        "moe_expert_decode": [vp, vp, i32, i32, vp, vp, vp, vp, vp],
        "moe_experts_routed": [vp, i32, vp, i32, i32, vp, vp, vp, vp],
        "moe_expert_decode_profiled": [vp, vp, i32, i32, vp, vp, vp, vp],
        "moe_expert_decode_timeline": [vp, vp, i32, vp, vp, i64, vp],
        "mxfp8_quantize": [vp, i32, i64, i64, vp, vp, vp],
        "mx_scale_words_bytes": [ctypes.POINTER(QMat), i32],
        "mx_stage_scales": [ctypes.POINTER(QMat), i32, vp, i64, vp],
        "mx_gemm_workspace": [i64, i64, i64],
        "mx_gemm": [ctypes.POINTER(QMat), vp, vp, i64, vp, vp, i64, vp],
        "moe_prefill_mx_workspace": [i64, i32, i32, i32, i32],
        "moe_prefill_mx": [ctypes.POINTER(LayerDesc), i32, i32, vp, i32, i64, vp, vp, vp, vp, i64, vp],
        "attn_rope_table": [ctypes.POINTER(Rope), i32, i64, vp, vp, vp, vp],
        "attn_decode_workspace": [i32, i32, i32, i32, i64],
        "attn_decode": [vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i64, vp, i64, f32, vp, i32, vp, vp,
                        i64, vp],
        "attn_decode_noalloc": [vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, i32, i64, vp, i64, f32, vp, i32, vp,
                                vp],
        "bdg_stream_read": [vp, i64, vp, i32, vp],
        "bdg_stream_copy": [vp, vp, i64, vp],
        "bdg_strerror": [i32],
        "bdg_version": [],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = (ctypes.c_char_p if name in ("bdg_strerror", "bdg_version")
                      else ctypes.c_int64 if name in ("moe_prefill_mx_workspace", "mx_gemm_workspace",
                                                      "mx_scale_words_bytes", "attn_decode_workspace",
                                                      "moe_expert_decode_timeline")
                      else ctypes.c_int)
    _lib = lib
    return lib


def check(fn_name, status):
    if status != BDG_OK:
        msg = load().bdg_strerror(status).decode()
        raise BdgError(fn_name, status, msg)
