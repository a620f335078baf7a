"""ctypes declarations of the C ABI in include/qlinear.h (argument marshalling only)."""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libqlinear.so")

c_i32, c_i64, c_vp, c_cp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_char_p


class QLConfig(ctypes.Structure):
    _fields_ = [(n, c_i32) for n in ("algo", "swap_ab", "split_k", "waves_n", "waves_k", "rows_per_wave",
                                     "prefetch", "a_mode", "w_lds", "w_layout", "tile_m", "tile_n")]


class QLPlanFacts(ctypes.Structure):
    _fields_ = [("source", c_i32), ("chunks", c_i32), ("chunk_k", c_i32), ("workgroups", c_i32),
                ("threads", c_i32), ("lds_bytes", c_i32), ("workspace_bytes", c_i64), ("epilogue", c_i32)]


# name -> (restype, argtypes); exactly the functions declared in include/qlinear.h
SIGNATURES = {
    "qlinear_version": (c_i32, []),
    "qlinear_status_string": (c_cp, [c_i32]),
    "qlinear_last_error": (c_cp, []),
    "qlinear_quantize_act": (c_i32, [c_i32, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "qlinear_quantize_weight": (c_i32, [c_i32, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "qlinear_packed_act_bytes": (c_i64, [c_i64, c_i64]),
    "qlinear_quantize_act_packed": (c_i32, [c_i32, c_vp, c_i64, c_i64, c_vp, c_vp, c_vp]),
    "qlinear_packed_weight_bytes": (c_i64, [c_i64, c_i64]),
    "qlinear_encode_e4m3": (c_i32, [c_vp, c_i64, c_vp, c_vp]),
    "qlinear_stream_read": (c_i32, [c_vp, c_i64, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "qlinear_stream_read_bcast": (c_i32, [c_vp, c_i64, c_vp, c_i64, c_i32, c_i32, c_i32, c_i32, c_vp, c_vp]),
    "qlinear_pack_weight": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_vp]),
    "qlinear_packed_mx_scale_bytes": (c_i64, [c_i64, c_i64]),
    "qlinear_packed_weight_bytes_fp4": (c_i64, [c_i64, c_i64]),
    "qlinear_pack_weight_fp4": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_vp]),
    "qlinear_pack_mx_scales": (c_i32, [c_vp, c_i64, c_i64, c_vp, c_vp]),
    "qlinear_table_load": (c_i32, [c_cp, ctypes.POINTER(c_i64)]),
    "qlinear_table_clear": (None, []),
    "qlinear_plan": (c_i32, [c_i32, c_i64, c_i64, c_i64, ctypes.POINTER(c_vp)]),
    "qlinear_plan_packed": (c_i32, [c_i32, c_i64, c_i64, c_i64, ctypes.POINTER(c_vp)]),
    "qlinear_plan_layouts": (c_i32, [c_i32, c_i64, c_i64, c_i64, c_i32, c_i32, ctypes.POINTER(c_vp)]),
    "qlinear_plan_from_table": (c_i32, [c_i32, c_i64, c_i64, c_i64, ctypes.POINTER(c_vp)]),
    "qlinear_plan_with_config": (c_i32, [c_i32, c_i64, c_i64, c_i64, ctypes.POINTER(QLConfig),
                                         ctypes.POINTER(c_vp)]),
    "qlinear_plan_info": (c_i32, [c_vp, ctypes.POINTER(QLConfig), ctypes.POINTER(QLPlanFacts)]),
    "qlinear_plan_glu": (c_i32, [c_i32, c_i64, c_i64, c_i64, c_i32, ctypes.POINTER(c_vp)]),
    "qlinear_plan_glu_with_config": (c_i32, [c_i32, c_i64, c_i64, c_i64, ctypes.POINTER(QLConfig),
                                             ctypes.POINTER(c_vp)]),
    "qlinear_workspace_bytes": (c_i64, [c_vp]),
    "qlinear_plan_destroy": (None, [c_vp]),
    "qlinear_run": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "qlinear_run_debug_acc": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "qlinear_forward": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "qlinear_forward_noalloc": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "qlinear_forward_glu_amax": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "qlinear_forward_amax": (c_i32, [c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp, c_vp]),
    "qlinear_graph_begin": (c_i32, [c_vp]),
    "qlinear_graph_end": (c_i32, [c_vp, ctypes.POINTER(c_vp)]),
    "qlinear_graph_launch": (c_i32, [c_vp, c_vp]),
    "qlinear_graph_destroy": (None, [c_vp]),
}

_lib = None


def load(path=LIB_PATH):
    """Load libqlinear.so (built in-tree) and declare every exported function.

    Raises OSError when the library is missing: there is no fallback path.
    """
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise OSError("libqlinear.so is not built (%s); run python -m quantized_gemm_decode_amd.build" % path)
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
