"""ctypes binding of libjattn.so.  Argument marshalling only: every step of
the computation runs inside the HIP library.

Functions keep the C names (see include/jattn.h for argument meaning, layout,
ownership and error behaviour).  A non-zero status raises JattnError.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjattn.so")

# constants mirrored from include/jattn.h
JATTN_OK = 0
JATTN_E_NULL, JATTN_E_OFFSETS, JATTN_E_SHAPE, JATTN_E_UNSUPPORTED = -1, -2, -3, -4
JATTN_E_ALIGN, JATTN_E_WORKSPACE, JATTN_E_STATE, JATTN_E_HIP, JATTN_E_ARG = -5, -6, -7, -8, -9
JATTN_SOFTMAX, JATTN_GELU_ERF, JATTN_SILU, JATTN_GELU_POLY = 0, 1, 2, 3
JATTN_MASK_NONE, JATTN_MASK_BLOCKDIAG64, JATTN_MASK_WINDOW = 0, 1, 2
JATTN_BF16, JATTN_F32, JATTN_MXFP8 = 0, 1, 2
JATTN_MX_Q, JATTN_MX_KV = 0, 1
JATTN_HEAVY_FIRST, JATTN_ZIGZAG, JATTN_LPT = 0, 1, 2
JATTN_PLAN_FWD, JATTN_PLAN_DKDV, JATTN_PLAN_DQ, JATTN_PLAN_BLOCK = 0, 1, 2, 3

JATTN_BWD_PREP, JATTN_BWD_DKDV, JATTN_BWD_DQ, JATTN_BWD_ALL = 1, 2, 4, 7

EXPORTED = ["jattn_plan_create", "jattn_plan_info", "jattn_plan_export", "jattn_plan_upload",
            "jattn_fwd", "jattn_bwd", "jattn_bwd_stages", "jattn_bwd_fixed_scratch", "jattn_plan_destroy",
            "jattn_strerror", "jattn_last_error", "jattn_l2norm_fwd", "jattn_l2norm_bwd", "jattn_mx_sizes",
            "jattn_mx_quantize", "jattn_mx_fwd", "jattn_mx_bwd"]


class JattnError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"jattn error {code}: {msg}")
        self.code = code


class jattn_desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("D", ctypes.c_int32),
                ("scale", ctypes.c_float), ("act", ctypes.c_int32), ("mask", ctypes.c_int32),
                ("has_bias", ctypes.c_int32), ("want_dbias", ctypes.c_int32),
                ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
                ("grad_dtype", ctypes.c_int32), ("split_operands", ctypes.c_int32),
                ("order", ctypes.c_int32), ("num_workers", ctypes.c_int32),
                ("dbias_dtype", ctypes.c_int32), ("window_left", ctypes.c_int32),
                ("window_right", ctypes.c_int32), ("rope", ctypes.c_int32), ("rope_base", ctypes.c_float)]


class jattn_mx_tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("codes_t", ctypes.c_void_p), ("scales", ctypes.c_void_p)]


class jattn_kernel_plan(ctypes.Structure):
    _fields_ = [("tile_rows", ctypes.c_int32), ("step_rows", ctypes.c_int32),
                ("num_workers", ctypes.c_int32), ("n_units", ctypes.c_int32)]


class jattn_plan_summary(ctypes.Structure):
    _fields_ = [("workspace_bytes", ctypes.c_int64), ("Tq", ctypes.c_int64), ("Tk", ctypes.c_int64),
                ("bias_elems", ctypes.c_int64), ("flops_fwd", ctypes.c_double),
                ("flops_bwd", ctypes.c_double), ("fwd", jattn_kernel_plan),
                ("dkdv", jattn_kernel_plan), ("dq", jattn_kernel_plan), ("block", jattn_kernel_plan)]


_lib = None


def lib():
    """Load libjattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m jagged_variable_length_amd.build` (no fallback exists)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.jattn_plan_create.argtypes = [ctypes.POINTER(jattn_desc), ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(vp)]
    L.jattn_plan_info.argtypes = [vp, ctypes.POINTER(jattn_plan_summary)]
    L.jattn_plan_export.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_int32), i64, ctypes.POINTER(i64)]
    L.jattn_plan_upload.argtypes = [vp, vp, i64, vp]
    L.jattn_fwd.argtypes = [vp] * 9
    L.jattn_bwd.argtypes = [vp] * 14
    L.jattn_bwd_stages.argtypes = [vp, i32] + [vp] * 13
    L.jattn_bwd_fixed_scratch.argtypes = [vp] * 14
    L.jattn_plan_destroy.argtypes = [vp]
    L.jattn_plan_destroy.restype = None
    L.jattn_strerror.argtypes = [ctypes.c_int]
    L.jattn_strerror.restype = ctypes.c_char_p
    L.jattn_last_error.argtypes = []
    L.jattn_last_error.restype = ctypes.c_char_p
    L.jattn_l2norm_fwd.argtypes = [vp, vp, vp, i64, i32, i32, i32, vp]
    L.jattn_l2norm_bwd.argtypes = [vp, vp, vp, i64, i32, i32, i32, i32, vp]
    mxp = ctypes.POINTER(jattn_mx_tensor)
    L.jattn_mx_sizes.argtypes = [vp, i32, ctypes.POINTER(i64), ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.jattn_mx_quantize.argtypes = [vp, i32, vp, mxp, vp, vp]
    L.jattn_mx_fwd.argtypes = [vp, mxp, mxp, mxp, vp, vp, vp, vp]
    L.jattn_mx_bwd.argtypes = [vp, i32, mxp, mxp, mxp, vp, vp, mxp, vp, vp, vp, vp, vp]
    for name in ["jattn_plan_create", "jattn_plan_info", "jattn_plan_export", "jattn_plan_upload",
                 "jattn_fwd", "jattn_bwd", "jattn_bwd_stages", "jattn_bwd_fixed_scratch", "jattn_l2norm_fwd",
                 "jattn_l2norm_bwd", "jattn_mx_sizes", "jattn_mx_quantize", "jattn_mx_fwd", "jattn_mx_bwd"]:
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _check(code):
    if code != JATTN_OK:
        L = lib()
        raise JattnError(code, f"{L.jattn_strerror(code).decode()}: {L.jattn_last_error().decode()}")


def _offsets(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))


def jattn_plan_create(desc: jattn_desc, q_offsets, kv_offsets) -> int:
    qa, qp = _offsets(q_offsets)
    ka, kp = _offsets(kv_offsets)
    h = ctypes.c_void_p()
    _check(lib().jattn_plan_create(ctypes.byref(desc), qp, kp, ctypes.byref(h)))
    return h.value


def jattn_plan_info(plan: int) -> jattn_plan_summary:
    s = jattn_plan_summary()
    _check(lib().jattn_plan_info(plan, ctypes.byref(s)))
    return s


def jattn_plan_export(plan: int, which: int) -> np.ndarray:
    n = ctypes.c_int64()
    _check(lib().jattn_plan_export(plan, which, None, 0, ctypes.byref(n)))
    out = np.zeros(max(n.value, 1), dtype=np.int32)
    _check(lib().jattn_plan_export(plan, which, out.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                                   out.size, ctypes.byref(n)))
    return out[:n.value]


def jattn_plan_upload(plan: int, workspace: int, workspace_bytes: int, stream: int) -> None:
    _check(lib().jattn_plan_upload(plan, workspace, workspace_bytes, stream))


def jattn_fwd(plan, q, k, v, bias, o, lse, workspace, stream) -> None:
    _check(lib().jattn_fwd(plan, q, k, v, bias, o, lse, workspace, stream))


def jattn_bwd(plan, q, k, v, bias, o, lse, dout, dq, dk, dv, dbias, workspace, stream) -> None:
    _check(lib().jattn_bwd(plan, q, k, v, bias, o, lse, dout, dq, dk, dv, dbias, workspace, stream))


def jattn_bwd_stages(plan, stages, q, k, v, bias, o, lse, dout, dq, dk, dv, dbias, workspace, stream) -> None:
    _check(lib().jattn_bwd_stages(plan, stages, q, k, v, bias, o, lse, dout, dq, dk, dv, dbias, workspace, stream))


def jattn_bwd_fixed_scratch(plan, q, k, v, bias, o, lse, dout, dq, dk, dv, dbias, workspace, stream) -> None:
    _check(lib().jattn_bwd_fixed_scratch(plan, q, k, v, bias, o, lse, dout, dq, dk, dv, dbias, workspace, stream))


def jattn_mx_sizes(plan, rows):
    """(codes, codes_t, scales) byte sizes of an MXFP8 tensor of the plan."""
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(lib().jattn_mx_sizes(plan, rows, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def jattn_mx_quantize(plan, rows, x, out: jattn_mx_tensor, workspace, stream) -> None:
    _check(lib().jattn_mx_quantize(plan, rows, x, ctypes.byref(out), workspace, stream))


def jattn_mx_fwd(plan, q: jattn_mx_tensor, k: jattn_mx_tensor, v: jattn_mx_tensor, o, lse, workspace,
                 stream) -> None:
    _check(lib().jattn_mx_fwd(plan, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), o, lse, workspace, stream))


def jattn_mx_bwd(plan, stages, q: jattn_mx_tensor, k: jattn_mx_tensor, v: jattn_mx_tensor, o, lse,
                 dout: jattn_mx_tensor, dq, dk, dv, workspace, stream) -> None:
    _check(lib().jattn_mx_bwd(plan, stages, ctypes.byref(q), ctypes.byref(k), ctypes.byref(v), o, lse,
                              ctypes.byref(dout), dq, dk, dv, workspace, stream))


def jattn_l2norm_fwd(x, y, rnorm, rows, D, x_dtype, y_dtype, stream) -> None:
    _check(lib().jattn_l2norm_fwd(x, y, rnorm, rows, D, x_dtype, y_dtype, stream))


def jattn_l2norm_bwd(x, dy, dx, rows, D, x_dtype, dy_dtype, dx_dtype, stream) -> None:
    _check(lib().jattn_l2norm_bwd(x, dy, dx, rows, D, x_dtype, dy_dtype, dx_dtype, stream))


def jattn_plan_destroy(plan: int) -> None:
    if plan:
        lib().jattn_plan_destroy(plan)


def jattn_strerror(code: int) -> str:
    return lib().jattn_strerror(code).decode()


def jattn_last_error() -> str:
    return lib().jattn_last_error().decode()
