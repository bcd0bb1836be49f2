"""Thin ctypes binding of libqgemm (include/qgemm.h), same names as the C ABI.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libqgemm.so.  Device buffers are passed as integer addresses
(e.g. ``tensor.data_ptr()``) and streams as integer handles
(``torch.cuda.current_stream().cuda_stream``).  If the library has not been
built this module raises on first use; there is no other implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemm.so")

DTYPES = {"f16": 1, "f32": 2, "i32": 3, "i8": 4, "i4": 5, "u4": 6, "i2": 7}
STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported format or shape",
          3: "out of host memory", 4: "device launch failed"}
QGEMM_OK, QGEMM_ERR_INVALID_ARG, QGEMM_ERR_UNSUPPORTED, QGEMM_ERR_NO_MEMORY, QGEMM_ERR_DEVICE = range(5)
QGEMM_DETERMINISTIC = 1
QGEMM_SPLIT_AUTO = 2
QGEMM_PATH_GEMV, QGEMM_PATH_MFMA = 1, 2

EXPORTED = ("qgemm_create", "qgemm_pack_weights", "qgemm_run", "qgemm_run_ex", "qgemm_run_noalloc",
            "qgemm_run_scaled", "qgemm_quantize_rows", "qgemm_destroy", "qgemm_plan_path",
            "qgemm_status_string")
NOALLOC_MAX_SCRATCH = 32 << 20


class QGemmError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)} (status {status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libqgemm.so (built in-tree by weight_quantized_mixed_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    # Device buffers and streams come from PyTorch, so libqgemm must bind to the
    # HIP runtime torch already loaded (torch ships its own libamdhip64); loading
    # libqgemm first would bring in a second runtime that cannot use torch's streams.
    try:
        import torch  # noqa: F401
    except ImportError:  # pragma: no cover - the binding is still usable from C pointers
        pass
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: build it with `python -m weight_quantized_mixed_amd.build`")
    lib = ctypes.CDLL(path)
    c_i64, c_i32, c_u32, c_p, c_sz = (ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32,
                                      ctypes.c_void_p, ctypes.c_size_t)
    lib.qgemm_create.argtypes = [ctypes.POINTER(c_p), c_i64, c_i64, c_i64, c_i32, c_i32, c_i32,
                                 c_i32, c_i32, c_i32, c_i32, c_u32,
                                 ctypes.POINTER(c_sz), ctypes.POINTER(c_sz)]
    lib.qgemm_create.restype = c_i32
    lib.qgemm_pack_weights.argtypes = [c_p, c_p, c_p, c_p, c_p, c_p]
    lib.qgemm_pack_weights.restype = c_i32
    lib.qgemm_run.argtypes = [c_p, c_p, c_p, c_p, c_p, c_sz, c_p]
    lib.qgemm_run.restype = c_i32
    lib.qgemm_run_ex.argtypes = [c_p, c_i64, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]
    lib.qgemm_run_ex.restype = c_i32
    lib.qgemm_run_noalloc.argtypes = [c_p, c_i64, c_p, c_p, c_p, c_p, c_p]
    lib.qgemm_run_noalloc.restype = c_i32
    lib.qgemm_run_scaled.argtypes = [c_p, c_i64, c_p, c_p, c_p, c_p, c_p, c_p, c_p, c_sz, c_p]
    lib.qgemm_run_scaled.restype = c_i32
    lib.qgemm_quantize_rows.argtypes = [c_p, c_i64, c_i64, c_p, c_p, c_p]
    lib.qgemm_quantize_rows.restype = c_i32
    lib.qgemm_destroy.argtypes = [c_p]
    lib.qgemm_destroy.restype = None
    lib.qgemm_plan_path.argtypes = [c_p]
    lib.qgemm_plan_path.restype = c_i32
    lib.qgemm_status_string.argtypes = [c_i32]
    lib.qgemm_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _dt(x) -> int:
    return DTYPES[x] if isinstance(x, str) else int(x)


def qgemm_create(M, N, K, a_dtype, w_dtype, out_dtype, accum_dtype, group_size=0,
                 has_zeros=0, k_parts=1, flags=0):
    """Returns (plan handle, packed_bytes, workspace_bytes); raises QGemmError."""
    lib = load()
    plan = ctypes.c_void_p()
    pb, wb = ctypes.c_size_t(), ctypes.c_size_t()
    st = lib.qgemm_create(ctypes.byref(plan), int(M), int(N), int(K), _dt(a_dtype), _dt(w_dtype),
                          _dt(out_dtype), _dt(accum_dtype), int(group_size), int(has_zeros),
                          int(k_parts), int(flags), ctypes.byref(pb), ctypes.byref(wb))
    if st != QGEMM_OK:
        raise QGemmError(st, "qgemm_create")
    return plan.value, pb.value, wb.value


def qgemm_pack_weights(plan, w, scales, zeros, packed, stream=0):
    st = load().qgemm_pack_weights(plan, w or None, scales or None, zeros or None, packed or None,
                                   stream or None)
    if st != QGEMM_OK:
        raise QGemmError(st, "qgemm_pack_weights")


def qgemm_run(plan, A, packed, C, workspace, workspace_bytes, stream=0):
    st = load().qgemm_run(plan, A or None, packed or None, C or None, workspace or None,
                          int(workspace_bytes), stream or None)
    if st != QGEMM_OK:
        raise QGemmError(st, "qgemm_run")


def qgemm_run_ex(plan, M, A, packed, bias, C, workspace, workspace_bytes, stream=0):
    st = load().qgemm_run_ex(plan, int(M), A or None, packed or None, bias or None, C or None,
                             workspace or None, int(workspace_bytes), stream or None)
    if st != QGEMM_OK:
        raise QGemmError(st, "qgemm_run_ex")


def qgemm_run_noalloc(plan, M, A, packed, bias, C, stream=0):
    st = load().qgemm_run_noalloc(plan, int(M), A or None, packed or None, bias or None, C or None,
                                  stream or None)
    if st != QGEMM_OK:
        raise QGemmError(st, "qgemm_run_noalloc")


def qgemm_run_scaled(plan, M, A, packed, row_scales, col_scales, bias, C, workspace, workspace_bytes,
                     stream=0):
    st = load().qgemm_run_scaled(plan, int(M), A or None, packed or None, row_scales or None,
                                 col_scales or None, bias or None, C or None, workspace or None,
                                 int(workspace_bytes), stream or None)
    if st != QGEMM_OK:
        raise QGemmError(st, "qgemm_run_scaled")


def qgemm_quantize_rows(A, M, K, Q, scales, stream=0):
    st = load().qgemm_quantize_rows(A or None, int(M), int(K), Q or None, scales or None, stream or None)
    if st != QGEMM_OK:
        raise QGemmError(st, "qgemm_quantize_rows")


def qgemm_destroy(plan):
    load().qgemm_destroy(plan)


def qgemm_plan_path(plan) -> int:
    return load().qgemm_plan_path(plan)


def qgemm_status_string(status: int) -> str:
    return load().qgemm_status_string(int(status)).decode()
