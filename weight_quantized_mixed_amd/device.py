"""torch device-tensor wrapper around the C ABI (marshalling only).

PyTorch provides device memory and the stream; every computation is a
libqgemm kernel.  Non-GPU tensors are rejected: there is no host fallback.
"""
from __future__ import annotations

import numpy as np
import torch

from . import qgemm as _q

A_DTYPE = {"i4": "f16", "u4": "f16", "f16": "f16", "i8": "i8", "i2": "i8"}
OUT_DTYPE = {"f16": ("f16", "f32"), "i8": ("i32", "i32")}


def _ptr(t):
    if t is None:
        return 0
    if not t.is_cuda:
        raise ValueError("qgemm takes device tensors only")
    if not t.is_contiguous():
        raise ValueError("qgemm takes contiguous tensors only")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def host_to_device(arr: np.ndarray, device="cuda") -> torch.Tensor:
    """Copy a numpy array to the device; uint32 words travel as int32 bits."""
    if arr is None:
        return None
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to(device)


def quantize_rows(A, Q=None, scales=None, stream=None):
    """Per-row symmetric int8 codes and fp32 scales of fp16 A [M, K] (one kernel)."""
    M, K = A.shape
    if Q is None:
        Q = torch.empty((M, K), dtype=torch.int8, device=A.device)
    if scales is None:
        scales = torch.empty(M, dtype=torch.float32, device=A.device)
    _q.qgemm_quantize_rows(_ptr(A), M, K, _ptr(Q), _ptr(scales), _stream(stream))
    return Q, scales


class QGemm:
    """One plan: C[M,N] = A[M,K] . dequant(W) for a fixed shape and format.

    dequant_output: int8 activations with an fp16 output dequantised by per-row
    and per-column scales (run_scaled) instead of the int32 accumulator.
    Split-K (k_parts > 1) reduces with atomics, or with ordered partials when
    deterministic; split_auto lets the library pick the faster of the two.
    """

    def __init__(self, M, N, K, w_dtype, group_size=0, has_zeros=False, k_parts=1,
                 deterministic=False, device="cuda", dequant_output=False, split_auto=False):
        self.M, self.N, self.K, self.w_dtype = int(M), int(N), int(K), w_dtype
        self.a_dtype = A_DTYPE[w_dtype]
        self.out_dtype, self.accum_dtype = OUT_DTYPE[self.a_dtype]
        if dequant_output:
            if self.a_dtype != "i8":
                raise ValueError("dequant_output is for int8 activations")
            self.out_dtype = "f16"
        self.device = torch.device(device)
        flags = (_q.QGEMM_DETERMINISTIC if deterministic else 0) | (_q.QGEMM_SPLIT_AUTO if split_auto else 0)
        self.plan, self.packed_bytes, self.ws_bytes = _q.qgemm_create(
            M, N, K, self.a_dtype, w_dtype, self.out_dtype, self.accum_dtype, group_size,
            int(bool(has_zeros)), k_parts, flags)
        self.path = _q.qgemm_plan_path(self.plan)
        self._ws = None

    def close(self):
        plan = getattr(self, "plan", None)
        if plan:
            self.plan = None
            destroy = getattr(_q, "qgemm_destroy", None)
            if callable(destroy):  # not at interpreter exit, when the module is torn down
                destroy(plan)

    __del__ = close

    def pack(self, w, s=None, z=None, out=None, stream=None):
        if out is None:
            out = torch.empty(self.packed_bytes, dtype=torch.uint8, device=self.device)
        _q.qgemm_pack_weights(self.plan, _ptr(w), _ptr(s), _ptr(z), _ptr(out), _stream(stream))
        return out

    def workspace(self):
        if self.ws_bytes and self._ws is None:
            self._ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        return self._ws

    def new_output(self, M=None):
        dt = torch.float16 if self.out_dtype == "f16" else torch.int32
        return torch.empty((self.M if M is None else int(M), self.N), dtype=dt, device=self.device)

    def run(self, A, packed, C=None, ws=None, stream=None, bias=None, M=None):
        """C = A . dequant(W) (+ bias[N]) for the plan's M rows, or M <= that."""
        if C is None:
            C = self.new_output(M)
        if ws is None:
            ws = self.workspace()
        wsb = 0 if ws is None else ws.numel()
        if bias is None and M is None:
            _q.qgemm_run(self.plan, _ptr(A), _ptr(packed), _ptr(C), _ptr(ws), wsb, _stream(stream))
        else:
            _q.qgemm_run_ex(self.plan, self.M if M is None else M, _ptr(A), _ptr(packed), _ptr(bias),
                            _ptr(C), _ptr(ws), wsb, _stream(stream))
        return C

    def run_scaled(self, A, packed, row_scales, col_scales, bias=None, C=None, ws=None, stream=None, M=None):
        """fp16 C = acc . row_scales[m] . col_scales[n] (+ bias) for int8 A (dequant_output plans)."""
        if C is None:
            C = self.new_output(M)
        if ws is None:
            ws = self.workspace()
        _q.qgemm_run_scaled(self.plan, self.M if M is None else M, _ptr(A), _ptr(packed), _ptr(row_scales),
                            _ptr(col_scales), _ptr(bias), _ptr(C), _ptr(ws),
                            0 if ws is None else ws.numel(), _stream(stream))
        return C
