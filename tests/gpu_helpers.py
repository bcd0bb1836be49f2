"""Shared helpers of the GPU parity tests: one seeded problem through the C ABI."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth
from weight_quantized_mixed_amd.device import QGemm, host_to_device


def say(*msg):
    print(*msg, flush=True)
    sys.stdout.flush()


class Case:
    """A seeded problem resident on the device, packed by the library."""

    def __init__(self, M, N, K, w_dtype, group_size=128, has_zeros=False, k_parts=1,
                 deterministic=False, seed=1, problem=None, split_auto=False):
        self.p = problem or synth.make_problem(M, N, K, w_dtype, group_size=group_size,
                                               has_zeros=has_zeros, seed=seed)
        p = self.p
        self.q = QGemm(p.M, p.N, p.K, p.w_dtype, p.group_size, p.has_zeros, k_parts, deterministic,
                       split_auto=split_auto)
        self.A = host_to_device(p.A)
        self.w = host_to_device(p.w)
        self.s = host_to_device(p.s)
        self.z = host_to_device(p.z)
        self.packed = self.q.pack(self.w, self.s, self.z)

    def run(self, bias=None, M=None):
        """qgemm_run, or qgemm_run_ex on the first M rows of A with an optional bias."""
        if bias is None and M is None:
            C = self.q.run(self.A, self.packed)
        else:
            A = self.A if M is None else self.A[:M]
            b = None if bias is None else host_to_device(bias)
            C = self.q.run(A, self.packed, bias=b, M=M)
        torch.cuda.synchronize()
        return C.cpu().numpy()

    def reference(self, rows=None, cols=None, bias=None):
        p = self.p
        return oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=p.N, K=p.K, w_dtype=p.w_dtype,
                                group_size=p.group_size, rows=rows, cols=cols, bias=bias)


def assert_matches(gpu, ref, what=""):
    """Integer results bit-exact; fp16 within |d| <= 1e-2 + 5e-3|ref|."""
    if ref.dtype == np.int64:
        bad = np.argwhere(gpu.astype(np.int64) != ref)
        assert bad.size == 0, f"{what}: {len(bad)} int mismatches, first {bad[:5].tolist()}"
    else:
        ok = oracle.fp16_within_tol(gpu, ref)
        if not ok.all():
            idx = np.argwhere(~ok)[:5]
            det = [(tuple(i), float(gpu[tuple(i)]), float(ref[tuple(i)])) for i in idx]
            raise AssertionError(f"{what}: {int((~ok).sum())} fp16 outside tolerance, first {det}")
        assert np.isfinite(gpu.astype(np.float64)).all()
