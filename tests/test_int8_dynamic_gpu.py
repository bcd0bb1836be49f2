"""GPU parity of the int8 dynamic-activation steps: the per-row quantiser
(codes and scales bit-exact against the oracle) and the fp16 output of the
int8 products dequantised with per-row and per-column scales."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_matches, say
from weight_quantized_mixed_amd.device import QGemm, host_to_device, quantize_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


def _edge_rows(A):
    """Rows the quantiser must treat exactly: zeros, fp16 subnormals, ties, one dominant value."""
    K = A.shape[1]
    A[0] = 0
    if A.shape[0] > 1:
        A[1] = np.float16(2**-20) * np.arange(K).astype(np.float16) % 7   # subnormal fp16 values
    if A.shape[0] > 2:
        A[2] = 0
        A[2, :5] = [254, 1, 3, 5, -5]                                       # quotients x.5
    if A.shape[0] > 3:
        A[3, K // 2] = np.float16(-65504)
    return A


@pytest.mark.parametrize("M,K", [(1, 16384), (7, 4096), (300, 1024), (2, 8), (5, 72), (3, 32768), (2, 40960)])
def test_quantize_rows_bit_exact(M, K):
    say(f"case quantize M={M} K={K}")
    A = _edge_rows(synth.draw_fp16_activations(M, K, seed=M + K))
    Q, S = quantize_rows(host_to_device(A))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(A)
    assert np.array_equal(S.cpu().numpy(), s_ref)
    bad = np.argwhere(Q.cpu().numpy() != q_ref)
    assert bad.size == 0, f"{len(bad)} codes differ, first {bad[:5].tolist()}"


class ScaledCase:
    def __init__(self, M, N, K, w_dtype, k_parts=1, det=False, seed=1):
        self.p = synth.make_problem(M, N, K, w_dtype, group_size=0, seed=seed)
        self.q = QGemm(M, N, K, w_dtype, 0, False, k_parts, det, dequant_output=True)
        self.A = host_to_device(self.p.A)
        self.packed = self.q.pack(host_to_device(self.p.w))
        self.rs = synth.draw_col_scales(M, seed + 1)
        self.cs = synth.draw_col_scales(N, seed + 2)
        self.b = synth.draw_bias(N, "f16", seed + 3)

    def run(self, M=None, bias=False):
        M = self.p.M if M is None else M
        C = self.q.run_scaled(self.A[:M], self.packed, host_to_device(self.rs[:M]), host_to_device(self.cs),
                              host_to_device(self.b) if bias else None, M=M)
        torch.cuda.synchronize()
        return C.cpu().numpy()

    def reference(self, M=None, bias=False):
        M = self.p.M if M is None else M
        p = self.p
        return oracle.qgemm_ref_scaled(p.A, p.w, N=p.N, K=p.K, w_dtype=p.w_dtype, row_scales=self.rs,
                                       col_scales=self.cs, bias=self.b if bias else None, rows=np.arange(M))


SCALED = [
    # M, N, K, w_dtype, k_parts, deterministic
    (1, 300, 1024, "i8", 1, False),     # GEMV, stored
    (1, 72, 2048, "i2", 1, False),      # 16-column GEMV
    (5, 200, 1024, "i8", 3, False),     # GEMV, int32 atomics in the workspace + finalize
    (4, 136, 2048, "i2", 2, True),      # GEMV, two-pass
    (40, 264, 1024, "i8", 1, False),    # direct-load MFMA, stored
    (129, 136, 512, "i8", 3, False),    # direct-load MFMA, atomics
    (160, 264, 1024, "i2", 2, True),    # direct-load MFMA, two-pass
]


@pytest.mark.parametrize("M,N,K,w_dtype,kp,det", SCALED)
def test_dequantised_output(M, N, K, w_dtype, kp, det):
    say(f"case scaled M={M} N={N} K={K} {w_dtype} kp={kp} det={det}")
    c = ScaledCase(M, N, K, w_dtype, kp, det, seed=900 + M + N)
    for bias in (False, True):
        assert_matches(c.run(bias=bias), c.reference(bias=bias), f"scaled {w_dtype} M={M} bias={bias}")
    for m in sorted({1, 3, M // 2}):
        if 1 <= m < M:
            assert_matches(c.run(M=m, bias=True), c.reference(M=m, bias=True), f"scaled rows {m}/{M}")


@pytest.mark.parametrize("M,N,K,w_dtype", [(1, 512, 4096, "i8"), (6, 264, 2048, "i2"), (64, 300, 1024, "i8")])
def test_fp16_activations_end_to_end(M, N, K, w_dtype):
    """fp16 A -> per-row int8 codes -> int8 product -> fp16, against the oracle's same steps."""
    say(f"case end-to-end M={M} N={N} K={K} {w_dtype}")
    A16 = synth.draw_fp16_activations(M, K, seed=M * 7 + K)
    p = synth.make_problem(M, N, K, w_dtype, group_size=0, seed=M + N)
    cs = synth.draw_col_scales(N, seed=N)
    qg = QGemm(M, N, K, w_dtype, dequant_output=True)
    packed = qg.pack(host_to_device(p.w))
    Q, S = quantize_rows(host_to_device(A16))
    C = qg.run_scaled(Q, packed, S, host_to_device(cs))
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quantize_rows(A16)
    ref = oracle.qgemm_ref_scaled(q_ref, p.w, N=N, K=K, w_dtype=w_dtype, row_scales=s_ref, col_scales=cs)
    assert_matches(C.cpu().numpy(), ref, f"end-to-end {w_dtype} M={M}")
