"""GPU parity of qgemm_run_ex: the bias epilogue on every path and reduction,
and run-time row counts below the plan's M, against the CPU oracle."""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import Case, assert_matches, say
from weight_quantized_mixed_amd import qgemm as q

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


def _bias(c, seed):
    return synth.draw_bias(c.p.N, "i32" if c.p.a_dtype == "i8" else "f16", seed)


BIAS_CASES = [
    # M, N, K, w_dtype, g, zeros, k_parts, split-K reduction
    (1, 300, 1024, "i4", 128, False, 1, "-"),         # GEMV, stored
    (1, 72, 512, "u4", 128, True, 1, "-"),            # 16-column GEMV
    (3, 136, 1024, "u4", 64, True, 3, "atomic"),      # GEMV, fp32 atomics + conversion pass
    (3, 136, 1024, "u4", 64, True, 3, "det"),         # GEMV, ordered partials + summing pass
    (5, 200, 1024, "i8", 0, False, 3, "atomic"),      # GEMV, int32 atomics onto the bias rows
    (5, 200, 2048, "i2", 0, False, 2, "det"),         # GEMV, two-pass
    (40, 264, 1024, "i4", 128, False, 1, "-"),        # direct-load MFMA, stored
    (20, 264, 1024, "i8", 0, False, 3, "atomic"),     # matrix-core GEMV, int32 atomics onto the bias rows
    (64, 72, 1024, "u4", 32, True, 1, "-"),           # LDS-staged MFMA (per-piece groups)
    (130, 264, 768, "i4", 64, False, 3, "det"),       # LDS-staged MFMA, two-pass
    (129, 136, 512, "i8", 0, False, 3, "auto"),       # direct-load, int32 partials (128 rows and more)
    (129, 136, 512, "i8", 0, False, 3, "atomic"),     # direct-load, int32 atomics onto the bias rows
    (300, 520, 512, "f16", 0, False, 2, "auto"),      # direct-load, ordered partials
    (300, 520, 512, "f16", 0, False, 2, "atomic"),    # direct-load, fp32 atomics + conversion pass
    (160, 264, 1024, "i2", 0, False, 1, "-"),         # direct-load int, stored
    (40, 264, 1024, "i4", -1, False, 1, "-"),         # direct-load, column scale in the epilogue
    (300, 520, 1024, "u4", -1, False, 2, "atomic"),   # the same, fp32 atomics + conversion pass
]


@pytest.mark.parametrize("M,N,K,w_dtype,g,zeros,kp,split", BIAS_CASES)
def test_bias_epilogue(M, N, K, w_dtype, g, zeros, kp, split):
    say(f"case bias M={M} N={N} K={K} {w_dtype} g={g} kp={kp} split={split}")
    c = Case(M, N, K, w_dtype, g, zeros, k_parts=kp, deterministic=split == "det", split_auto=split == "auto",
             seed=5000 + M + N)
    b = _bias(c, 5001 + N)
    assert_matches(c.run(bias=b), c.reference(bias=b), f"bias M={M} {w_dtype} kp={kp}")


# the automatic choice keeps the atomic reductions where the partials would pass 256 MiB:
# fp32 into the zero-filled workspace (bias added by the conversion pass) and int32 onto
# the bias rows
@pytest.mark.parametrize("w_dtype,g", [("i4", 128), ("i8", 0)])
def test_bias_with_atomic_split(w_dtype, g):
    M, N, K = 4100, 8400, 256
    say(f"case bias atomic split M={M} N={N} K={K} {w_dtype} kp=2")
    c = Case(M, N, K, w_dtype, g, False, k_parts=2, seed=5100, split_auto=True)
    # int4 on the 256 x 256 tiles adds the folding's planes (row sums over K / g = 2 groups
    # padded to 32, the per-column term for the 8448 padded columns)
    assert c.q.ws_bytes == (M * N * 4 + (M + 8448) * 32 * 2 * 2 if w_dtype == "i4" else 0)
    b = _bias(c, 5101)
    rng = np.random.default_rng(4)
    rows = np.unique(np.concatenate([rng.choice(M, 150, replace=False), [0, M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(N, 150, replace=False), [0, N - 1]]))
    gpu = c.run(bias=b)
    assert_matches(gpu[np.ix_(rows, cols)], c.reference(rows=rows, cols=cols, bias=b), f"bias atomic {w_dtype}")


ROW_PLANS = [
    # plan M, N, K, w_dtype, g, zeros, k_parts, deterministic
    (300, 264, 1024, "i4", 128, False, 1, False),
    (300, 200, 1024, "u4", 128, True, 2, True),
    (160, 136, 1024, "i8", 0, False, 3, False),
    (64, 300, 2048, "i2", 0, False, 1, False),
    (8, 520, 512, "f16", 0, False, 2, False),
]


@pytest.mark.parametrize("Mp,N,K,w_dtype,g,zeros,kp,det", ROW_PLANS)
def test_run_time_rows(Mp, N, K, w_dtype, g, zeros, kp, det):
    say(f"case rows plan M={Mp} N={N} K={K} {w_dtype} kp={kp} det={det}")
    c = Case(Mp, N, K, w_dtype, g, zeros, k_parts=kp, deterministic=det, seed=6000 + Mp + N)
    b = _bias(c, 6001 + N)
    for M in sorted({1, 2, 5, 8, 9, 33, Mp // 2, Mp}):
        if M < 1 or M > Mp:
            continue
        say(f"  rows M={M}")
        ref = c.reference(rows=np.arange(M))
        assert_matches(c.run(M=M), ref, f"rows M={M}/{Mp} {w_dtype}")
        refb = c.reference(rows=np.arange(M), bias=b)
        assert_matches(c.run(M=M, bias=b), refb, f"rows+bias M={M}/{Mp} {w_dtype}")


def test_run_ex_at_plan_rows_equals_run():
    c = Case(40, 264, 1024, "i8", 0, False, k_parts=1, seed=7)
    assert np.array_equal(c.run(), c.run(M=40))


def test_run_time_rows_reject_more_than_the_plan():
    c = Case(4, 72, 512, "i4", 128, False, seed=8)
    C = torch.empty((5, 72), dtype=torch.float16, device="cuda")
    A = torch.zeros((5, 512), dtype=torch.float16, device="cuda")
    with pytest.raises(q.QGemmError) as e:
        c.q.run(A, c.packed, C=C, M=5)
    assert e.value.status == q.QGEMM_ERR_INVALID_ARG
