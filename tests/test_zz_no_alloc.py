"""qgemm_run_noalloc (the entry point for callers that cannot allocate device
memory) against qgemm_run_ex with a caller-provided workspace, through the C
ABI: two calls in a row on each plan, the second with fewer rows, so the
second call finds the first one's leftovers in the shared scratch array.

Integer outputs and the ordered reductions must match bit for bit; fp16
outputs reduced with fp32 atomics (whose summation order may change between
runs) must each lie within the oracle's tolerance of the float64 result.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import Case, assert_matches, say
from weight_quantized_mixed_amd import qgemm as q

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


CASES = [
    # M, N, K, w_dtype, g, zeros, k_parts, split-K reduction
    (1, 4096, 4096, "i4", 128, False, 4, "atomic"),     # GEMV, fp32 atomics in scratch + conversion
    (8, 4096, 11008, "i4", 128, False, 4, "det"),      # matrix-core GEMV, ordered partials in scratch
    (128, 4096, 4096, "u4", 128, True, 4, "atomic"),   # direct-load MFMA, fp32 atomics
    (128, 4096, 4096, "f16", 0, False, 2, "det"),      # direct-load MFMA, ordered partials
    (32, 2048, 4096, "i8", 0, False, 4, "atomic"),     # int32 atomics straight into C (no scratch)
    (300, 1000, 1024, "i2", 0, False, 4, "auto"),      # int32 ordered partials in scratch
    (4, 1000, 1024, "i4", 0, False, 1, "-"),           # no split: no scratch at all
    (8, 1000, 4104, "i4", 0, False, 3, "atomic"),      # K padded: activation rows in scratch too
    (40, 264, 4100, "i8", 0, False, 1, "-"),           # K padded, no split
    (4100, 3836, 512, "u4", 128, True, 1, "-"),        # 256 x 256 tiles: zero-point planes in scratch
]


def _noalloc(c, M, bias=None):
    C = c.q.new_output(M)
    q.qgemm_run_noalloc(c.q.plan, M, c.A.data_ptr(), c.packed.data_ptr(),
                        0 if bias is None else bias.data_ptr(), C.data_ptr(),
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return C.cpu().numpy()


@pytest.mark.parametrize("M,N,K,w_dtype,g,zeros,kp,split", CASES)
def test_noalloc_matches_run_ex(M, N, K, w_dtype, g, zeros, kp, split):
    say(f"noalloc M={M} N={N} K={K} {w_dtype} g={g} kp={kp} split={split}")
    c = Case(M, N, K, w_dtype, g, zeros, k_parts=kp, deterministic=split == "det",
             split_auto=split == "auto", seed=9000 + M + N)
    exact = w_dtype in ("i8", "i2") or split in ("det", "-") or kp == 1
    bias_host = synth.draw_bias(N, c.q.out_dtype, 9001 + N)
    bias = torch.from_numpy(bias_host).cuda()
    for m_run in (M, max(1, M // 3)):   # the second call with fewer rows
        for b in (None, bias):
            got = _noalloc(c, m_run, b)
            ref_ex = c.run(bias=None if b is None else bias_host, M=m_run)
            oracle_ref = c.reference(rows=np.arange(m_run), bias=None if b is None else bias_host)
            assert_matches(got, oracle_ref, f"noalloc M={m_run} bias={b is not None}")
            if exact:
                assert np.array_equal(got, ref_ex), f"noalloc differs from run_ex at M={m_run}"
            else:
                assert_matches(ref_ex, oracle_ref, f"run_ex M={m_run}")


def test_noalloc_rejects_more_scratch_than_it_has():
    c = Case(1024, 16384, 1024, "i4", 128, False, k_parts=2, seed=9100)   # 64 MiB of fp32 atomics
    with pytest.raises(q.QGemmError) as e:
        _noalloc(c, 1024)
    assert e.value.status == q.QGEMM_ERR_UNSUPPORTED
    got = _noalloc(c, 256)                                                 # 16 MiB: fits
    assert_matches(got, c.reference(rows=np.arange(256)), "noalloc 256 of 1024 rows")
