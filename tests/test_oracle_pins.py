"""Pins of the CPU oracle to facts that do not come from the oracle itself.

The pages print no output values for this computation (only timings), so the
oracle is pinned by: the canonical storage layout worked by hand, exact
brute force in rational arithmetic on tiny shapes, closed forms (zero
weights, identity weights, one-hot activations, constant operands), the
parallel-k decomposition, and exact invariants.  A last group of tests plants
plausible mistakes in a copy of the oracle and checks that a pin catches each.
"""
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import core as ref
import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# --------------------------------------------------------------------------- layout by hand
def test_int4_layout_by_hand():
    # value k of a row sits in bits 4*(k%8) of word k//8, two's complement
    words = np.array([[0x76543210, 0xFEDCBA98]], dtype=np.uint32)   # N=1, K=16
    q = oracle.unpack_weights(words, "i4", 1, 16)[:, 0]
    assert q.tolist() == [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]
    qu = oracle.unpack_weights(words, "u4", 1, 16)[:, 0]
    assert qu.tolist() == list(range(16))


def test_int2_layout_by_hand():
    # value k in bits 2*(k%16) of word k//16: 0b01 -> 1, 0b10 -> -2, 0b11 -> -1
    w = (1 << 0) | (2 << 2) | (3 << 4) | (0 << 6) | (3 << 30)
    q = oracle.unpack_weights(np.array([[w]], dtype=np.uint32), "i2", 1, 16)[:, 0]
    assert q.tolist() == [1, -2, -1, 0] + [0] * 11 + [-1]


def test_nt_orientation_by_hand():
    # two output columns with different rows of K values: C[0, n] = sum_k A[k]*W[n][k]
    w = np.array([[0x00000021], [0x00000003]], dtype=np.uint32)  # col0: q=(1,2,0..), col1: q=(3,0..)
    A = np.zeros((1, 8), dtype=np.float16)
    A[0, 0], A[0, 1] = 10.0, 100.0
    C = oracle.qgemm_ref(A, w, None, None, N=2, K=8, w_dtype="i4", group_size=0)
    assert C.tolist() == [[10 * 1 + 100 * 2, 10 * 3]]


@pytest.mark.parametrize("w_dtype", ["i4", "u4", "i2", "i8"])
def test_encode_unpack_round_trip(w_dtype):
    p = synth.make_problem(2, 24, 256, w_dtype, group_size=64, seed=7)
    q = oracle.unpack_weights(p.w, w_dtype, p.N, p.K)
    assert np.array_equal(q, p.q.T.astype(np.int64))


# --------------------------------------------------------------------------- brute force
def _brute(p, kparts=None, bias=None):
    """Exact C by a triple loop over rationals, from the integer weight values."""
    M, N, K, g = p.M, p.N, p.K, p.group_size
    out = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                a = Fraction(int(p.A[m, k])) if p.a_dtype == "i8" else Fraction(float(p.A[m, k]))
                qv = p.q[n, k]
                wv = Fraction(float(qv)) if p.w_dtype == "f16" else Fraction(int(qv))
                if p.s is not None:
                    gi = 0 if g < 0 else k // g
                    if p.z is not None:
                        wv = wv - Fraction(float(p.z[n, gi]))
                    wv = wv * Fraction(float(p.s[n, gi]))
                acc += a * wv
            if bias is not None:
                acc += Fraction(int(bias[n])) if p.a_dtype == "i8" else Fraction(float(bias[n]))
            out[m][n] = acc
    return out


CASES = [
    # (M, N, K, w_dtype, g, zeros)
    (1, 16, 64, "i4", 32, False),
    (3, 5, 128, "i4", 64, False),
    (2, 7, 128, "u4", 32, True),
    (2, 3, 96, "u4", -1, True),
    (2, 9, 64, "i4", 0, False),
    (3, 16, 256, "i4", -1, False),
    (2, 11, 64, "i8", 0, False),
    (3, 6, 256, "i2", 0, False),
    (2, 5, 64, "f16", 0, False),
]


@pytest.mark.parametrize("M,N,K,w_dtype,g,zeros", CASES)
def test_oracle_vs_exact_brute_force(M, N, K, w_dtype, g, zeros):
    p = synth.make_problem(M, N, K, w_dtype, group_size=g, has_zeros=zeros, seed=1234 + K + N)
    C = oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype=w_dtype, group_size=p.group_size)
    exact = _brute(p)
    for m in range(M):
        for n in range(N):
            e = exact[m][n]
            if p.a_dtype == "i8":
                assert int(C[m, n]) == e, (m, n)
            else:
                # float64 rounding of K products and sums: far below 1e-9 at these sizes
                assert abs(Fraction(float(C[m, n])) - e) <= Fraction(1, 10**9) * (1 + abs(e)), (m, n)


BIAS_CASES = [(3, 7, 128, "i4", 32, False), (2, 5, 128, "u4", -1, True), (2, 9, 256, "i2", 0, False),
              (3, 6, 64, "i8", 0, False), (2, 5, 64, "f16", 0, False)]


@pytest.mark.parametrize("M,N,K,w_dtype,g,zeros", BIAS_CASES)
def test_oracle_bias_vs_exact_brute_force(M, N, K, w_dtype, g, zeros):
    p = synth.make_problem(M, N, K, w_dtype, group_size=g, has_zeros=zeros, seed=777 + K + N)
    b = synth.draw_bias(N, "i32" if p.a_dtype == "i8" else "f16", seed=778 + N)
    C = oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype=w_dtype, group_size=p.group_size, bias=b)
    exact = _brute(p, bias=b)
    for m in range(M):
        for n in range(N):
            e = exact[m][n]
            if p.a_dtype == "i8":
                assert int(C[m, n]) == e, (m, n)
            else:
                assert abs(Fraction(float(C[m, n])) - e) <= Fraction(1, 10**9) * (1 + abs(e)), (m, n)
    # the split-K form adds it once, not once per part
    Ck = oracle.qgemm_ref_kparts(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype=w_dtype, group_size=p.group_size,
                                 k_parts=2, granule=32, bias=b)
    if p.a_dtype == "i8":
        assert np.array_equal(Ck, C)
    else:
        assert np.allclose(Ck, C, rtol=0, atol=1e-9)


def test_zero_activations_give_the_bias():
    N, K = 12, 128
    p = synth.make_problem(3, N, K, "i4", group_size=128, seed=9)
    b = synth.draw_bias(N, "f16", seed=10)
    C = oracle.qgemm_ref(np.zeros_like(p.A), p.w, p.s, p.z, N=N, K=K, w_dtype="i4", group_size=128, bias=b)
    assert np.array_equal(C, np.broadcast_to(b.astype(np.float64), (3, N)))


# --------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("w_dtype", ["i4", "i2", "i8"])
def test_zero_weights_give_zero(w_dtype):
    N, K = 8, 256
    q = np.zeros((N, K), dtype=np.int8)
    p = synth.make_problem(3, N, K, w_dtype, group_size=128, q=q, seed=3)
    C = oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype=w_dtype, group_size=p.group_size)
    assert np.all(C == 0)


def test_uint4_q_equal_zero_point_gives_zero():
    N, K = 8, 256
    q = np.full((N, K), 8, dtype=np.int8)
    z = np.full((N, 2), 8.0, dtype=np.float16)
    p = synth.make_problem(2, N, K, "u4", group_size=128, has_zeros=True, q=q, z=z, seed=4)
    C = oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype="u4", group_size=128)
    assert np.all(C == 0.0)


@pytest.mark.parametrize("w_dtype", ["i4", "i2", "i8"])
def test_identity_weights_give_A(w_dtype):
    K = N = 64
    q = np.eye(N, K, dtype=np.int8)
    s = np.ones((N, 2), dtype=np.float16)
    p = synth.make_problem(3, N, K, w_dtype, group_size=32, q=q, s=s, seed=5)
    C = oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype=w_dtype, group_size=p.group_size)
    assert np.array_equal(C, p.A.astype(C.dtype))


@pytest.mark.parametrize("w_dtype,zeros", [("i4", False), ("u4", True)])
def test_one_hot_activation_picks_one_weight(w_dtype, zeros):
    M, N, K, g = 1, 12, 256, 64
    p = synth.make_problem(M, N, K, w_dtype, group_size=g, has_zeros=zeros, seed=6)
    for k0 in (0, 63, 64, 200, 255):
        A = np.zeros((1, K), dtype=np.float16)
        A[0, k0] = 1.0
        C = oracle.qgemm_ref(A, p.w, p.s, p.z, N=N, K=K, w_dtype=w_dtype, group_size=g)
        for n in range(N):
            wv = Fraction(int(p.q[n, k0]))
            if zeros:
                wv -= Fraction(float(p.z[n, k0 // g]))
            wv *= Fraction(float(p.s[n, k0 // g]))
            assert Fraction(float(C[0, n])) == wv


@pytest.mark.parametrize("zeros", [False, True])
def test_constant_operands_closed_form(zeros):
    M, N, K, g, c = 2, 6, 512, 128, 5
    A = np.ones((M, K), dtype=np.float16)
    q = np.full((N, K), c, dtype=np.int8)
    s0, z0 = np.float16(0.0125), np.float16(6.5)
    s = np.full((N, K // g), s0, dtype=np.float16)
    z = np.full((N, K // g), z0, dtype=np.float16)
    wd = "u4" if zeros else "i4"
    p = synth.make_problem(M, N, K, wd, group_size=g, has_zeros=zeros, q=q, A=A, s=s, z=z)
    C = oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype=wd, group_size=g)
    expect = K * ((c - float(z0)) if zeros else c) * float(s0)
    assert np.all(C == expect)


def test_int_closed_form_extremes():
    # A = -128 everywhere, W = -128 everywhere: C = K * 16384 (largest int8 product)
    M, N, K = 1, 4, 1024
    A = np.full((M, K), -128, dtype=np.int8)
    q = np.full((N, K), -128, dtype=np.int8)
    p = synth.make_problem(M, N, K, "i8", q=q, A=A)
    C = oracle.qgemm_ref(p.A, p.w, None, None, N=N, K=K, w_dtype="i8", group_size=0)
    assert np.all(C == K * 16384)


# --------------------------------------------------------------------------- parallel-k
def test_k_part_bounds_group_aligned():
    assert oracle.k_part_bounds(11008, 128, 4) == [(0, 21 * 128), (21 * 128, 43 * 128),
                                                   (43 * 128, 64 * 128), (64 * 128, 86 * 128)]
    b = oracle.k_part_bounds(16384, 0, 4, granule=256)
    assert b[0] == (0, 4096) and b[-1] == (12288, 16384)


@pytest.mark.parametrize("w_dtype,g,zeros", [("i4", 128, False), ("u4", 128, True),
                                             ("i8", 0, False), ("i2", 0, False)])
def test_kparts_agree_with_single_part(w_dtype, g, zeros):
    M, N, K = 3, 40, 1408   # 11 groups of 128: uneven parts
    p = synth.make_problem(M, N, K, w_dtype, group_size=g, has_zeros=zeros, seed=8)
    C1 = oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype=w_dtype, group_size=p.group_size)
    C4 = oracle.qgemm_ref_kparts(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype=w_dtype,
                                 group_size=p.group_size, k_parts=4, granule=64)
    if p.a_dtype == "i8":
        assert np.array_equal(C1, C4)
    else:
        assert np.allclose(C1, C4, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- invariants
def test_sign_symmetry_int_exact():
    p = synth.make_problem(3, 20, 512, "i2", seed=9)
    A = np.clip(p.A, -127, 127).astype(np.int8)
    C = oracle.qgemm_ref(A, p.w, None, None, N=20, K=512, w_dtype="i2", group_size=0)
    Cn = oracle.qgemm_ref(-A, p.w, None, None, N=20, K=512, w_dtype="i2", group_size=0)
    assert np.array_equal(Cn, -C)


def test_column_permutation_permutes_output():
    N, K = 24, 256
    p = synth.make_problem(2, N, K, "u4", group_size=64, has_zeros=True, seed=10)
    perm = np.random.default_rng(0).permutation(N)
    C = oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype="u4", group_size=64)
    Cp = oracle.qgemm_ref(p.A, p.w[perm], p.s[perm], p.z[perm], N=N, K=K, w_dtype="u4", group_size=64)
    assert np.array_equal(Cp, C[:, perm])


def test_row_col_subset_matches_full():
    M, N, K = 40, 48, 256
    p = synth.make_problem(M, N, K, "u4", group_size=128, has_zeros=True, seed=11)
    C = oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype="u4", group_size=128)
    rows, cols = [0, 5, 39], [1, 2, 47]
    Cs = oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype="u4", group_size=128,
                          rows=rows, cols=cols)
    assert np.array_equal(Cs, C[np.ix_(rows, cols)])


def test_fp16_tolerance_and_rounding():
    ref64 = np.array([0.0, 1.0, 100.0, -7.3])
    assert oracle.fp16_within_tol(np.array([0.0099, 1.0149, 100.5, -7.3]), ref64).all()
    assert not oracle.fp16_within_tol(np.array([0.0101, 1.0, 100.0, -7.3]), ref64).all()
    # round to nearest even at the fp16 half-ulp of 1.0 (ulp 2**-10)
    assert oracle.round_fp16(np.array([1 + 2**-11]))[0] == np.float16(1.0)
    assert oracle.round_fp16(np.array([1 + 3 * 2**-11]))[0] == np.float16(1 + 2**-9)


# --------------------------------------------------------------------------- planted mistakes
def _pins_pass():
    """Run a subset of the pins; return False as soon as one fails."""
    try:
        test_int4_layout_by_hand()
        test_int2_layout_by_hand()
        test_nt_orientation_by_hand()
        for c in CASES[:4] + CASES[6:8]:
            test_oracle_vs_exact_brute_force(*c)
        test_one_hot_activation_picks_one_weight("u4", True)
        test_constant_operands_closed_form(True)
        for c in BIAS_CASES:
            test_oracle_bias_vs_exact_brute_force(*c)
    except AssertionError:
        return False
    return True


def _mut_no_sign_extension(w, w_dtype, N, K):
    q = ORIG_UNPACK(w, "u4" if w_dtype == "i4" else w_dtype, N, K)
    return q


def _mut_group_mod(k, K, group_size):
    if group_size < 0:
        return np.zeros_like(np.asarray(k))
    return (np.asarray(k) % group_size) % max(1, K // group_size)


def _mut_zero_dropped(q, s, z, group_size, K):
    return ORIG_DEQUANT(q, s, None, group_size, K)


def _mut_transposed_nibbles(w, w_dtype, N, K):
    q = ORIG_UNPACK(w, w_dtype, N, K)
    if w_dtype in ("i4", "u4"):
        q = q.reshape(K // 8, 8, N)[:, ::-1, :].reshape(K, N)
    return q


def _mut_bias_on_rows(C, bias, cols, integer):
    if bias is None:
        return C
    b = np.resize(np.asarray(bias, dtype=np.float64), C.shape[0])
    return C + (b.astype(np.int64) if integer else b)[:, None]


def _mut_bias_dropped(C, bias, cols, integer):
    return C


ORIG_UNPACK = ref.unpack_weights
ORIG_DEQUANT = ref.dequantize


@pytest.mark.parametrize("target,mutant", [
    ("unpack_weights", _mut_no_sign_extension),
    ("group_index", _mut_group_mod),
    ("dequantize", _mut_zero_dropped),
    ("unpack_weights", _mut_transposed_nibbles),
    ("_add_bias", _mut_bias_on_rows),
    ("_add_bias", _mut_bias_dropped),
])
def test_planted_mistakes_are_caught(monkeypatch, target, mutant):
    assert _pins_pass()
    monkeypatch.setattr(ref, target, mutant)
    monkeypatch.setattr(oracle, target, mutant, raising=False)
    assert not _pins_pass()


# --------------------------------------------------------------------------- int8 activation quantiser
def _f32(x: float) -> float:
    """Round a Python float (binary64) to the nearest binary32 value."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def _quantize_loop(A):
    """Per-row codes and scales by plain loops: binary64 division then one
    rounding to binary32 is the correctly rounded binary32 quotient of binary32
    operands, and Python's round() takes ties to even."""
    codes, scales = [], []
    for row in np.asarray(A, dtype=np.float16).tolist():
        amax = max(abs(float(v)) for v in row)
        s = _f32(amax / 127.0)
        scales.append(s)
        if s == 0.0:
            codes.append([0] * len(row))
            continue
        codes.append([max(-127, min(127, round(_f32(float(v) / s)))) for v in row])
    return codes, scales


def test_quantize_rows_matches_loops():
    A = synth.draw_fp16_activations(6, 96, seed=31)
    A[2] *= np.float16(1e-3)   # small magnitudes
    A[3] = 0                   # all-zero row
    A[4, 7] = np.float16(-60000)  # one dominant value
    q, s = oracle.quantize_rows(A)
    qc, sc = _quantize_loop(A)
    assert s.dtype == np.float32 and q.dtype == np.int8
    assert [float(v) for v in s] == sc
    assert q.tolist() == qc


def test_quantize_rows_closed_forms():
    # exact multiples of a power-of-two scale map to their multipliers
    row = np.array([0, 1, -2, 127, -127, 64], dtype=np.float16) / np.float16(64)
    q, s = oracle.quantize_rows(row[None, :])
    assert s[0] == np.float32(1 / 64) and q[0].tolist() == [0, 1, -2, 127, -127, 64]
    # ties go to even: scale 2, quotients 0.5, 1.5, 2.5, -2.5 -> 0, 2, 2, -2
    q, s = oracle.quantize_rows(np.array([[254, 1, 3, 5, -5]], dtype=np.float16))
    assert s[0] == 2 and q[0].tolist() == [127, 0, 2, 2, -2]
    # an all-zero row: scale 0, codes 0
    q, s = oracle.quantize_rows(np.zeros((1, 8), dtype=np.float16))
    assert s[0] == 0 and not q.any()


def test_quantize_rows_error_bound():
    A = synth.draw_fp16_activations(16, 256, seed=32)
    q, s = oracle.quantize_rows(A)
    err = np.abs(A.astype(np.float64) - q.astype(np.float64) * s[:, None].astype(np.float64))
    # half a step, plus the fp32 rounding of the scale and the quotient
    assert np.all(err <= s[:, None] * (0.5 + 1e-5))
    assert np.all(np.abs(q.astype(np.int64)).max(axis=1) == 127)


def test_scaled_products_vs_exact_brute_force():
    M, N, K = 3, 5, 128
    for w_dtype in ("i8", "i2"):
        p = synth.make_problem(M, N, K if w_dtype == "i8" else 256, w_dtype, group_size=0, seed=41)
        rs = synth.draw_col_scales(M, seed=42)          # any positive fp32 values serve as row scales
        cs = synth.draw_col_scales(N, seed=43)
        b = synth.draw_bias(N, "f16", seed=44)
        C = oracle.qgemm_ref_scaled(p.A, p.w, N=N, K=p.K, w_dtype=w_dtype, row_scales=rs, col_scales=cs, bias=b)
        exact = _brute(p)
        for m in range(M):
            for n in range(N):
                e = exact[m][n] * Fraction(float(rs[m])) * Fraction(float(cs[n])) + Fraction(float(b[n]))
                assert abs(Fraction(float(C[m, n])) - e) <= Fraction(1, 10**9) * (1 + abs(e)), (w_dtype, m, n)


def _mut_round_half_away(A):
    A32 = np.asarray(A, dtype=np.float16).astype(np.float32)
    amax = np.max(np.abs(A32), axis=1)
    scale = (amax / np.float32(127)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
    x = (A32 / safe[:, None]).astype(np.float32)
    codes = np.sign(x) * np.floor(np.abs(x) + 0.5)
    return np.where(scale[:, None] > 0, np.clip(codes, -127, 127), 0).astype(np.int8), scale


def _mut_scale_128(A):
    A32 = np.asarray(A, dtype=np.float16).astype(np.float32)
    scale = (np.max(np.abs(A32), axis=1) / np.float32(128)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
    codes = np.rint((A32 / safe[:, None]).astype(np.float32))
    return np.where(scale[:, None] > 0, np.clip(codes, -127, 127), 0).astype(np.int8), scale


@pytest.mark.parametrize("mutant", [_mut_round_half_away, _mut_scale_128])
def test_quantizer_planted_mistakes_are_caught(monkeypatch, mutant):
    def pins():
        try:
            test_quantize_rows_matches_loops()
            test_quantize_rows_closed_forms()
        except AssertionError:
            return False
        return True
    assert pins()
    monkeypatch.setattr(oracle, "quantize_rows", mutant)
    assert not pins()
