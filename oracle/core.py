"""Plain, slow CPU oracle: C[M,N] = A[M,K] . dequant(Wq[K,N]).

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the CPU
baseline leg of the benchmark; never by the library or its binding.

What is computed, and which passage each step follows:

* The problem statement (BitBLAS issue #252 "Default Backend Should be changed
  into tilelang ...", reproduction script: MatmulConfig fields M, N, K,
  A_dtype, W_dtype, out_dtype, accum_dtype, layout "nt", group_size,
  with_scaling, with_zeros, and the five op_configs): A is [M, K]
  row-major; the weight is stored transposed ("nt"), one row of K values per
  output column n.
* Affine dequantisation w = (q - z) * s with per-group scale s and zero point
  z (torchao issue #2752 "Migrating from AffineQuantizedTensor + Layouts ...",
  Context: affine quantised tensors for int4/intx).  Without zero points
  w = q * s; without scaling (with_scaling False) w = q.
* int8 x int8 (and int8 x int2) products accumulate and are returned in int32
  (Triton PR #3595 "[BACKEND] Add support to convert INT8 MMAV2 accumulator
  layout ...": the output type of an int8 matrix product is always int32).
* Parallel-k (hidet issue #364 "[Graph][Quantization] Multi-stage software
  pipelining and update parallel k rule": the K dimension split into k-parts
  whose partial products are summed): qgemm_ref_kparts.
* Dynamic per-token int8 quantisation of fp16 activations and the fp16 output
  of the int8 products dequantised with per-row and per-column scales
  (torchao issue #2752, Int8DynamicActivation* configurations): quantize_rows,
  qgemm_ref_scaled.
* Optional bias (the with_bias field of the same MatmulConfig, left False in
  that script's configurations): one value per output column n, added to
  every row of the product (fp16 bias to the unrounded float64 result, int32
  bias to the exact integer result).

Precision: dequantisation and accumulation in float64.  Every fp16 value is a
dyadic rational with an 11-bit significand and every integer weight is below
2**7 in magnitude, so q*s and (q - z)*s are exact in float64; the fp64
contraction differs from the exact sum only by float64 rounding.  For the
integer formats every partial sum is below K*128*128 <= 2**31, far under 2**53,
so the float64 product is the exact integer result in any summation order.

Readings where the pages are silent (each also listed with the design notes):
signed int4/int2 are two's complement; uint4 is plain binary; group_size -1
means one group over all of K; group_size 0 means no scaling; the zero point
is subtracted before scaling; fp16 results are compared before rounding,
with the tolerance |gpu - ref| <= 1e-2 + 5e-3*|ref|.
"""
from __future__ import annotations

import numpy as np

FP16_ATOL = 1e-2
FP16_RTOL = 5e-3

_BITS = {"i4": 4, "u4": 4, "i2": 2}


def group_index(k: np.ndarray | int, K: int, group_size: int):
    """Scale-group index of reduction position k (group_size -1 -> group 0)."""
    if group_size < 0:
        return np.zeros_like(np.asarray(k))
    return np.asarray(k) // group_size


def unpack_weights(w: np.ndarray, w_dtype: str, N: int, K: int) -> np.ndarray:
    """Integer weight values as a [K, N] int64 array (fp16 weights as float64).

    Canonical storage ("nt": one row of K values per output column):
    int4/uint4 uint32 [N, K/8], value k in bits 4*(k%8) of word k//8;
    int2 uint32 [N, K/16], value k in bits 2*(k%16) of word k//16;
    int8 and fp16 [N, K] as they are.
    """
    if w_dtype == "f16":
        return np.asarray(w, dtype=np.float16).reshape(N, K).T.astype(np.float64)
    if w_dtype == "i8":
        return np.asarray(w, dtype=np.int8).reshape(N, K).T.astype(np.int64)
    bits = _BITS[w_dtype]
    per = 32 // bits
    words = np.asarray(w, dtype=np.uint32).reshape(N, K // per).astype(np.int64)
    k = np.arange(K)
    field = (words[:, k // per] >> (bits * (k % per))) & ((1 << bits) - 1)  # [N, K]
    if w_dtype in ("i4", "i2"):
        # two's complement of the field width
        field = field - (field >= (1 << (bits - 1))) * (1 << bits)
    return field.T.copy()


def dequantize(q: np.ndarray, s, z, group_size: int, K: int) -> np.ndarray:
    """w[k, n] = (q[k, n] - z[n, g(k)]) * s[n, g(k)] in float64 ([K, N] in, [K, N] out).

    s is None -> no scaling (w = q); z is None -> no zero point (w = q * s).
    """
    w = np.asarray(q, dtype=np.float64)
    if s is None:
        return w
    g = group_index(np.arange(K), K, group_size)               # [K]
    s64 = np.asarray(s, dtype=np.float16).astype(np.float64)   # [N, G]
    sk = s64[:, g].T                                           # [K, N]
    if z is not None:
        z64 = np.asarray(z, dtype=np.float16).astype(np.float64)
        w = w - z64[:, g].T
    return w * sk


def _select_cols(arr, cols):
    return arr if cols is None else arr[np.asarray(cols)]


def _add_bias(C, bias, cols, integer: bool):
    """C[m, n] + bias[n] (bias None -> C unchanged)."""
    if bias is None:
        return C
    b = _select_cols(np.asarray(bias).reshape(-1), cols)
    if integer:
        out = C + np.asarray(b, dtype=np.int32).astype(np.int64)[None, :]
        assert np.all(np.abs(out) < 2**31), "int32 output overflow"
        return out
    return C + np.asarray(b, dtype=np.float16).astype(np.float64)[None, :]


def qgemm_ref(A, w, s, z, *, N: int, K: int, w_dtype: str, group_size: int,
              rows=None, cols=None, bias=None) -> np.ndarray:
    """Reference result of C = A . dequant(W) (+ bias).

    Returns float64 [M', N'] for fp16 activations (unrounded) and int64 for
    int8 activations (exact; asserted to fit int32).  rows / cols select a
    subset of output rows / columns (sampled tiles of large problems); the
    other rows and columns are never touched.  bias: [N] fp16 (fp16
    activations) or int32 (int8 activations), or None.
    """
    A = np.asarray(A)
    if rows is not None:
        A = A[np.asarray(rows)]
    # restrict the weight to the requested output columns before unpacking
    w_rows = np.asarray(w).reshape(N, -1)
    w_sel = _select_cols(w_rows, cols)
    n_sel = w_sel.shape[0]
    q = unpack_weights(w_sel, w_dtype, n_sel, K)                # [K, n_sel]
    if A.dtype == np.int8:
        C = A.astype(np.float64) @ q.astype(np.float64)
        Ci = np.rint(C).astype(np.int64)
        assert np.all(np.abs(Ci) < 2**31), "int32 accumulator overflow"
        return _add_bias(Ci, bias, cols, True)
    s_sel = None if s is None else _select_cols(np.asarray(s).reshape(N, -1), cols)
    z_sel = None if z is None else _select_cols(np.asarray(z).reshape(N, -1), cols)
    W = dequantize(q, s_sel, z_sel, group_size, K)              # [K, n_sel] float64
    return _add_bias(A.astype(np.float64) @ W, bias, cols, False)


def k_part_bounds(K: int, group_size: int, k_parts: int, granule: int = 1):
    """Contiguous K ranges of the parallel-k split, aligned to whole groups.

    With G units (scale groups, or K/granule blocks without grouping) part p
    covers units [floor(p*G/kp), floor((p+1)*G/kp)).
    """
    unit = group_size if group_size > 0 else granule
    G = K // unit
    return [((p * G // k_parts) * unit, ((p + 1) * G // k_parts) * unit)
            for p in range(k_parts)]


def qgemm_ref_kparts(A, w, s, z, *, N: int, K: int, w_dtype: str, group_size: int,
                     k_parts: int, granule: int = 1, bias=None) -> np.ndarray:
    """Parallel-k form: the sum over k-parts of A[:, Kp] . dequant(W)[Kp, :] (+ bias)."""
    A = np.asarray(A)
    q = unpack_weights(w, w_dtype, N, K)
    s_all = None if s is None else np.asarray(s).reshape(N, -1)
    z_all = None if z is None else np.asarray(z).reshape(N, -1)
    if A.dtype == np.int8:
        W = q.astype(np.float64)
        acc = np.zeros((A.shape[0], N), dtype=np.int64)
    else:
        W = dequantize(q, s_all, z_all, group_size, K)
        acc = np.zeros((A.shape[0], N), dtype=np.float64)
    for k0, k1 in k_part_bounds(K, group_size, k_parts, granule):
        part = A[:, k0:k1].astype(np.float64) @ W[k0:k1]
        acc += np.rint(part).astype(np.int64) if A.dtype == np.int8 else part
    return _add_bias(acc, bias, None, A.dtype == np.int8)


def quantize_rows(A) -> tuple[np.ndarray, np.ndarray]:
    """Dynamic per-token symmetric int8 quantisation of fp16 activations [M, K].

    The activation step of the int8 dynamic-activation configurations (torchao
    issue #2752: Int8DynamicActivationInt8WeightConfig,
    Int8DynamicActivationIntxWeightConfig).  The pages name the scheme, not its
    arithmetic; the reading taken here: one symmetric scale per row,
    scale = max|a| / 127 in fp32 (rounded to nearest), codes
    rint(a / scale) (fp32 division, ties to even) clamped to [-127, 127], and
    scale 0 with codes 0 for an all-zero row.  Returns (int8 [M, K], fp32 [M]).
    """
    A32 = np.asarray(A, dtype=np.float16).astype(np.float32)
    amax = np.max(np.abs(A32), axis=1)                        # exact
    scale = (amax / np.float32(127)).astype(np.float32)
    safe = np.where(scale > 0, scale, np.float32(1)).astype(np.float32)
    codes = np.rint((A32 / safe[:, None]).astype(np.float32))
    codes = np.where(scale[:, None] > 0, np.clip(codes, -127, 127), 0)
    return codes.astype(np.int8), scale


def qgemm_ref_scaled(Aq, w, *, N: int, K: int, w_dtype: str, row_scales, col_scales, bias=None,
                     rows=None, cols=None) -> np.ndarray:
    """fp16-output form of the int8 products: acc[m, n] * row_scales[m] *
    col_scales[n] (+ bias[n]), from the exact int32 accumulator, unrounded
    float64 (the dequantising step after an int8 x int8 / int2 product with
    per-token activation and per-channel weight scales)."""
    acc = qgemm_ref(Aq, w, None, None, N=N, K=K, w_dtype=w_dtype, group_size=0, rows=rows, cols=cols)
    rs = np.asarray(row_scales, dtype=np.float32).astype(np.float64)
    if rows is not None:
        rs = rs[np.asarray(rows)]
    cs = _select_cols(np.asarray(col_scales, dtype=np.float32).astype(np.float64), cols)
    return _add_bias(acc.astype(np.float64) * rs[:, None] * cs[None, :], bias, cols, False)


def round_fp16(C64: np.ndarray) -> np.ndarray:
    """Round to fp16, nearest-even (numpy's float64 -> float16 cast)."""
    return np.asarray(C64, dtype=np.float64).astype(np.float16)


def fp16_within_tol(gpu: np.ndarray, ref64: np.ndarray) -> np.ndarray:
    """Elementwise |gpu - ref| <= 1e-2 + 5e-3*|ref| (ref unrounded)."""
    g = np.asarray(gpu, dtype=np.float64)
    return np.abs(g - ref64) <= FP16_ATOL + FP16_RTOL * np.abs(ref64)
