"""Seeded synthetic inputs for the weight-quantized matmul.

This module only draws random numbers and writes them in the canonical input
encoding that the C header documents (activation rows, weight words packed
along K, per-group scale and zero-point tables).  It holds none of the
method's arithmetic: no unpacking, no dequantisation, no contraction.  Both
the CPU oracle and the GPU path are fed from here, so they see identical bytes.

Distributions follow the workloads of the pages' benchmark grid (BitBLAS issue
#252, reproduction script: shapes M x 16384 x 16384 and the five op configs)
with the value ranges stated for the formats: fp16 activations ~ N(0,1), int8
activations uniform over [-128, 127], signed int4 weights over [-8, 7],
unsigned int4 over [0, 15], signed int2 over [-2, 1], int8 over [-128, 127],
fp16 scales uniform over [0.005, 0.02] and fp16 zero points uniform over
[6, 9].
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

# stream ids of the counter-based seed sequence, one per operand
STREAM_A, STREAM_W, STREAM_S, STREAM_Z, STREAM_B, STREAM_C = 0, 1, 2, 3, 4, 5

W_DTYPES = ("i4", "u4", "i2", "i8", "f16")
A_OF_W = {"i4": "f16", "u4": "f16", "f16": "f16", "i8": "i8", "i2": "i8"}
PACK_FACTOR = {"i4": 8, "u4": 8, "i2": 16, "i8": 1, "f16": 1}
Q_RANGE = {"i4": (-8, 7), "u4": (0, 15), "i2": (-2, 1), "i8": (-128, 127)}


def seed_for(config: int, variant: int = 0) -> int:
    """Seed of a benchmark configuration: 20260000 + 100*config + variant."""
    return 20260000 + 100 * int(config) + int(variant)


def _rng(seed: int, stream: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def num_groups(K: int, group_size: int) -> int:
    """Number of scale groups along K: 0 without scaling, 1 per channel (g=-1)."""
    if group_size == 0:
        return 0
    if group_size < 0:
        return 1
    return K // group_size


def encode_weights(q: np.ndarray, w_dtype: str) -> np.ndarray:
    """Write integer weight values q[N, K] in the canonical storage format.

    int4/uint4: uint32 [N, K/8], element k of row n in bits 4*(k%8) of word k//8.
    int2:       uint32 [N, K/16], element k in bits 2*(k%16) of word k//16.
    int8, fp16: [N, K] row-major, stored as is.
    Signed values are stored in two's complement of the field width.
    """
    if w_dtype in ("i8", "f16"):
        return np.ascontiguousarray(q)
    bits = 4 if w_dtype in ("i4", "u4") else 2
    per = 32 // bits
    N, K = q.shape
    if K % per:
        raise ValueError(f"K={K} is not a multiple of {per}")
    field = (q.astype(np.int64) & ((1 << bits) - 1)).astype(np.uint32)
    field = field.reshape(N, K // per, per)
    shifts = (np.arange(per, dtype=np.uint32) * bits)[None, None, :]
    words = np.bitwise_or.reduce(field << shifts, axis=2)
    return np.ascontiguousarray(words.astype(np.uint32))


@dataclass
class Problem:
    M: int
    N: int
    K: int
    a_dtype: str
    w_dtype: str
    group_size: int
    has_zeros: bool
    A: np.ndarray               # [M, K] float16 or int8
    q: np.ndarray               # [N, K] integer weight values (int8), or fp16 weights
    w: np.ndarray               # canonical storage of q (see encode_weights)
    s: Optional[np.ndarray]     # [N, G] float16 or None
    z: Optional[np.ndarray]     # [N, G] float16 or None

    @property
    def G(self) -> int:
        return num_groups(self.K, self.group_size)


def draw_activations(M: int, K: int, a_dtype: str, seed: int) -> np.ndarray:
    r = _rng(seed, STREAM_A)
    if a_dtype == "f16":
        return r.standard_normal((M, K), dtype=np.float32).astype(np.float16)
    if a_dtype == "i8":
        return r.integers(-128, 128, size=(M, K), dtype=np.int8)
    raise ValueError(a_dtype)


def draw_weights(N: int, K: int, w_dtype: str, seed: int) -> np.ndarray:
    r = _rng(seed, STREAM_W)
    if w_dtype == "f16":
        return r.standard_normal((N, K), dtype=np.float32).astype(np.float16)
    lo, hi = Q_RANGE[w_dtype]
    return r.integers(lo, hi + 1, size=(N, K), dtype=np.int8)


def draw_scales(N: int, G: int, seed: int) -> np.ndarray:
    r = _rng(seed, STREAM_S)
    return r.uniform(0.005, 0.02, size=(N, G)).astype(np.float16)


def draw_bias(N: int, out_dtype: str, seed: int) -> np.ndarray:
    """Output bias [N]: fp16 ~ N(0, 1), or int32 uniform over [-2**20, 2**20]."""
    r = _rng(seed, STREAM_B)
    if out_dtype == "f16":
        return r.standard_normal(N).astype(np.float16)
    return r.integers(-2**20, 2**20 + 1, size=N).astype(np.int32)


def draw_col_scales(N: int, seed: int) -> np.ndarray:
    """Per-channel fp32 weight scales [N], uniform over [0.001, 0.01]."""
    return _rng(seed, STREAM_C).uniform(0.001, 0.01, size=N).astype(np.float32)


def draw_fp16_activations(M: int, K: int, seed: int) -> np.ndarray:
    """fp16 [M, K] ~ N(0, 1) (the activations that the int8 quantiser reads)."""
    return draw_activations(M, K, "f16", seed)


def draw_zeros(N: int, G: int, seed: int) -> np.ndarray:
    r = _rng(seed, STREAM_Z)
    return r.uniform(6.0, 9.0, size=(N, G)).astype(np.float16)


def make_problem(M: int, N: int, K: int, w_dtype: str, group_size: int = 128,
                 has_zeros: bool = False, seed: int = 1, q: np.ndarray | None = None,
                 A: np.ndarray | None = None, s: np.ndarray | None = None,
                 z: np.ndarray | None = None) -> Problem:
    """Draw (or take) every operand of one problem and encode the weights.

    Any of q, A, s, z may be given explicitly (structured test inputs); the
    rest are drawn from the seeded streams.
    """
    if w_dtype not in W_DTYPES:
        raise ValueError(w_dtype)
    a_dtype = A_OF_W[w_dtype]
    if w_dtype in ("i8", "i2", "f16"):
        group_size, has_zeros = 0, False
    G = num_groups(K, group_size)
    if A is None:
        A = draw_activations(M, K, a_dtype, seed)
    if q is None:
        q = draw_weights(N, K, w_dtype, seed)
    if G and s is None:
        s = draw_scales(N, G, seed)
    if has_zeros and z is None:
        z = draw_zeros(N, G, seed)
    if not G:
        s = None
    if not has_zeros:
        z = None
    w = encode_weights(q, w_dtype)
    return Problem(M, N, K, a_dtype, w_dtype, group_size, bool(has_zeros),
                   np.ascontiguousarray(A), np.ascontiguousarray(q), w,
                   None if s is None else np.ascontiguousarray(s, dtype=np.float16),
                   None if z is None else np.ascontiguousarray(z, dtype=np.float16))
