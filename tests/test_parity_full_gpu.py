"""GPU parity at the benchmark's full sizes, in the launch configuration the
benchmark times, on sampled outputs the oracle computes directly.

Workloads: the pages' grid N = K = 16384 with M in {1, 32, 128, 512, 16384}
(BitBLAS issue #252, reproduction script), the LLaMA-7B projection shapes of
hidet issue #364 with k-parts 1 and 4, and W4A16 with g = 128.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import Case, assert_matches, say

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)


def _sample(n, k, rng):
    """k sorted distinct indices in [0, n), always including the first and last."""
    idx = set(rng.choice(n, size=min(k, n), replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(idx))


def _check_sampled(c, rows, cols, what):
    gpu = c.run()
    ref = c.reference(rows=rows, cols=cols)
    assert_matches(gpu[np.ix_(rows, cols)], ref, what)
    return gpu


LLAMA = [(1, 4096, 4096), (1, 4096, 11008), (1, 11008, 4096), (1, 4096, 32000), (8, 4096, 11008),
         (32, 11008, 4096), (128, 4096, 11008), (128, 11008, 4096), (128, 4096, 4096), (128, 4096, 32000)]


@pytest.mark.parametrize("M,K,N", LLAMA)
@pytest.mark.parametrize("kp,split", [(1, "none"), (4, "atomic"), (4, "det"), (4, "auto")])
def test_w4a16_llama_shapes(M, K, N, kp, split):
    """The LLaMA-7B projection shapes with k-parts 1 and 4 (hidet issue #364): the default
    split-K reduction is fp32 atomics into one accumulator (workspace M * N * 4 bytes),
    run three times (the summation order may change, every result within tolerance);
    the ordered two-pass form is bitwise reproducible."""
    say(f"W4A16 M={M} K={K} N={N} kp={kp} split={split}")
    c = Case(M, N, K, "i4", 128, k_parts=kp, deterministic=split == "det", split_auto=split == "auto",
             seed=synth.seed_for(1, M + kp))
    if split == "atomic":
        assert c.q.ws_bytes == M * N * 4
    elif split == "det":
        assert c.q.ws_bytes == kp * M * N * 4
    rng = np.random.default_rng(0)
    rows = np.arange(M) if M <= 8 else _sample(M, 24, rng)
    cols = _sample(N, 512, rng)
    ref = c.reference(rows=rows, cols=cols)
    first = None
    for r in range(3 if kp > 1 else 1):
        gpu = c.run()
        assert_matches(gpu[np.ix_(rows, cols)], ref, f"W4A16 {M}x{K}x{N} kp={kp} {split} run {r}")
        if split == "det":
            assert first is None or np.array_equal(gpu, first)
            first = gpu


@pytest.mark.parametrize("M", [1, 8, 32, 128, 512])
@pytest.mark.parametrize("w_dtype,kp", [("i8", 1), ("i8", 4), ("i2", 1), ("i2", 4)])
def test_int_grid_full(M, w_dtype, kp):
    say(f"{w_dtype} M={M} N=K=16384 kp={kp}")
    c = Case(M, 16384, 16384, w_dtype, 0, k_parts=kp, seed=synth.seed_for(2 if w_dtype == "i8" else 3, M))
    rng = np.random.default_rng(1)
    rows = np.arange(M) if M <= 32 else _sample(M, 32, rng)
    cols = _sample(16384, 384, rng)
    _check_sampled(c, rows, cols, f"{w_dtype} M={M}")


@pytest.mark.parametrize("kp", [1, 4])
def test_w4a16_m1_16384(kp):
    c = Case(1, 16384, 16384, "i4", 128, k_parts=kp, seed=synth.seed_for(5, kp))
    gpu = c.run()
    assert_matches(gpu, c.reference(), f"W4A16 M=1 16384 kp={kp}")


def _tile_samples(rng, n_tiles=64, T=128, grid=128):
    coords = {(0, 0), (0, grid - 1), (grid - 1, 0), (grid - 1, grid - 1)}
    while len(coords) < n_tiles:
        coords.add(tuple(rng.integers(0, grid, size=2).tolist()))
    return sorted(coords)


@pytest.mark.parametrize("variant", ["dense_f16", "u4_zeros_g128"])
def test_large_m_sampled_tiles(variant):
    """M = N = K = 16384 on 64 sampled 128 x 128 output tiles (incl. the 4 corners)."""
    M = N = K = 16384
    if variant == "dense_f16":
        c = Case(M, N, K, "f16", 0, seed=synth.seed_for(4, 0))
    else:
        c = Case(M, N, K, "u4", 128, True, seed=synth.seed_for(4, 1))
    say(f"large-M {variant}: path {c.q.path}")
    gpu = c.run()
    rng = np.random.default_rng(4)
    for (ti, tj) in _tile_samples(rng):
        rows = np.arange(ti * 128, ti * 128 + 128)
        cols = np.arange(tj * 128, tj * 128 + 128)
        ref = c.reference(rows=rows, cols=cols)
        assert_matches(gpu[np.ix_(rows, cols)], ref, f"{variant} tile ({ti},{tj})")


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 16, 24, 32])
@pytest.mark.parametrize("w_dtype", ["i4", "u4"])
def test_unscaled_int4_long_k(M, w_dtype):
    """Unscaled int4 (the pages' fp16 x int4 configuration without scaling) over K = 16384:
    results spread to about 600 (uint4: several thousand), so those near zero hold the
    absolute 1e-2 tolerance only if no accumulator carries the 1024 + offset of the
    fp16 upcast.  Every output of 1000 columns (dot-product GEMV at M <= 2, matrix-core
    GEMV above)."""
    say(f"unscaled {w_dtype} M={M} N=1000 K=16384")
    c = Case(M, 1000, 16384, w_dtype, 0, seed=synth.seed_for(6, 40 + M))
    assert_matches(c.run(), c.reference(), f"unscaled {w_dtype} M={M}")
