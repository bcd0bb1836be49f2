"""GPU parity of every configuration the benchmark times, in the launch
configuration it times it: the plan comes from the benchmark's own
constructor (same M, N, K, formats, group size, zero points, k-parts, split-K
reduction and output form) and runs through the same entry point
(qgemm_run, qgemm_run_ex with a bias, qgemm_run_scaled), on seeded inputs
with the benchmark's distributions, compared with the CPU oracle on sampled
outputs: every row up to 32 rows (else 32 sampled rows and the edges) and
640 sampled columns with the edges; the M = N = K = 16384 products on 16
sampled 128 x 128 tiles (the four corners among them).

The grid is the pages' N = K = 16384 benchmark shapes with M in {1, 32, 128,
512, 16384} and their op configurations (BitBLAS issue #252, reproduction
script: unscaled int4, per-channel scales, int8 x int8, int8 x int2, dense
fp16), the LLaMA-7B projection shapes with k-parts 1 and 4 (hidet issue #364),
and the bias, dequantised int8 output and int8 quantiser rows.
"""
import zlib

import numpy as np
import pytest
import torch

import bench
import oracle
import synth
from gpu_helpers import assert_matches, say
from weight_quantized_mixed_amd.device import host_to_device, quantize_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


def _key(c):
    return (c["w"], c.get("N", 0), c["K"], c.get("g", 0), c.get("zeros", False))


# grouped by weight so that consecutive entries share one drawn weight
ENTRIES = sorted([bench.HEADLINE] + bench.GRID, key=lambda c: (str(_key(c)), c["M"]))

_cache = {}


def _weights(c):
    """Drawn weights of an entry's (format, N, K, g, zeros), the last one kept."""
    key = _key(c)
    if key not in _cache:
        _cache.clear()
        g = c.get("g", 0) if c["w"] in ("i4", "u4") else 0
        _cache[key] = synth.make_problem(1, c["N"], c["K"], c["w"], group_size=g,
                                         has_zeros=c.get("zeros", False),
                                         seed=synth.seed_for(6, zlib.crc32(str(key).encode()) % 97))
    return _cache[key]


def _sample(n, k, rng, edges=()):
    idx = set(rng.choice(n, size=min(k, n), replace=False).tolist()) | {0, n - 1} | {e for e in edges if e < n}
    return np.array(sorted(idx))


def _tiles(rng, grid, n_tiles):
    coords = {(0, 0), (0, grid - 1), (grid - 1, 0), (grid - 1, grid - 1)}
    while len(coords) < n_tiles:
        coords.add(tuple(rng.integers(0, grid, size=2).tolist()))
    return sorted(coords)


def _check_quantiser(c):
    M, K = c["M"], c["K"]
    A = synth.draw_fp16_activations(M, K, seed=synth.seed_for(7, M))
    Q, S = quantize_rows(host_to_device(A))
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 512 else _sample(M, 256, np.random.default_rng(M))
    q_ref, s_ref = oracle.quantize_rows(A[rows])
    assert np.array_equal(S.cpu().numpy()[rows], s_ref)
    assert np.array_equal(Q.cpu().numpy()[rows], q_ref)


@pytest.mark.parametrize("c", ENTRIES, ids=bench.label)
def test_bench_entry_matches_oracle(c):
    say(f"bench entry {bench.label(c)}")
    if c["w"] == "quant":
        _check_quantiser(c)
        return
    M, N, K = c["M"], c["N"], c["K"]
    base = _weights(c)
    q = bench.make_qgemm(c)
    seed = synth.seed_for(6, M)
    A = synth.draw_activations(M, K, q.a_dtype, seed)
    p = synth.make_problem(M, N, K, c["w"], group_size=base.group_size, has_zeros=base.has_zeros,
                           q=base.q, A=A, s=base.s, z=base.z)
    packed = q.pack(host_to_device(p.w), host_to_device(p.s), host_to_device(p.z))
    bias = synth.draw_bias(N, q.out_dtype, seed + 5) if c.get("bias") else None
    rs = synth.draw_col_scales(M, seed + 6) if c.get("dq") else None
    cs = synth.draw_col_scales(N, seed + 7) if c.get("dq") else None
    C = q.new_output()
    bench.run_entry(q, c, host_to_device(p.A), packed, C, q.workspace(),
                    host_to_device(bias), host_to_device(rs), host_to_device(cs))
    torch.cuda.synchronize()
    gpu = C.cpu().numpy()
    q.close()

    def ref(rows, cols):
        if c.get("dq"):
            return oracle.qgemm_ref_scaled(p.A, p.w, N=N, K=K, w_dtype=p.w_dtype, row_scales=rs,
                                           col_scales=cs, bias=bias, rows=rows, cols=cols)
        return oracle.qgemm_ref(p.A, p.w, p.s, p.z, N=N, K=K, w_dtype=p.w_dtype, group_size=p.group_size,
                                rows=rows, cols=cols, bias=bias)

    rng = np.random.default_rng(M + N + K)
    what = bench.label(c)
    if M == 16384:
        for (ti, tj) in _tiles(rng, M // 128, 16):
            rows = np.arange(ti * 128, ti * 128 + 128)
            cols = np.arange(tj * 128, tj * 128 + 128)
            assert_matches(gpu[np.ix_(rows, cols)], ref(rows, cols), f"{what} tile ({ti},{tj})")
        return
    rows = np.arange(M) if M <= 32 else _sample(M, 32, rng, edges=(63, 64, 127, 128, 255, 256))
    cols = _sample(N, 640, rng, edges=(15, 16, 63, 64, 255, 256))
    assert_matches(gpu[np.ix_(rows, cols)], ref(rows, cols), what)
