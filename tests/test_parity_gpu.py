"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer formats must match bit for bit; fp16 outputs within
|gpu - ref| <= 1e-2 + 5e-3*|ref| of the unrounded float64 reference.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import Case, assert_matches, say
from weight_quantized_mixed_amd import qgemm as q

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU containers
    pytest.skip("needs a GPU", allow_module_level=True)


# ---------------------------------------------------------------- small shapes, every path
SMALL = [
    # M, N, K, w_dtype, g, zeros
    (1, 72, 512, "i4", 128, False),
    (3, 300, 1024, "i4", 128, False),
    (8, 136, 768, "i4", 64, False),
    (2, 200, 512, "i4", 32, False),
    (1, 264, 1024, "i4", -1, False),
    (5, 88, 512, "i4", 0, False),
    (4, 136, 1024, "u4", 128, True),
    (1, 72, 512, "u4", 32, True),
    (6, 100, 1024, "u4", 256, False),
    (1, 200, 1024, "f16", 0, False),
    (7, 72, 512, "f16", 0, False),
    (1, 300, 1024, "i8", 0, False),
    (8, 136, 512, "i8", 0, False),
    (1, 200, 2048, "i2", 0, False),
    (5, 72, 1024, "i2", 0, False),
    (1, 88, 512, "i4", 64, False),
    (1, 136, 1024, "i4", 0, False),
    # group sizes that are not whole 128-position superblocks (per-piece scales), and a
    # deeper group that is not a power of two (its index by division)
    (1, 300, 1920, "i4", 160, False),
    (4, 136, 1920, "u4", 96, True),
    (1, 72, 1920, "u4", 160, True),
    (1, 200, 1536, "i4", 384, False),
    (40, 264, 1920, "u4", 160, True),
    (70, 136, 1920, "i4", 96, False),
    (40, 264, 1536, "u4", 384, True),
    (300, 520, 1536, "i4", 384, False),
    # int4 / uint4 rows 3..32 on the matrix cores (bias-folded operands, per-superblock fold)
    (4, 520, 2048, "i4", 0, False),
    (3, 136, 1024, "u4", -1, True),
    (28, 200, 1024, "i4", 0, False),
    (5, 200, 1024, "i4", 128, False),
    (16, 264, 1024, "u4", 128, True),
    (17, 300, 2048, "i4", -1, False),
    (32, 520, 1024, "u4", 128, True),
    (12, 136, 512, "i4", 0, False),
    (24, 72, 1536, "u4", 384, True),
    # int8 / int2 rows 9..32 on the matrix cores (two row blocks past 16)
    (16, 200, 2048, "i2", 0, False),
    (17, 136, 1024, "i2", 0, False),
    (32, 264, 2048, "i2", 0, False),
    (24, 520, 512, "i8", 0, False),
    # the matrix-core GEMVs with two 16-column blocks per workgroup (N = 6000) and one
    # (N = 4096 at k_parts 1)
    (8, 6000, 512, "i8", 0, False),
    (20, 6000, 1024, "i4", 128, False),
    (4, 6000, 1024, "f16", 0, False),
    (3, 6000, 2048, "i2", 0, False),
    (30, 4096, 1024, "u4", 128, True),
    (12, 4096, 1024, "i2", 0, False),
    # two int4 rows on the matrix cores when N is narrow
    (2, 4096, 1024, "i4", 128, False),
    (2, 520, 1024, "u4", 128, True),
    (2, 1000, 512, "i4", 0, False),
    # int8 / int2 rows 2..8 on the matrix cores (ragged last 64-column block)
    (2, 200, 1024, "i8", 0, False),
    (3, 72, 2048, "i2", 0, False),
    (8, 264, 2048, "i2", 0, False),
    (6, 1000, 512, "i8", 0, False),
    # M = 1 with 16-column workgroups at k_parts 1, 64-column blocks at k_parts 3
    (1, 2752, 512, "u4", 128, True),
    (1, 2752, 1024, "i2", 0, False),
    (1, 2752, 256, "f16", 0, False),
    # MFMA path (M > 8): several tiles and ragged tails in M and N
    (9, 72, 512, "i4", 128, False),
    (33, 200, 1024, "i4", 128, False),
    (130, 264, 768, "i4", 64, False),
    (129, 136, 512, "u4", 128, True),
    (64, 72, 1024, "u4", 32, True),
    (40, 88, 512, "i4", 0, False),
    (70, 136, 512, "i4", -1, False),
    (33, 200, 512, "f16", 0, False),
    (257, 300, 256, "f16", 0, False),
    (33, 300, 1024, "i8", 0, False),
    (129, 136, 512, "i8", 0, False),
    (9, 72, 2048, "i2", 0, False),
    (160, 264, 1024, "i2", 0, False),
]


@pytest.mark.parametrize("M,N,K,w_dtype,g,zeros", SMALL)
@pytest.mark.parametrize("kp,det", [(1, False), (3, False), (3, True)])
def test_small_parity(M, N, K, w_dtype, g, zeros, kp, det):
    say(f"case M={M} N={N} K={K} {w_dtype} g={g} zeros={zeros} kp={kp} det={det}")
    c = Case(M, N, K, w_dtype, g, zeros, k_parts=kp, deterministic=det, seed=M * 1000 + N + K)
    assert c.q.path == (q.QGEMM_PATH_GEMV if M <= 8 else q.QGEMM_PATH_MFMA)
    assert_matches(c.run(), c.reference(), f"M={M} N={N} K={K} {w_dtype} kp={kp}")


# ---------------------------------------------------------------- layout pins (one-hot A)
@pytest.mark.parametrize("M,w_dtype", [(1, "i4"), (20, "i4"), (1, "i2"), (40, "i2"), (1, "i8"), (40, "i8"),
                                       (1, "f16"), (40, "f16")])
def test_one_hot_activation_bitwise(M, w_dtype):
    """A = e_k0 in every row: C[:, n] is the single dequantised weight, rounded once."""
    N, K = 72, 512
    base = synth.make_problem(M, N, K, w_dtype, group_size=128, seed=77)
    for k0 in (0, 37, 128, 300, 511):
        A = np.zeros((M, K), dtype=base.A.dtype)
        A[:, k0] = 1
        p = synth.make_problem(M, N, K, w_dtype, group_size=128, q=base.q, A=A, s=base.s, seed=77)
        say(f"one-hot M={M} {w_dtype} k0={k0}")
        c = Case(0, 0, 0, None, problem=p)
        gpu = c.run()
        ref = c.reference()
        if ref.dtype == np.int64:
            assert np.array_equal(gpu.astype(np.int64), ref)
        else:
            assert np.array_equal(gpu, oracle.round_fp16(ref)), k0


def test_constant_closed_form_zeros():
    """A = 1, q = c, zero point z, scale s0: C = K (c - z) s0 everywhere (MFMA and GEMV)."""
    for M in (1, 24):
        N, K, c0 = 80, 1024, 11
        A = np.ones((M, K), dtype=np.float16)
        qv = np.full((N, K), c0, dtype=np.int8)
        s = np.full((N, K // 128), 0.0125, dtype=np.float16)
        z = np.full((N, K // 128), 7.5, dtype=np.float16)
        p = synth.make_problem(M, N, K, "u4", 128, True, q=qv, A=A, s=s, z=z)
        gpu = Case(0, 0, 0, None, problem=p).run()
        expect = K * (c0 - 7.5) * float(np.float16(0.0125))
        assert np.all(gpu == np.float16(expect)), (M, gpu[0, :4], expect)


# ---------------------------------------------------------------- split-K properties
@pytest.mark.parametrize("M,w_dtype,g", [(1, "i4", 128), (4, "i8", 0), (64, "i4", 128), (33, "i2", 0)])
def test_two_pass_is_bitwise_reproducible(M, w_dtype, g):
    c = Case(M, 264, 2048, w_dtype, g, k_parts=4, deterministic=True, seed=5)
    first = c.run()
    for _ in range(9):
        assert np.array_equal(c.run(), first)
    assert_matches(first, c.reference(), "two-pass")


@pytest.mark.parametrize("M,w_dtype", [(1, "i8"), (2, "i2"), (100, "i8"), (40, "i2")])
def test_int_atomics_exact_every_run(M, w_dtype):
    c = Case(M, 200, 4096, w_dtype, 0, k_parts=4, seed=6)
    ref = c.reference()
    for _ in range(3):
        assert np.array_equal(c.run().astype(np.int64), ref)


def test_kparts_agree_on_int():
    p = synth.make_problem(3, 136, 4096, "i2", seed=9)
    outs = [Case(0, 0, 0, None, k_parts=kp, problem=p).run() for kp in (1, 2, 4, 16)]
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


# ---------------------------------------------------------------- host-side errors on a live device
def test_run_rejects_small_workspace():
    c = Case(2, 72, 512, "i4", 128, k_parts=2, deterministic=True, seed=3)
    ws = torch.empty(c.q.ws_bytes - 4, dtype=torch.uint8, device="cuda")
    C = c.q.new_output()
    with pytest.raises(q.QGemmError) as e:
        q.qgemm_run(c.q.plan, c.A.data_ptr(), c.packed.data_ptr(), C.data_ptr(), ws.data_ptr(),
                    ws.numel(), torch.cuda.current_stream().cuda_stream)
    assert e.value.status == q.QGEMM_ERR_INVALID_ARG


def test_shared_blob_across_plans():
    """One packed weight serves the GEMV and the MFMA plan of the same (N, K, format)."""
    N, K = 136, 1024
    p1 = synth.make_problem(1, N, K, "i4", 128, seed=12)
    c1 = Case(0, 0, 0, None, problem=p1)
    p2 = synth.make_problem(48, N, K, "i4", 128, q=p1.q, s=p1.s, seed=13)
    c2 = Case(0, 0, 0, None, problem=p2)
    assert c1.q.packed_bytes == c2.q.packed_bytes
    out = c2.q.run(c2.A, c1.packed)
    torch.cuda.synchronize()
    assert_matches(out.cpu().numpy(), c2.reference(), "shared blob")


# ---------------------------------------------------------------- 256 x 256 tile path (large M)
BIG = [
    # M, N, K, w_dtype, g, zeros   (>= 256 workgroups of 256 x 256, ragged M and N)
    (4100, 4104, 512, "f16", 0, False),
    (4096, 4100, 512, "i8", 0, False),
    (4097, 4096, 768, "i2", 0, False),
    (4096, 4104, 512, "i4", 128, False),
    (4100, 4096, 512, "u4", 128, True),
    (4096, 4096, 512, "u4", 256, False),
    (4096, 4096, 384, "i4", -1, False),
    (4096, 4096, 256, "i4", 0, False),
    # uint4 with zero points and int4 with scale groups, folded out of the K loop (255
    # tiles of 256 x 256 fill the CUs at k_parts 1 as well): one group over K (with a K
    # tail read zero-padded), groups of three superblocks
    (4100, 3836, 1000, "u4", -1, True),
    (4100, 3836, 768, "u4", 384, True),
    (4100, 3836, 512, "i4", 128, False),
    (4100, 3836, 768, "i4", 384, False),
]


@pytest.mark.parametrize("M,N,K,w_dtype,g,zeros", BIG)
@pytest.mark.parametrize("kp,det", [(1, False), (2, False), (2, True)])
def test_big_tile_parity(M, N, K, w_dtype, g, zeros, kp, det):
    say(f"big M={M} N={N} K={K} {w_dtype} g={g} zeros={zeros} kp={kp} det={det}")
    c = Case(M, N, K, w_dtype, g, zeros, k_parts=kp, deterministic=det, seed=M + N + K + kp)
    rng = np.random.default_rng(2)
    rows = np.unique(np.concatenate([rng.choice(M, 300, replace=False), [0, 255, 256, M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(N, 300, replace=False), [0, 255, 256, N - 1]]))
    gpu = c.run()
    assert_matches(gpu[np.ix_(rows, cols)], c.reference(rows=rows, cols=cols),
                   f"big {w_dtype} M={M} N={N} kp={kp}")


# uint4 with zero points on the 256 x 256 tiles subtracts rne(z) in the K loop and
# adds -sum_g R[m, g] s (z - rne(z)) after it, R the row sums of A over each scale group
# (held as bf16 hi + lo).  A bias, runs of fewer rows than the plan's (4100 rows of 3836
# columns: 255 tiles, 2900 rows: 180, both on 256 x 256 tiles), and activations whose
# group sums pass the fp16 range (a constant 1000: R = 128000 per group; scales 2^-6,
# so that both sides are exact up to the fp32 sums and any overflow of R shows).
@pytest.mark.parametrize("w_dtype,zeros", [("u4", True), ("i4", False)])
def test_zero_fold_bias_fewer_rows_and_large_sums(w_dtype, zeros):
    M, N, K = 4100, 3836, 512
    say(f"zero fold M={M} N={N} K={K} {w_dtype} g=128 zeros={zeros}: bias, fewer rows, large sums")
    c = Case(M, N, K, w_dtype, 128, zeros, seed=91)
    b = synth.draw_bias(N, "f16", 92)
    rng = np.random.default_rng(93)
    cols = np.unique(np.concatenate([rng.choice(N, 300, replace=False), [0, 255, 256, N - 1]]))
    for m in (M, 2900):
        rows = np.unique(np.concatenate([rng.choice(m, 200, replace=False), [0, 255, 256, m - 1]]))
        gpu = c.run(bias=b, M=m)
        assert gpu.shape == (m, N)
        assert_matches(gpu[np.ix_(rows, cols)], c.reference(rows=rows, cols=cols, bias=b),
                       f"zero fold bias M={m}")
    M, N = 4096, 4096
    p = synth.make_problem(M, N, K, w_dtype, group_size=128, has_zeros=zeros, seed=94)
    big = synth.make_problem(M, N, K, w_dtype, group_size=128, has_zeros=zeros, seed=94,
                             A=np.full((M, K), 1000, dtype=np.float16), q=p.q,
                             s=np.full_like(p.s, 2.0 ** -6), z=p.z)
    c2 = Case(M, N, K, w_dtype, 128, zeros, problem=big)
    rows = np.unique(np.concatenate([rng.choice(M, 100, replace=False), [0, M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(N, 300, replace=False), [0, N - 1]]))
    gpu = c2.run()
    assert_matches(gpu[np.ix_(rows, cols)], c2.reference(rows=rows, cols=cols), "zero fold large sums")


# fp16 outputs reduce split-K with ordered partials unless those would pass 256 MiB of
# workspace; past it the atomic accumulator (zero fill, fp32 atomics, finalize) remains
@pytest.mark.parametrize("w_dtype,g,zeros", [("i4", 128, False), ("u4", 128, True), ("f16", 0, False)])
def test_atomic_split_past_the_partials_cap(w_dtype, g, zeros):
    M, N, K = 4100, 8400, 256
    say(f"atomic split M={M} N={N} K={K} {w_dtype} g={g} zeros={zeros} kp=2")
    c = Case(M, N, K, w_dtype, g, zeros, k_parts=2, seed=M + N + 17)
    # uint4 with zero points and int4 with scale groups on the 256 x 256 tiles: after
    # the accumulator, the two bf16 planes of the row sums over the scale groups (K / g
    # = 2, padded to 32 per plane) and those of the per-column term for the 8448 padded
    # columns
    zr = (M + 8448) * 32 * 2 * 2 if w_dtype in ("i4", "u4") else 0
    assert c.q.ws_bytes == M * N * 4 + zr
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([rng.choice(M, 200, replace=False), [0, 255, 256, M - 1]]))
    cols = np.unique(np.concatenate([rng.choice(N, 200, replace=False), [0, 255, 256, N - 1]]))
    gpu = c.run()
    assert_matches(gpu[np.ix_(rows, cols)], c.reference(rows=rows, cols=cols), f"atomic split {w_dtype}")


# ---------------------------------------------------------------- direct-load tiles of every shape
# The tile is the largest one within M's power-of-two row cap whose last wave of
# workgroups (N / BN x M / BM x k_parts) still occupies 60 % of the 256 CUs; up to 32
# rows every format takes a matrix-core GEMV instead.  These shapes select, in order:
# 32x64, 32x128 (33..64 rows and few columns), 64x128, 64x256, 128x256, 256x256,
# 128x128 (int4 / uint4 / int2; 64x256 for the others), the skinny matrix-core GEMV
# with k_parts 4, and 128x256 at 400 rows (rows and columns ragged).
DL_SHAPES = [(40, 1000, 1, False), (40, 12000, 1, False), (40, 16376, 2, False), (40, 16376, 4, True),
             (100, 16376, 4, False), (300, 16376, 2, True), (100, 24000, 1, False), (20, 16376, 4, False),
             (400, 16376, 1, False)]
DL_FORMATS = [("i4", 128, False), ("u4", 128, True), ("u4", 256, False), ("i4", 0, False), ("f16", 0, False),
              ("i8", 0, False), ("i2", 0, False), ("i4", -1, False)]


@pytest.mark.parametrize("M,N,kp,det", DL_SHAPES)
@pytest.mark.parametrize("w_dtype,g,zeros", DL_FORMATS)
def test_direct_load_tiles(M, N, kp, det, w_dtype, g, zeros):
    K = 1024
    say(f"dl M={M} N={N} K={K} {w_dtype} g={g} zeros={zeros} kp={kp} det={det}")
    c = Case(M, N, K, w_dtype, g, zeros, k_parts=kp, deterministic=det, seed=7 * M + kp)
    rng = np.random.default_rng(M + kp)
    cols = np.unique(np.concatenate([rng.choice(N, 400, replace=False), [0, 63, 64, 255, 256, N - 1]]))
    gpu = c.run()
    assert_matches(gpu[:, cols], c.reference(cols=cols), f"dl {w_dtype} M={M} kp={kp}")


# ---------------------------------------------------------------- four-group tiles, odd superblock counts
# The int4 tiles of four K groups (32x64 at 40 and 100 rows of 1000 columns, 32x128 at
# 40 rows of 12000) load four stages, two superblocks, per round; a part of an odd
# number of superblocks ends inside a round, whose missing stages are clamped copies,
# and scale groups of two or three superblocks change inside a round.
ODD_SB_SHAPES = [(40, 1000, 1), (40, 1000, 3), (100, 1000, 3), (40, 12000, 2)]
ODD_SB_FORMATS = [("i4", 128, False, 4224), ("u4", 128, True, 4224), ("i4", 0, False, 4224),
                  ("u4", 256, False, 4352), ("i4", 384, False, 4224)]


@pytest.mark.parametrize("M,N,kp", ODD_SB_SHAPES)
@pytest.mark.parametrize("w_dtype,g,zeros,K", ODD_SB_FORMATS)
def test_direct_load_odd_superblocks(M, N, kp, w_dtype, g, zeros, K):
    say(f"odd superblocks M={M} N={N} K={K} {w_dtype} g={g} zeros={zeros} kp={kp}")
    c = Case(M, N, K, w_dtype, g, zeros, k_parts=kp, seed=5 * M + kp + g)
    rng = np.random.default_rng(M + N + kp)
    cols = np.unique(np.concatenate([rng.choice(N, min(N, 300), replace=False), [0, 63, 64, N - 1]]))
    gpu = c.run()
    assert_matches(gpu[:, cols], c.reference(cols=cols), f"odd superblocks {w_dtype} g={g} M={M} kp={kp}")


# ---------------------------------------------------------------- HIP graph capture
GRAPH_CASES = [(1, 200, 1024, "i4", 128, False, 1, False), (1, 2752, 1024, "i2", 0, False, 3, False),
               (4, 300, 1024, "u4", 128, True, 1, False), (40, 264, 1024, "i4", 128, False, 2, False),
               (1, 4096, 4096, "i4", 128, False, 4, False), (40, 264, 1024, "i4", 128, False, 2, True),
               (40, 264, 1024, "i8", 0, False, 2, True), (300, 520, 512, "f16", 0, False, 1, False)]


@pytest.mark.parametrize("M,N,K,w_dtype,g,zeros,kp,det", GRAPH_CASES)
def test_graph_replays_match_eager(M, N, K, w_dtype, g, zeros, kp, det):
    """qgemm_run captured in a HIP graph (with its zero-fill and conversion kernels for
    split-K): every replay, with eager work between them, matches the oracle, and gives
    the eager result bit for bit where the reduction is ordered (integers, k_parts = 1,
    two-pass)."""
    say(f"graph M={M} N={N} K={K} {w_dtype} g={g} zeros={zeros} kp={kp} det={det}")
    c = Case(M, N, K, w_dtype, g, zeros, k_parts=kp, deterministic=det, seed=11 * M + N)
    if kp > 1 and not det and w_dtype in ("i4", "u4", "f16"):
        assert c.q.ws_bytes == M * N * 4   # fp32 atomics into one accumulator
    ref = c.reference()
    eager = c.run()
    assert_matches(eager, ref, "eager")
    C = c.q.new_output()
    ws = c.q.workspace()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            c.q.run(c.A, c.packed, C, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    exact = w_dtype in ("i8", "i2") or kp == 1 or det
    for r in range(3):
        C.zero_()
        graph.replay()
        torch.cuda.synchronize()
        got = C.cpu().numpy()
        assert_matches(got, ref, f"graph replay {r}")
        if exact:
            assert np.array_equal(got, eager), f"replay {r} differs from the eager result"
        c.run()  # eager work between replays
        torch.cuda.synchronize()


# ---------------------------------------------------------------- K not a multiple of the block depth
# K needs only whole canonical words (8 int4, 16 int2 values) and whole groups: the
# blob pads K to whole blocks with zero codes (zero scales for 96-position groups past
# K) and each run reads activations zero-padded in the workspace.
ODD_K = [
    # M, N, K, w_dtype, g, zeros
    (1, 300, 4104, "i4", 0, False),       # dot-product GEMV
    (1, 300, 4104, "i4", -1, False),
    (3, 300, 4104, "u4", -1, True),       # matrix-core int4 GEMV
    (8, 136, 4104, "i4", 0, False),
    (20, 264, 4104, "i4", -1, False),
    (40, 264, 4104, "u4", -1, True),      # direct-load MFMA
    (300, 520, 4104, "i4", 0, False),
    (1, 200, 4128, "i4", 96, False),      # per-piece groups, one padded scale row
    (40, 136, 4128, "u4", 96, True),      # LDS-staged MFMA
    (1, 200, 4112, "i2", 0, False),
    (5, 72, 4112, "i2", 0, False),
    (40, 264, 4112, "i2", 0, False),
    (1, 300, 4100, "i8", 0, False),       # int8 rows 4100 bytes apart (not 16-byte aligned)
    (8, 136, 4100, "i8", 0, False),
    (130, 264, 4100, "i8", 0, False),
    (1, 200, 4099, "f16", 0, False),      # fp16 rows 8198 bytes apart
    (33, 200, 4099, "f16", 0, False),
    (7, 72, 1000, "f16", 0, False),
]


@pytest.mark.parametrize("M,N,K,w_dtype,g,zeros", ODD_K)
@pytest.mark.parametrize("kp,det", [(1, False), (3, False), (3, True)])
def test_k_not_a_multiple_of_the_block(M, N, K, w_dtype, g, zeros, kp, det):
    say(f"odd K M={M} N={N} K={K} {w_dtype} g={g} zeros={zeros} kp={kp} det={det}")
    c = Case(M, N, K, w_dtype, g, zeros, k_parts=kp, deterministic=det, seed=M * 7 + N + K)
    assert_matches(c.run(), c.reference(), f"odd K M={M} N={N} K={K} {w_dtype} kp={kp}")


def test_k_of_one_int4_word():
    c = Case(3, 100, 8, "i4", 0, False, seed=31)
    assert_matches(c.run(), c.reference(), "K = 8")


@pytest.mark.parametrize("w_dtype,g,zeros,kp", [("i4", 0, False, 1), ("u4", -1, True, 3), ("i8", 0, False, 2)])
def test_k_tail_with_fewer_rows_and_bias(w_dtype, g, zeros, kp):
    """qgemm_run_ex on fewer rows than the plan's, with a bias, at a padded K."""
    K = {"i4": 4104, "u4": 4104, "i8": 4100}[w_dtype]
    c = Case(40, 264, K, w_dtype, g, zeros, k_parts=kp, seed=32 + kp)
    b = synth.draw_bias(264, c.q.out_dtype, 33)
    for M in (1, 7, 40):
        assert_matches(c.run(M=M, bias=b), c.reference(rows=np.arange(M), bias=b), f"rows {M} K={K}")


# ---------------------------------------------------------------- the library's own K split
@pytest.mark.parametrize("M,w_dtype,g,zeros", [(32, "i4", 128, False), (20, "u4", 128, True), (12, "i4", -1, False)])
def test_library_k_split_skinny(M, w_dtype, g, zeros):
    """Plans of 9..32 rows at N <= 4096, K >= 8192 (the matrix-core int4 GEMV): the
    library takes four ordered parts for runs of 17 rows and more (two below 17 rows
    when the plan itself has at most 16): oracle parity, bitwise repeats, and run-time
    row counts on both sides of the threshold."""
    N, K = 4096, 11008
    say(f"library split skinny M={M} {w_dtype} g={g} zeros={zeros}")
    c = Case(M, N, K, w_dtype, g, zeros, seed=4500 + M)
    assert c.q.ws_bytes == (4 if M > 16 else 2) * M * N * 4
    first = c.run()
    assert_matches(first, c.reference(), f"skinny split M={M}")
    assert np.array_equal(c.run(), first)
    b = synth.draw_bias(N, "f16", 4501)
    for m in (1, 8, 9, 16, 17, M):
        if m <= M:
            assert_matches(c.run(M=m, bias=b), c.reference(rows=np.arange(m), bias=b), f"rows {m} of {M}")


@pytest.mark.parametrize("M,w_dtype,g,zeros", [(33, "i4", 128, False), (128, "u4", 128, True),
                                               (256, "i4", -1, False), (100, "u4", 0, False)])
def test_library_k_split_reproducible(M, w_dtype, g, zeros):
    """Plans of k_parts 1 that the library splits itself (int4 / uint4, 33..256 rows,
    N >= 4096, K >= 8192; at N = 4096 eight parts up to 128 rows, four above): oracle
    parity, bitwise-identical repeats, and run-time row counts on both sides of the split
    (32 rows and fewer run unsplit)."""
    N, K = 4096, 8192
    say(f"library split M={M} {w_dtype} g={g} zeros={zeros}")
    c = Case(M, N, K, w_dtype, g, zeros, seed=4400 + M)
    assert c.q.ws_bytes == (8 if M <= 128 else 4) * M * N * 4
    first = c.run()
    assert_matches(first, c.reference(), f"library split M={M}")
    for _ in range(3):
        assert np.array_equal(c.run(), first)
    b = synth.draw_bias(N, "f16", 4401)
    for m in (1, 8, 32, 33, M):
        if m <= M:
            assert_matches(c.run(M=m, bias=b), c.reference(rows=np.arange(m), bias=b), f"rows {m} of {M}")
