"""Host-side checks of the C ABI (no device calls): the library loads, exports
every function the header declares, and qgemm_create / qgemm_pack_weights /
qgemm_run reject bad arguments with the documented status before any launch.
"""
import os
import re

import pytest

from weight_quantized_mixed_amd import qgemm as q

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qgemm.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "bitblas_matmul_grid.txt")


def test_library_exports_every_declared_function():
    lib = q.load()
    text = open(HEADER).read()
    declared = set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**(qgemm_[a-z_]+)\s*\(", text, re.M))
    assert declared == set(q.EXPORTED), declared
    for name in declared:
        assert hasattr(lib, name), name


def _create(**kw):
    args = dict(M=1, N=4096, K=4096, a_dtype="f16", w_dtype="i4", out_dtype="f16", accum_dtype="f32",
                group_size=128, has_zeros=0, k_parts=1, flags=0)
    args.update(kw)
    return q.qgemm_create(**args)


def _status(**kw):
    try:
        plan, _, _ = _create(**kw)
    except q.QGemmError as e:
        return e.status
    q.qgemm_destroy(plan)
    return q.QGEMM_OK


def test_create_valid_formats():
    for kw in [dict(), dict(w_dtype="u4", has_zeros=1), dict(w_dtype="f16", group_size=0),
               dict(a_dtype="i8", w_dtype="i8", out_dtype="i32", accum_dtype="i32", group_size=0),
               dict(a_dtype="i8", w_dtype="i2", out_dtype="i32", accum_dtype="i32", group_size=0),
               dict(a_dtype="i8", w_dtype="i8", out_dtype="f16", accum_dtype="i32", group_size=0),
               dict(a_dtype="i8", w_dtype="i2", out_dtype="f16", accum_dtype="i32", group_size=0)]:
        assert _status(**kw) == q.QGEMM_OK, kw


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), q.QGEMM_ERR_INVALID_ARG),
    (dict(N=-3), q.QGEMM_ERR_INVALID_ARG),
    (dict(K=0), q.QGEMM_ERR_INVALID_ARG),
    (dict(k_parts=0), q.QGEMM_ERR_INVALID_ARG),
    (dict(k_parts=33), q.QGEMM_ERR_INVALID_ARG),          # 4096 / 128 = 32 units
    (dict(flags=4), q.QGEMM_ERR_INVALID_ARG),
    (dict(has_zeros=2), q.QGEMM_ERR_INVALID_ARG),
    (dict(group_size=-2), q.QGEMM_ERR_INVALID_ARG),
    (dict(a_dtype=99), q.QGEMM_ERR_INVALID_ARG),
    (dict(accum_dtype="f16"), q.QGEMM_ERR_UNSUPPORTED),   # fp16 accumulation
    (dict(a_dtype="i8", w_dtype="i8", out_dtype="i8", accum_dtype="i32", group_size=0),
     q.QGEMM_ERR_UNSUPPORTED),                              # int8 output
    (dict(w_dtype="i8"), q.QGEMM_ERR_UNSUPPORTED),          # fp16 x int8
    (dict(has_zeros=1), q.QGEMM_ERR_UNSUPPORTED),           # zeros need uint4
    (dict(w_dtype="u4", has_zeros=1, group_size=0), q.QGEMM_ERR_UNSUPPORTED),
    (dict(group_size=48), q.QGEMM_ERR_UNSUPPORTED),         # not a multiple of 32
    (dict(group_size=96, K=4096), q.QGEMM_ERR_UNSUPPORTED),  # does not divide K
    (dict(K=4000), q.QGEMM_ERR_UNSUPPORTED),                # g = 128 does not divide K
    (dict(K=4100, group_size=0), q.QGEMM_ERR_UNSUPPORTED),  # not whole int4 words (8 values)
    (dict(K=4100, group_size=-1), q.QGEMM_ERR_UNSUPPORTED),
    (dict(a_dtype="i8", w_dtype="i2", out_dtype="i32", accum_dtype="i32", group_size=0, K=4104),
     q.QGEMM_ERR_UNSUPPORTED),                              # not whole int2 words (16 values)
    (dict(a_dtype="i8", w_dtype="i2", out_dtype="i32", accum_dtype="i32", group_size=128),
     q.QGEMM_ERR_UNSUPPORTED),                              # int formats are unscaled
])
def test_create_rejects(kw, status):
    assert _status(**kw) == status


@pytest.mark.parametrize("g,K,max_parts", [
    (128, 4096, 32),    # groups of whole superblocks: one split unit per superblock
    (512, 4096, 8),     # ... and per group when groups are deeper
    (-1, 4096, 32),     # one group over K
    (160, 1920, 15),    # groups that are not whole superblocks (per-piece scales):
    (96, 1920, 15),     #   parts split at superblocks, not at groups
])
def test_split_unit_follows_the_scale_mode(g, K, max_parts):
    assert _status(group_size=g, K=K, k_parts=max_parts) == q.QGEMM_OK
    assert _status(group_size=g, K=K, k_parts=max_parts + 1) == q.QGEMM_ERR_INVALID_ARG


def test_sizes_and_paths():
    plan, pb, wb = _create()
    assert pb == 4096 * 4096 // 2 + 4096 * 32 * 2 and wb == 0
    assert q.qgemm_plan_path(plan) == q.QGEMM_PATH_GEMV
    q.qgemm_destroy(plan)
    plan, pb, wb = _create(M=9, N=100, k_parts=4)
    npad = 256
    assert pb == npad * 4096 // 2 + npad * 32 * 2
    assert wb == 9 * 100 * 4                                # default split-K: one fp32 accumulator
    assert q.qgemm_plan_path(plan) == q.QGEMM_PATH_MFMA
    q.qgemm_destroy(plan)
    plan, pb, wb = _create(M=9, N=100, k_parts=4, flags=q.QGEMM_DETERMINISTIC)
    assert wb == 4 * 9 * 100 * 4                            # per-part partials
    q.qgemm_destroy(plan)
    plan, pb, wb = _create(M=9, N=100, k_parts=4, flags=q.QGEMM_SPLIT_AUTO)
    assert wb == 4 * 9 * 100 * 4                            # auto: fp16 outputs take the partials
    q.qgemm_destroy(plan)
    # int4 with g = 128 on the 256 x 256 tiles: the workspace ends with the planes of the
    # offset folding (row sums of A over 32 groups for each row, the per-column term for
    # each of the 8448 padded columns; two bf16 planes of 32 values each)
    fold = (4100 + 8448) * 32 * 2 * 2
    plan, pb, wb = _create(M=4100, N=8400, K=4096, k_parts=2, flags=q.QGEMM_SPLIT_AUTO)
    assert wb == 4100 * 8400 * 4 + fold                     # ... until they pass 256 MiB
    q.qgemm_destroy(plan)
    plan, pb, wb = _create(M=4100, N=8400, K=4096, k_parts=2,
                           flags=q.QGEMM_DETERMINISTIC | q.QGEMM_SPLIT_AUTO)
    assert wb == 2 * 4100 * 8400 * 4 + fold                 # deterministic: partials regardless
    q.qgemm_destroy(plan)
    i8 = dict(a_dtype="i8", w_dtype="i8", out_dtype="i32", accum_dtype="i32", group_size=0)
    plan, pb, wb = _create(k_parts=4, **i8)
    assert wb == 0                                          # int32 atomics go straight into C
    q.qgemm_destroy(plan)
    plan, pb, wb = _create(M=128, k_parts=4, **i8)
    assert wb == 0                                          # ... at any M by default
    q.qgemm_destroy(plan)
    plan, pb, wb = _create(M=128, k_parts=4, flags=q.QGEMM_SPLIT_AUTO, **i8)
    assert wb == 4 * 128 * 4096 * 4                         # auto: partials from 128 rows
    q.qgemm_destroy(plan)
    plan, pb, wb = _create(M=127, k_parts=4, flags=q.QGEMM_SPLIT_AUTO, **i8)
    assert wb == 0                                          # ... atomics below
    q.qgemm_destroy(plan)
    plan, pb, wb = _create(w_dtype="u4", has_zeros=1, N=4096)
    assert pb == 4096 * 4096 // 2 + 32 * 4096 * 4           # (scale, zero) pairs
    q.qgemm_destroy(plan)


def test_null_and_misaligned_arguments_rejected_before_launch():
    plan, pb, wb = _create(k_parts=2, flags=q.QGEMM_DETERMINISTIC)
    try:
        for args in [(0, 16, 16, 16), (16, 0, 16, 16), (16, 16, 0, 16), (16, 16, 16, 0)]:
            with pytest.raises(q.QGemmError) as e:
                q.qgemm_run(plan, args[0], args[1], args[2], args[3], wb, 0)
            assert e.value.status == q.QGEMM_ERR_INVALID_ARG
        with pytest.raises(q.QGemmError) as e:
            q.qgemm_run(plan, 16, 16, 16, 16, wb - 1, 0)       # workspace too small
        assert e.value.status == q.QGEMM_ERR_INVALID_ARG
        with pytest.raises(q.QGemmError) as e:
            q.qgemm_run(plan, 18, 16, 16, 16, wb, 0)           # A not 16-byte aligned
        assert e.value.status == q.QGEMM_ERR_INVALID_ARG
        with pytest.raises(q.QGemmError) as e:
            q.qgemm_pack_weights(plan, 16, 0, 0, 16, 0)        # scales missing
        assert e.value.status == q.QGEMM_ERR_INVALID_ARG
        with pytest.raises(q.QGemmError) as e:
            q.qgemm_pack_weights(plan, 16, 16, 0, 0, 0)        # no output
        assert e.value.status == q.QGEMM_ERR_INVALID_ARG
        # the run-time row count and the bias of qgemm_run_ex (plan M = 1 here)
        for M in (0, 2, -1):
            with pytest.raises(q.QGemmError) as e:
                q.qgemm_run_ex(plan, M, 16, 16, 0, 16, 16, wb, 0)
            assert e.value.status == q.QGEMM_ERR_INVALID_ARG
        with pytest.raises(q.QGemmError) as e:
            q.qgemm_run_ex(plan, 1, 16, 16, 17, 16, 16, wb, 0)  # fp16 bias not 2-byte aligned
        assert e.value.status == q.QGEMM_ERR_INVALID_ARG
        with pytest.raises(q.QGemmError) as e:
            q.qgemm_run_ex(plan, 1, 0, 16, 16, 16, 16, wb, 0)   # no A
        assert e.value.status == q.QGEMM_ERR_INVALID_ARG
    finally:
        q.qgemm_destroy(plan)
    plan, pb, wb = _create(a_dtype="i8", w_dtype="i8", out_dtype="i32", accum_dtype="i32", group_size=0, M=4)
    try:
        with pytest.raises(q.QGemmError) as e:
            q.qgemm_run_ex(plan, 3, 16, 16, 18, 16, 0, 0, 0)    # int32 bias not 4-byte aligned
        assert e.value.status == q.QGEMM_ERR_INVALID_ARG
    finally:
        q.qgemm_destroy(plan)
    assert q.qgemm_plan_path(0) == -1
    q.qgemm_destroy(0)                                         # NULL is a no-op
    # dequantised int8 plans run only with their scales, other plans never with scales
    dq, _, wb = _create(a_dtype="i8", w_dtype="i8", out_dtype="f16", accum_dtype="i32", group_size=0,
                        M=4, k_parts=2)
    i32, _, _ = _create(a_dtype="i8", w_dtype="i8", out_dtype="i32", accum_dtype="i32", group_size=0, M=4)
    try:
        assert wb == 4 * 4096 * 4                              # fp16 output: one int32 accumulator
        for call in [lambda: q.qgemm_run(dq, 16, 16, 16, 16, wb, 0),
                     lambda: q.qgemm_run_ex(dq, 4, 16, 16, 0, 16, 16, wb, 0),
                     lambda: q.qgemm_run_scaled(dq, 4, 16, 16, 0, 16, 0, 16, 16, wb, 0),   # no row scales
                     lambda: q.qgemm_run_scaled(dq, 4, 16, 16, 16, 0, 0, 16, 16, wb, 0),   # no column scales
                     lambda: q.qgemm_run_scaled(dq, 4, 16, 16, 18, 16, 0, 16, 16, wb, 0),  # misaligned
                     lambda: q.qgemm_run_scaled(dq, 5, 16, 16, 16, 16, 0, 16, 16, wb, 0),  # M > plan M
                     lambda: q.qgemm_run_scaled(i32, 4, 16, 16, 16, 16, 0, 16, 0, 0, 0)]:   # int32 plan
            with pytest.raises(q.QGemmError) as e:
                call()
            assert e.value.status == q.QGEMM_ERR_INVALID_ARG
    finally:
        q.qgemm_destroy(dq)
        q.qgemm_destroy(i32)
    for args in [(0, 4, 64, 16, 16), (16, 0, 64, 16, 16), (16, 4, 60, 16, 16), (16, 4, 0, 16, 16),
                 (18, 4, 64, 16, 16), (16, 4, 64, 20, 16), (16, 4, 64, 16, 18), (16, 4, 64, 0, 16),
                 (16, 4, 64, 16, 0)]:
        with pytest.raises(q.QGemmError) as e:
            q.qgemm_quantize_rows(args[0], args[1], args[2], args[3], args[4], 0)
        assert e.value.status == q.QGEMM_ERR_INVALID_ARG, args
    assert q.qgemm_status_string(2) == "unsupported format or shape"


# the pages' benchmark grid: config strings of the BitBLAS issue #252 tables
_FIELDS = ["M", "N", "K", "A_dtype", "W_dtype", "out_dtype", "accum_dtype", "layout", "with_bias",
           "group_size", "with_scaling", "with_zeros", "zeros_mode"]
_DT = {"float16": "f16", "int8": "i8", "int4": "i4", "int2": "i2", "int32": "i32"}


def _parse(line):
    # "1-16384-16384-float16-int4-float16-float16-nt-False--1-True-False-None": the group size
    # -1 shows up as an empty field followed by "1"
    parts = line.split("-")
    if parts[9] == "" and parts[10] == "1":
        parts = parts[:9] + ["-1"] + parts[11:]
    assert len(parts) == 13, line
    return dict(zip(_FIELDS, parts))


def golden_grid():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            rows.append(_parse(line))
    return rows


def plan_args(cfg):
    """Map one of the pages' configs to qgemm_create arguments.

    fp16 accumulation becomes fp32 and int8 output becomes int32 (this library
    returns the int32 accumulator); with_scaling False means group_size 0.
    """
    a, w = _DT[cfg["A_dtype"]], _DT[cfg["W_dtype"]]
    out, acc = ("f16", "f32") if a == "f16" else ("i32", "i32")
    g = int(cfg["group_size"]) if (w in ("i4", "u4") and cfg["with_scaling"] == "True") else 0
    return dict(M=int(cfg["M"]), N=int(cfg["N"]), K=int(cfg["K"]), a_dtype=a, w_dtype=w,
                out_dtype=out, accum_dtype=acc, group_size=g,
                has_zeros=int(cfg["with_zeros"] == "True"), k_parts=1, flags=0)


def test_pages_grid_maps_to_plans():
    grid = golden_grid()
    assert len(grid) == 25
    assert {(c["M"]) for c in grid} == {"1", "32", "128", "512", "16384"}
    for cfg in grid:
        assert cfg["layout"] == "nt" and cfg["with_bias"] == "False"
        args = plan_args(cfg)
        plan, pb, wb = q.qgemm_create(**args)
        want = q.QGEMM_PATH_GEMV if args["M"] <= 8 else q.QGEMM_PATH_MFMA
        assert q.qgemm_plan_path(plan) == want
        q.qgemm_destroy(plan)


def test_noalloc_rejects_before_any_device_call():
    """qgemm_run_noalloc checks its arguments and the scratch it would need before it
    looks up the scratch array or launches anything."""
    assert q.NOALLOC_MAX_SCRATCH == 32 << 20
    big, _, wb = _create(M=4096, N=16384, K=4096, k_parts=2)   # fp32 atomics: 256 MiB of scratch
    dq, _, _ = _create(a_dtype="i8", w_dtype="i8", out_dtype="f16", accum_dtype="i32", group_size=0, M=4)
    try:
        assert wb == 4096 * 16384 * 4 + (4096 + 16384) * 32 * 2 * 2   # and the int4 folding's planes
        with pytest.raises(q.QGemmError) as e:
            q.qgemm_run_noalloc(big, 4096, 16, 16, 0, 16, 0)
        assert e.value.status == q.QGEMM_ERR_UNSUPPORTED
        for M in (0, 4097):
            with pytest.raises(q.QGemmError) as e:
                q.qgemm_run_noalloc(big, M, 16, 16, 0, 16, 0)
            assert e.value.status == q.QGEMM_ERR_INVALID_ARG
        with pytest.raises(q.QGemmError) as e:
            q.qgemm_run_noalloc(dq, 4, 16, 16, 0, 16, 0)          # needs its scales
        assert e.value.status == q.QGEMM_ERR_INVALID_ARG
        with pytest.raises(q.QGemmError) as e:
            q.qgemm_run_noalloc(0, 1, 16, 16, 0, 16, 0)
        assert e.value.status == q.QGEMM_ERR_INVALID_ARG
    finally:
        q.qgemm_destroy(big)
        q.qgemm_destroy(dq)


@pytest.mark.parametrize("kw,Kpad", [
    (dict(K=4104, group_size=0), 4224),                      # int4: whole words, not whole 128-blocks
    (dict(K=4104, group_size=-1, w_dtype="u4", has_zeros=1), 4224),
    (dict(K=4128, group_size=96), 4224),                     # groups of 96: 44 scale rows stored
    (dict(K=8, group_size=0), 128),
    (dict(a_dtype="i8", w_dtype="i2", out_dtype="i32", accum_dtype="i32", group_size=0, K=4112), 4352),
    # int8 / fp16: granules of two blocks (the matrix-core tiles stage 128-byte activation rows)
    (dict(a_dtype="i8", w_dtype="i8", out_dtype="i32", accum_dtype="i32", group_size=0, K=4100), 4224),
    (dict(a_dtype="i8", w_dtype="i8", out_dtype="i32", accum_dtype="i32", group_size=0, K=4160), 4224),
    (dict(w_dtype="f16", group_size=0, K=4099), 4160),
    (dict(w_dtype="f16", group_size=0, K=4128), 4160),
])
def test_k_granularity_pads_to_whole_blocks(kw, Kpad):
    """K needs only whole canonical words and whole groups: the blob is padded to whole
    blocks and the workspace gains the zero-padded activation rows."""
    M, N = 3, 100
    plan, pb, wb = _create(M=M, N=N, **kw)
    try:
        w = kw.get("w_dtype", "i4")
        bits = {"i4": 4, "u4": 4, "i2": 2, "i8": 8, "f16": 16}[w]
        g = kw["group_size"]
        rows = 0 if g == 0 else 1 if g < 0 else -(-Kpad // g)
        per = 4 if kw.get("has_zeros") else 2
        assert pb == 256 * Kpad * bits // 8 + rows * 256 * per
        esz = 1 if kw.get("a_dtype") == "i8" else 2
        assert wb == M * Kpad * esz
    finally:
        q.qgemm_destroy(plan)
    # with split-K the padded rows follow the accumulator, 256-byte aligned
    if Kpad == 128:
        return                                                 # one block: no split
    plan, pb, wb = _create(M=M, N=N, k_parts=2, **kw)
    try:
        acc = M * N * 4 if kw.get("a_dtype") != "i8" else 0
        assert wb == -(-acc // 256) * 256 + M * Kpad * (1 if kw.get("a_dtype") == "i8" else 2)
    finally:
        q.qgemm_destroy(plan)


def test_library_splits_long_int4_tiles_itself():
    """k_parts 1 with int4 / uint4 and K >= 8192: at 33..256 rows and N >= 4096 2, 4 or 8
    parts (enough for 256 workgroups of 128 x 128 tiles), at 9..32 rows and N <= 4096 two
    or four, summed in order, so the plan reports a workspace of that many fp32
    partials; elsewhere none."""
    for kw, wb_expect in [
        (dict(M=128, N=16384, K=16384), 2 * 128 * 16384 * 4),
        (dict(M=256, N=16384, K=8192), 2 * 256 * 16384 * 4),   # 256 tiles: still two
        (dict(M=128, N=8192, K=8192), 4 * 128 * 8192 * 4),     # 64 tiles: four
        (dict(M=128, N=4096, K=11008), 8 * 128 * 4096 * 4),    # 32 tiles: eight
        (dict(M=40, N=4096, K=8192), 8 * 40 * 4096 * 4),
        (dict(M=256, N=4096, K=11008, group_size=-1, w_dtype="u4", has_zeros=1), 4 * 256 * 4096 * 4),
        # 9..32 rows at N <= 4096 (the matrix-core GEMV): four parts from 17 rows, two below
        (dict(M=32, N=4096, K=11008), 4 * 32 * 4096 * 4),
        (dict(M=20, N=2048, K=8192, group_size=-1), 4 * 20 * 2048 * 4),
        (dict(M=16, N=4096, K=11008), 2 * 16 * 4096 * 4),
        (dict(M=9, N=4096, K=8192, w_dtype="u4", has_zeros=1), 2 * 9 * 4096 * 4),
        (dict(M=8, N=4096, K=11008), 0),                       # GEMV rows
        (dict(M=32, N=4096, K=4096), 0),                       # short K
        (dict(M=32, N=8192, K=11008), 0),                      # wide
        (dict(M=32, N=4096, K=11008, group_size=64), 0),       # per-piece groups
        (dict(M=32, N=16384, K=16384), 0),                     # skinny: matrix-core GEMV
        (dict(M=512, N=16384, K=16384), 0),                    # enough tiles
        (dict(M=128, N=16384, K=4096), 0),                     # short K
        (dict(M=128, N=2048, K=16384), 0),                     # narrow
        (dict(M=128, N=16384, K=16384, w_dtype="f16", group_size=0), 0),
    ]:
        plan, _, wb = _create(**kw)
        q.qgemm_destroy(plan)
        assert wb == wb_expect, kw
