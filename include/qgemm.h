/*
 * qgemm — weight-quantized mixed-precision matrix product for AMD MI355X (gfx950).
 *
 *     C[M,N] = A[M,K] . dequant(Wq[K,N])
 *
 * Problem statement: BitBLAS issue #252 ("Default Backend Should be changed
 * into tilelang ..."), reproduction script — a MatmulConfig is M, N, K,
 * A_dtype, W_dtype, out_dtype, accum_dtype, layout "nt", with_bias,
 * group_size, with_scaling, with_zeros, zeros_mode.  Parallel-k (k-parts)
 * follows hidet issue #364 ("[Graph][Quantization] Multi-stage software
 * pipelining and update parallel k rule"): K is split into parts whose
 * partial products are reduced with atomics.  Affine dequantisation
 * w = (q - z) * s follows torchao issue #2752 (AffineQuantizedTensor).
 * int8 products accumulate into and return int32 (Triton PR #3595).
 *
 * Supported formats (a_dtype, w_dtype, out_dtype, accum_dtype):
 *   W4A16 : (F16, I4 | U4, F16, F32)   per-group fp16 scales, optional zero points (U4)
 *   dense : (F16, F16,     F16, F32)
 *   W8A8  : (I8,  I8,      I32, I32)   exact
 *   W2A8  : (I8,  I2,      I32, I32)   exact
 *   W8A8 / W2A8 dequantised: (I8, I8 | I2, F16, I32), run with per-row and
 *           per-column fp32 scales through qgemm_run_scaled
 * Any other tuple returns QGEMM_ERR_UNSUPPORTED (fp16 accumulation and int8
 * output are not provided: the int8 narrowing rule is unspecified).
 *
 * Canonical input layout ("nt"; all row-major, little-endian):
 *   A        [M, K]      fp16 or int8
 *   W  I4/U4 uint32 [N, K/8]   value (k, n) in bits 4*(k%8) of word n*(K/8) + k/8
 *      I2    uint32 [N, K/16]  value (k, n) in bits 2*(k%16) of word n*(K/16) + k/16
 *      I8    int8   [N, K]     F16 fp16 [N, K]
 *      signed values are two's complement of the field width; U4 is plain binary.
 *   scales   fp16 [N, G], zeros fp16 [N, G]; G = K/g for g > 0, G = 1 for g = -1.
 *   C        [M, N]      fp16 or int32
 * Dequantised weight: w = q (g == 0), w = q*s (no zeros), w = (q - z)*s (zeros),
 * with s, z taken at column n and group k / g.
 *
 * Packed weights: qgemm_pack_weights writes an opaque blob of packed_bytes
 * (weights pre-shuffled into the MFMA operand order of gfx950, 1 KiB per
 * 16-column x KB-row block, plus relaid scales and zeros).  The blob depends
 * only on (N, K, w_dtype, group_size, has_zeros): plans that differ only in M,
 * k_parts or flags can share one packed weight.
 *
 * Ownership and streams: every device buffer is allocated and owned by the
 * caller; the library allocates no device memory.  A plan owns only host
 * memory and is immutable after creation, so it may be used from several
 * threads at once.  `stream` is a hipStream_t passed as void* (NULL = the
 * null stream); every device call is asynchronous on it.  Concurrent
 * qgemm_run calls on one plan need distinct workspaces and outputs.
 *
 * Errors: every call returns a status; nothing is thrown across the ABI.
 * Argument errors are found before any device call (qgemm_create makes no
 * HIP call at all).  A failed launch returns QGEMM_ERR_DEVICE.
 */
#ifndef QGEMM_H
#define QGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qgemm_plan qgemm_plan;

typedef enum {
  QGEMM_OK = 0,
  QGEMM_ERR_INVALID_ARG = 1, /* NULL pointer, non-positive size, bad flag, too-small buffer */
  QGEMM_ERR_UNSUPPORTED = 2, /* legal request outside the supported formats or shapes */
  QGEMM_ERR_NO_MEMORY = 3,   /* host allocation of the plan failed */
  QGEMM_ERR_DEVICE = 4       /* a kernel launch failed */
} qgemm_status;

typedef enum {
  QGEMM_F16 = 1,
  QGEMM_F32 = 2,
  QGEMM_I32 = 3,
  QGEMM_I8 = 4,
  QGEMM_I4 = 5, /* signed int4, [-8, 7] */
  QGEMM_U4 = 6, /* unsigned int4, [0, 15] */
  QGEMM_I2 = 7  /* signed int2, [-2, 1] */
} qgemm_dtype;

/* flags for qgemm_create (k_parts > 1 only; without flags the parts are reduced
   with global atomics, the parallel-k reduction of hidet issue #364) */
#define QGEMM_DETERMINISTIC 1u /* fixed-order two-pass reduction: bitwise reproducible */
#define QGEMM_SPLIT_AUTO 2u    /* the reduction that measured faster for the plan's shape:
                                  two-pass for fp16 outputs and for int32 outputs from 128
                                  rows while the partials stay within 256 MiB, else atomics;
                                  QGEMM_DETERMINISTIC takes precedence */

/* execution path chosen by a plan (qgemm_plan_path) */
#define QGEMM_PATH_GEMV 1 /* M <= 8: skinny kernels streaming the weights once (dot products at
                             one row; matrix cores from 2 rows, 3 for int4) */
#define QGEMM_PATH_MFMA 2 /* M > 8: matrix cores (skinny kernels up to 32 rows, then
                             LDS-staged tiles) */

/*
 * Create a plan: the problem statement of BitBLAS issue #252's Matmul
 * configuration (M, N, K, A_dtype, W_dtype, out_dtype, accum_dtype, group_size,
 * with_scaling as group_size != 0, with_zeros) plus hidet issue #364's k-parts.
 * No device call.
 *   M, N, K       problem sizes, each >= 1.  K must be a multiple of the values
 *                 per canonical word: 8 (I4/U4), 16 (I2), 1 (I8/F16), and of
 *                 group_size when that is > 0, else QGEMM_ERR_UNSUPPORTED.  The
 *                 kernels work on whole granules of 128 (I4/U4, I8), 256 (I2) or
 *                 64 (F16) positions: when K is not a multiple of the granule,
 *                 the blob is zero-padded and every run first copies A into the
 *                 workspace with its rows zero-padded (the workspace then also
 *                 holds M * roundup(K, granule) activation elements).  The
 *                 activations, M * roundup(K, granule) elements, must stay below
 *                 4 GiB, else QGEMM_ERR_UNSUPPORTED.
 *   group_size    0 = no scaling (with_scaling False), -1 = one group per output
 *                 column over all of K, g > 0 = groups of g along K.  Scaled
 *                 formats are I4/U4 only; g > 0 must divide K and be a multiple
 *                 of 32.  Other weight formats require 0.
 *   has_zeros     0 or 1; 1 only with w_dtype U4 and group_size != 0.
 *                 Scales of U4 weights: |s| < 64, and with zero points
 *                 |s| * (1024 + z) < 65504 with 0 <= z < 1024; of I4 weights
 *                 with g > 0: |s| < 63; for rows that take the 256 x 256 tiles
 *                 (large M): those tiles upcast and scale a weight with one
 *                 fp16 fma whose addend, -1024 s, -fp16(1024 + z) s or -1032 s,
 *                 must be finite (BitBLAS issue #252, the int4 / uint4 op
 *                 configs with scaling and zero points).
 *   k_parts       >= 1: number of contiguous, group-aligned K ranges computed by
 *                 separate workgroups and reduced with fp32/int32 global atomics
 *                 (default) or by ordered partials and one summing pass
 *                 (QGEMM_DETERMINISTIC; see qgemm_run).  At most K / unit, where
 *                 unit = group_size when it is a multiple of 128 (and larger),
 *                 else the granule (K rounded up to it).
 *   flags         0, or QGEMM_DETERMINISTIC and / or QGEMM_SPLIT_AUTO.
 *   packed_bytes  out: size of the packed blob for qgemm_pack_weights/qgemm_run.
 *   workspace_bytes out: size of the device workspace qgemm_run needs (0 if none).
 *                 A plan of k_parts 1 may need one too: for I4 / U4 weights and
 *                 K >= 8192 the library splits K itself and sums the partial
 *                 products in a fixed order, so results stay bitwise reproducible;
 *                 the workspace holds those parts' fp32 partials.  With 33 to 256
 *                 rows and N >= 4096: 2, 4 or 8 parts (as many as one wave of 256
 *                 workgroups of 128 x 128 output tiles takes), for runs of more than
 *                 32 rows.  With 9 to 32 rows, N <= 4096 and groups of whole
 *                 superblocks (or none): 4 parts for runs of 17 rows or more when the
 *                 plan has more than 16 rows, else 2 parts for runs of 9 or more.
 *                 U4 with zero points and groups that are whole multiples of 128
 *                 (or one group over K), and I4 with such groups (its offset 8
 *                 as the zero point): runs that take the 256 x 256 tiles apply
 *                 the zero points after their K loop as sum_g R[m, g] P[g, n],
 *                 with R the row sums of A over each group and P from the scales
 *                 and zeros (each held as two bf16 planes of roundup(G, 32)
 *                 values per row of A and per padded column); the workspace then
 *                 ends with those planes, sized for the largest run of the plan
 *                 that takes those tiles.
 */
qgemm_status qgemm_create(qgemm_plan** out, int64_t M, int64_t N, int64_t K,
                          qgemm_dtype a_dtype, qgemm_dtype w_dtype, qgemm_dtype out_dtype,
                          qgemm_dtype accum_dtype, int32_t group_size, int32_t has_zeros,
                          int32_t k_parts, uint32_t flags, size_t* packed_bytes,
                          size_t* workspace_bytes);

/*
 * Pack canonical weights (device memory, layout above) into the plan's blob: the
 * backend-specific pre-shuffled weight of torchao issue #2752's "dtype +
 * packing_format" tensors, built from BitBLAS issue #252's "nt" weight layout.
 *   w       device, canonical weights.
 *   scales  device, fp16 [N, G]; required iff group_size != 0, else ignored.
 *   zeros   device, fp16 [N, G]; required iff has_zeros, else ignored.
 *   packed  device, >= packed_bytes, 16-byte aligned; fully overwritten.
 * Asynchronous on `stream`; run once per weight, outside the hot loop.
 */
qgemm_status qgemm_pack_weights(const qgemm_plan* plan, const void* w, const void* scales,
                                const void* zeros, void* packed, void* stream);

/*
 * C = A . dequant(W) on `stream` (the quantized matmul of hidet issue #364 and
 * BitBLAS issue #252; int8 x int8 / int2 products accumulate and return int32,
 * Triton PR #3595).
 *   A          device, [M, K] fp16 or int8, 16-byte aligned (rows are K elements
 *              apart, whatever their alignment).
 *   packed     device, the blob written by qgemm_pack_weights.
 *   C          device, [M, N] fp16 or int32; fully overwritten.
 *   workspace  device, >= workspace_bytes (may be NULL when that is 0),
 *              16-byte aligned; scratch for split-K and padded activations, its
 *              contents on entry are ignored.
 * Split-K (k_parts > 1) reduces the parts with global atomics unless a flag says
 * otherwise: fp16 outputs add fp32 partials into the zero-filled workspace
 * (M * N * 4 bytes), which one more pass rounds into C; int32 outputs add
 * straight into C (no workspace).  fp32 atomics add in the order the parts
 * finish, so fp16 results may differ in the last bits between runs (each within
 * the accuracy of the fp32 sum); int32 results are exact and identical.  With
 * QGEMM_DETERMINISTIC (and with QGEMM_SPLIT_AUTO where it picks them) the parts
 * write ordered partials (k_parts * M * N * 4 bytes) that one pass sums in part
 * order: bitwise reproducible.
 */
qgemm_status qgemm_run(const qgemm_plan* plan, const void* A, const void* packed, void* C,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * C = A . dequant(W) (+ bias) for a run-time number of rows, on `stream`: the
 * serving form of qgemm_run (decode batches vary from call to call), and the
 * bias epilogue that BitBLAS's Matmul configuration names with_bias (its
 * benchmark configurations leave it off; BitBLAS issue #252, reproduction script).
 *   M          rows this call computes, 1 <= M <= the plan's M, else
 *              QGEMM_ERR_INVALID_ARG.  The kernels are chosen for this M (as
 *              qgemm_create would for a plan of M rows); the plan's workspace
 *              size covers every M.
 *   A          device, [M, K], as in qgemm_run.
 *   packed     device, the plan's blob.
 *   bias       device, [N] of the output type (fp16 or int32), or NULL for none:
 *              C[m, n] = sum + bias[n].  fp16 outputs add it in fp32 before the
 *              one rounding to fp16; int32 outputs add it exactly.  Naturally
 *              aligned (2 / 4 bytes), else QGEMM_ERR_INVALID_ARG.
 *   C          device, [M, N]; fully overwritten.
 *   workspace, workspace_bytes, stream: as in qgemm_run.
 * qgemm_run(plan, A, packed, C, ...) is qgemm_run_ex with the plan's M and no bias.
 */
qgemm_status qgemm_run_ex(const qgemm_plan* plan, int64_t M, const void* A, const void* packed,
                          const void* bias, void* C, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * qgemm_run_ex without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Split-K runs in a fixed scratch array inside the
 * library, one per GPU, of QGEMM_NOALLOC_MAX_SCRATCH bytes, which each GPU the
 * library runs on holds until the process ends; this call itself allocates
 * nothing.  It needs the workspace that qgemm_run_ex would for run-time M (the
 * atomic accumulator or the two-pass partials, plus the zero-padded activation
 * rows when K is not a whole number of blocks, plus the zero-point planes of U4 /
 * I4 plans on the 256 x 256 tiles; none for an unsplit plan of
 * whole blocks otherwise); more than the maximum returns QGEMM_ERR_UNSUPPORTED
 * before any device call.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap in
 * time on one GPU (other streams, other threads) race and must be serialised by
 * the caller.  The stream must belong to the current device.  Plans with
 * dequantised int8 output (qgemm_run_scaled) are rejected (QGEMM_ERR_INVALID_ARG).
 *   M, A, packed, bias, C, stream: as in qgemm_run_ex.
 * The first call that needs scratch on a device looks up its address
 * (QGEMM_ERR_DEVICE if that fails).
 */
#define QGEMM_NOALLOC_MAX_SCRATCH ((size_t)32 << 20)
qgemm_status qgemm_run_noalloc(const qgemm_plan* plan, int64_t M, const void* A, const void* packed,
                               const void* bias, void* C, void* stream);

/*
 * int8 activations with fp16 output (plans created with the tuple
 * (I8, I8 | I2, F16, I32)): C[m, n] = fp16(acc[m, n] * row_scales[m] *
 * col_scales[n] (+ bias[n])), the dequantising epilogue of the int8
 * dynamic-activation configurations (torchao issue #2752), computed in fp32
 * from the exact int32 accumulator with one rounding.  Such plans run only
 * through this call (qgemm_run / qgemm_run_ex return QGEMM_ERR_INVALID_ARG).
 *   M          rows, 1 <= M <= the plan's M.
 *   A          device, int8 [M, K] (e.g. from qgemm_quantize_rows).
 *   row_scales device, fp32 [M] (per-token activation scales).
 *   col_scales device, fp32 [N] (per-channel weight scales).
 *   bias       device, fp16 [N], or NULL.
 *   C          device, fp16 [M, N]; fully overwritten.
 *   workspace, workspace_bytes, stream: as in qgemm_run.
 */
qgemm_status qgemm_run_scaled(const qgemm_plan* plan, int64_t M, const void* A, const void* packed,
                              const float* row_scales, const float* col_scales, const void* bias,
                              void* C, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dynamic per-token int8 quantisation of fp16 activations (the activation step
 * of torchao issue #2752's Int8DynamicActivation* configurations), symmetric
 * with one scale per row:
 *   scales[m] = max_k |A[m, k]| / 127                  (fp32, round to nearest)
 *   Q[m, k]   = clamp(rint(A[m, k] / scales[m]), -127, 127)
 * with the division in fp32, correctly rounded, rint to nearest even; an
 * all-zero row gets scale 0 and codes 0.
 *   A       device, fp16 [M, K], 16-byte aligned.
 *   M, K    M >= 1; K >= 8 and a multiple of 8.
 *   Q       device, int8 [M, K], 8-byte aligned; fully overwritten.
 *   scales  device, fp32 [M], 4-byte aligned; fully overwritten.
 * Asynchronous on `stream`.  QGEMM_ERR_INVALID_ARG on a bad argument (checked
 * before any launch), QGEMM_ERR_DEVICE if the launch fails.
 */
qgemm_status qgemm_quantize_rows(const void* A, int64_t M, int64_t K, void* Q, float* scales,
                                 void* stream);

/* Release a plan; NULL is a no-op.  Device buffers are the caller's. */
void qgemm_destroy(qgemm_plan* plan);

/* Path the plan chose (QGEMM_PATH_GEMV or QGEMM_PATH_MFMA), or -1 for NULL. */
int32_t qgemm_plan_path(const qgemm_plan* plan);

/* Short static description of a status code. */
const char* qgemm_status_string(qgemm_status status);

#ifdef __cplusplus
}
#endif

#endif /* QGEMM_H */
