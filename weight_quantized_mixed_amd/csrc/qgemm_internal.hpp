// Internal definitions shared by the host ABI and the kernels of libqgemm.
//
// Packed blob layout (written by the pack kernel, read by every compute kernel)
// ---------------------------------------------------------------------------
// Columns are padded to Npad = roundup(N, 256).  The weight region is a grid of
// 1 KiB "superblocks", each 16 columns x KB reduction positions:
//     superblock (nb, kb) at byte ((kb * (Npad/16)) + nb) * 1024
// KB = 128 (int4), 256 (int2), 64 (int8), 32 (fp16): 16 bytes per column per
// quarter of the block.  Inside a superblock, the 16-byte "piece" of column
// nn = n % 16 and quarter kq sits at byte (kq*16 + nn) * 16, so one wave-wide
// 16-byte load (lane l -> piece l) fetches the whole block in the lane order of
// a gfx950 16x16 MFMA B operand (lane l: column l%16, K slice l/16).  A piece
// covers the KB/4 consecutive positions kb*KB + kq*KB/4 + [0, KB/4):
//   int4  4 words x 8 values; word t holds positions 8t..8t+7 with nibble
//         slots (0..7) <- positions (0,2,4,6,1,3,5,7), stored offset-binary
//         (q + 8 for signed, q for unsigned), so (w >> 4j) & 0x000F000F,
//         or-ed with 0x6400 per half, is the fp16 pair (1024 + s[2j], 1024 + s[2j+1]).
//   int2  4 words x 16 values; word t holds positions 16t..16t+15, value e in
//         byte e%4 at bit 2*(e/4), so (w >> 2j) & 0x03030303 gives the four
//         consecutive positions 4j..4j+3.  Classes j = 0..2 are stored
//         offset-binary (q + 2); class 3 (bits 6..7 of each byte) is stored two's
//         complement, so w & 0xC0C0C0C0 reads as the signed bytes 64q.
//   int8  16 bytes = 16 consecutive positions.
//   fp16  8 halves = 8 consecutive positions.
// After the weights (256-byte aligned) come the scales as [G][Npad] fp16, or
// (scale, zero) half pairs as [G][Npad] when zero points are present.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemm.h"

namespace qg {

enum Fmt : int { FMT_I4 = 0, FMT_U4 = 1, FMT_F16 = 2, FMT_I8 = 3, FMT_I2 = 4 };

// output modes of a compute kernel
enum OutMode : int {
  OUT_STORE = 0,    // write C directly (k_parts == 1)
  OUT_ATOMIC = 1,   // atomic add into fp32 workspace (fp16 out) or into C (int32 out)
  OUT_PARTIAL = 2   // write the part's partial to workspace[part][M][N] (two-pass)
};

// scale modes
enum ScaleMode : int {
  SC_NONE = 0,   // group_size == 0
  SC_BLOCK = 1,  // one group per superblock (g >= KB or g == -1)
  SC_PIECE = 2   // one group per 32-position piece (g in {32, 64} for int4)
};

constexpr int kb_of(int fmt) {
  return fmt == FMT_I2 ? 256 : fmt == FMT_I8 ? 64 : fmt == FMT_F16 ? 32 : 128;
}

// fp16 / int8 direct-load MFMA stages of two superblocks (128-byte activation rows;
// 1) or one (64-byte rows; 0).  A direct load of 16 rows x 64 bytes moves half as
// many bytes per clock as one of 8 rows x 128 bytes (a probe of global_load_lds_dwordx4
// from L2 at a 32 KiB row stride: 70 against 143 bytes per ns per CU).
#ifndef QG_DL_WIDE
#define QG_DL_WIDE 1
#endif
// K granule of a format: K is padded to it and k-parts split at it (two superblocks
// for fp16 / int8 with two-superblock stages, else one)
constexpr int kgrain_of(int fmt) {
  return (QG_DL_WIDE && (fmt == FMT_F16 || fmt == FMT_I8)) ? 2 * kb_of(fmt) : kb_of(fmt);
}

// K is padded to whole K granules (Kpad = roundup(K, kgrain_of)): the blob holds zero
// codes at positions K .. Kpad - 1 and, where scale groups are smaller than a
// superblock, zero scales for the groups past K (G_store rows in all), and runs
// read activations zero-padded to Kpad, so those positions add exactly nothing.
struct Layout {
  int fmt;
  int64_t N, K, Kpad, Npad, NB, nkb;
  int32_t group_size;  // as given: 0, -1 or g > 0
  int64_t G;           // number of scale groups of the input table (0 without scaling)
  int64_t G_store;     // scale rows in the blob (G, or more to cover Kpad)
  bool zeros;
  size_t w_bytes, s_offset, s_bytes, total;
};

// canonical weight values per 32-bit word (int8 / fp16 rows are plain arrays)
constexpr int pack_factor(int fmt) { return fmt == FMT_I2 ? 16 : (fmt == FMT_I4 || fmt == FMT_U4) ? 8 : 1; }

// Arguments of every compute kernel (GEMV and MFMA), passed by value.
struct RunArgs {
  const void* A;        // [M, K]
  const uint4* W;       // packed superblocks
  const void* S;        // scales (half) or (scale, zero) half2 pairs, [G][Npad]
  void* C;              // [M, N] fp16 or int32
  void* ws;             // fp32/int32 workspace
  int32_t M, N, K;
  int32_t Npad, NB, nkb;
  int32_t group_size;   // 0, -1 or g
  int32_t smode;        // ScaleMode
  int32_t zeros;        // 0/1
  int32_t out_mode;     // OutMode
  int32_t k_parts;
  int32_t unit_kb;      // superblocks per split unit
  int32_t n_units;      // nkb / unit_kb
  int32_t waves;        // GEMV: waves per workgroup (K split inside the workgroup)
  int32_t sb_per_group; // superblocks per scale group (nkb when one group spans K)
  int32_t g_shift;      // group of position p = p >> g_shift, or -1: p / group_size
  int32_t gemv_cb;      // matrix-core GEMV: 16-column blocks per workgroup (1, 2 or 4)
  const void* bias;     // [N] of the output type, or null
  // int8 activations with fp16 output: C = fp16(acc * row_scale[m] * col_scale[n]
  // (+ bias)); null for int32 output
  const float* row_scale;
  const float* col_scale;
  // int4 / uint4 with one scale group over K and no zero points on the matrix-core
  // tiles: the per-column scale applied to the fp32 sum in the epilogue (the tiles
  // then upcast without it); null otherwise
  const _Float16* epi_scale;
  // uint4 with zero points (and signed int4, its offset 8 as the zero point) on the
  // 256 x 256 tiles of four waves: the zero points are folded out of the K loop
  // (C = sum_k A q s - sum_g R[m, g] s[g, n] z[g, n], R the row sums of A over scale
  // group g).  zr holds R of each row, zp the per-column term P of each column (Npad of
  // them), each as two bf16 planes of zr_gp values, [hi | lo] with hi = bf16(x),
  // lo = bf16(x - hi), groups zr_G .. zr_gp - 1 zero; both null without the folding
  const uint16_t* zr;
  const uint16_t* zp;
  int32_t zr_gp;  // groups per plane: zr_G rounded up to 32
  int32_t zr_G;   // scale groups over K
};

// bias of output column col (0 without bias): fp16 outputs add it in fp32 before
// their one rounding, int32 outputs exactly
__device__ __forceinline__ float bias_f(const RunArgs& a, int col) {
  return a.bias ? (float)static_cast<const _Float16*>(a.bias)[col] : 0.f;
}
__device__ __forceinline__ int bias_i(const RunArgs& a, int col) {
  return a.bias ? static_cast<const int*>(a.bias)[col] : 0;
}
// fp16 output of an int32 accumulator: the per-row (activation) and per-column
// (weight) scales and the bias applied in fp32, one rounding to fp16
__device__ __forceinline__ _Float16 dq_out(const RunArgs& a, int row, int col, int acc) {
  return (_Float16)((float)acc * a.row_scale[row] * a.col_scale[col] + bias_f(a, col));
}
// where integer split-K atomics add up: C itself, or the workspace when the
// output is dequantised afterwards
__device__ __forceinline__ int* int_atomic_target(const RunArgs& a) {
  return static_cast<int*>(a.row_scale ? a.ws : a.C);
}

// Split units [u0, u1) of K part `part` (contiguous, as even as integers allow).
// Without a split the 64-bit division, which costs a measurable part of a
// microsecond-scale kernel's start, is skipped.
__device__ __forceinline__ void part_units(const RunArgs& a, int part, int& u0, int& u1) {
  u0 = 0;
  u1 = a.n_units;
  if (a.k_parts != 1) {
    u0 = (int)((int64_t)part * a.n_units / a.k_parts);
    u1 = (int)((int64_t)(part + 1) * a.n_units / a.k_parts);
  }
}

// the 256 x 256 tiles of four 128 x 128 waves (mfma_big.hip) for the formats that
// take them (0: the eight-wave tile of mfma_dl.hip for every format)
#ifndef QG_BIG4
#define QG_BIG4 1
#endif

// kernel launchers (return hipSuccess or the launch error)
hipError_t launch_pack(const Layout& L, const void* w, const void* s, const void* z, void* packed,
                       hipStream_t st);
hipError_t launch_gemv(int fmt, const RunArgs& a, hipStream_t st);
// M = 1 with 16-column workgroups (gemv16.hip), for matrices with few 64-column blocks
hipError_t launch_gemv16(int fmt, const RunArgs& a, hipStream_t st);
// int8 / int2 skinny-M on the matrix cores, B operands straight from the blob (gemv_mfma.hip)
hipError_t launch_gemv_mfma(int fmt, const RunArgs& a, hipStream_t st);
// int4 / uint4 skinny-M (M <= 32) on the matrix cores, bias-folded B operands (gemv_mfma4.hip)
hipError_t launch_gemv_mfma4(int fmt, const RunArgs& a, hipStream_t st);
hipError_t launch_mfma(int fmt, int tile, const RunArgs& a, hipStream_t st);
// direct-load ring kernel (mfma_dl.hip): the tile for a problem, or -1 when the
// problem needs the LDS-staged kernel (int4 with per-piece scale groups)
enum DlTile : int {
  DL_32x64 = 0, DL_32x128, DL_32x256, DL_64x128, DL_64x256, DL_128x256, DL_256x256, DL_128x128, DL_NUM
};
void dl_tile_dims(int tile, int* bm, int* bn);
int choose_dl_tile(int fmt, int64_t M, int64_t N, int k_parts, int smode);
hipError_t launch_mfma_dl(int fmt, int tile, const RunArgs& a, hipStream_t st);
// 256 x 256 tiles of four 128 x 128 waves (mfma_big.hip) for the formats that
// big_tile_takes; same arguments and stage layout as launch_mfma_dl's 256 x 256 tile
bool big_tile_takes(int fmt, const RunArgs& a);
hipError_t launch_mfma_big(int fmt, const RunArgs& a, hipStream_t st);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st);
// zr = the bf16 planes [R_hi | R_lo] of the group row sums of a.A (rows of a.K fp16
// values, scale groups of a.group_size positions, or one group when it is negative)
// for the zero-point folding of the 256 x 256 tiles; a.K / 32 <= ROWSUM_MAX_UNITS
constexpr int ROWSUM_MAX_UNITS = 8192;
hipError_t launch_group_rowsum(const RunArgs& a, uint16_t* zr, hipStream_t st);
// zp = the bf16 planes [P_hi | P_lo] of the per-column term of the folding for each of
// the Npad columns, from the (scale, zero) pairs a.S ([zr_G][Npad]), or for signed int4
// (a.zeros 0) from its fp16 scales with the offset 8 as the zero point
hipError_t launch_zero_planes(const RunArgs& a, uint16_t* zp, hipStream_t st);
// dst[m, k] = k < K ? A[m, k] : 0 for rows of Kpad elements of esz bytes (Kpad * esz a
// multiple of 16, dst 16-byte aligned; A any alignment of its element size)
hipError_t launch_pad_rows(const void* A, void* dst, int64_t M, int64_t K, int64_t Kpad, int esz,
                           hipStream_t st);
// C[m, n] = bias[n] (int32) for the integer atomics to add into
hipError_t launch_fill_bias(const RunArgs& a, hipStream_t st);
// per-row symmetric int8 quantisation of fp16 activations (quant.hip)
hipError_t launch_quantize_rows(const void* A, int64_t M, int64_t K, void* Q, float* scales, hipStream_t st);
// sums the per-part partials (or converts the atomic accumulator) into C;
// acc_fp: fp32 accumulator (fp16 activations), else int32
hipError_t launch_finalize(const RunArgs& a, int acc_fp, hipStream_t st);

// GEMV tuning: most waves per workgroup (they split the workgroup's K range)
// and superblocks per register stage
#ifndef QG_GEMV_MAX_WAVES
#define QG_GEMV_MAX_WAVES 8
#endif
#ifndef QG_GEMV_UNR
#define QG_GEMV_UNR 1
#endif
#ifndef QG_GEMV_UNR_I2
#define QG_GEMV_UNR_I2 1
#endif
constexpr int GEMV_MAX_WAVES = QG_GEMV_MAX_WAVES;

// tiles of the LDS-staged MFMA kernel (mfma.hip), used where the direct-load kernel
// is not: TILE_BIG is 256 x 256 for fp16 / int8 and 256 x 128 for int4 / int2
enum Tile : int { TILE_32x64 = 0, TILE_64x64 = 1, TILE_128x128 = 2, TILE_BIG = 3 };
void tile_dims(int fmt, int tile, int* bm, int* bn);

}  // namespace qg
