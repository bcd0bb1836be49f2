// Host side of the C ABI: argument validation, the packed-blob layout, path and
// tile selection, and the launch sequence of one qgemm_run.
//
// The arguments follow the problem statement of BitBLAS issue #252
// (reproduction script: M, N, K, A_dtype, W_dtype, out_dtype, accum_dtype,
// group_size, with_scaling, with_zeros) plus hidet issue #364's k-parts.
#include <mutex>
#include <new>

#include "qgemm_internal.hpp"

using namespace qg;

// the kernels that compute a given number of rows
struct qg_choice {
  int path;          // QGEMM_PATH_GEMV or QGEMM_PATH_MFMA
  int dl_tile;       // direct-load MFMA tile, or -1
  int tile;          // LDS-staged MFMA tile (used when dl_tile < 0)
  int gemv_waves;    // GEMV waves per workgroup
  int gemv_cb;       // matrix-core GEMV: 16-column blocks per workgroup
  bool gemv_narrow;  // M = 1 with fewer than 128 blocks of 64 columns: 16-column workgroups
  bool gemv_mfma;    // int8 / int2 GEMV on the matrix cores
  bool gemv_mfma4;   // int4 / uint4 GEMV on the matrix cores (also for 8 < M <= 32)
};

struct qgemm_plan {
  int64_t M, N, K;
  qgemm_dtype a_dtype, w_dtype, out_dtype, accum_dtype;
  int32_t group_size, has_zeros, k_parts;
  uint32_t flags;
  Layout L;
  qg_choice ch;      // kernels for M rows (calls with fewer rows choose again)
  int32_t unit_kb, n_units;
  bool two_pass;     // split-K reduced by partials + one ordered pass (else atomics)
  int32_t auto_parts;  // k_parts 1: parts the library splits K into on its own (0: none) ...
  int32_t auto_min_m;  // ... for runs of at least this many rows
  size_t ws_bytes;
};

namespace {

int fmt_of(qgemm_dtype w) {
  switch (w) {
    case QGEMM_I4: return FMT_I4;
    case QGEMM_U4: return FMT_U4;
    case QGEMM_F16: return FMT_F16;
    case QGEMM_I8: return FMT_I8;
    case QGEMM_I2: return FMT_I2;
    default: return -1;
  }
}

bool known_dtype(int d) { return d >= QGEMM_F16 && d <= QGEMM_I2; }

int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

qgemm_status fill_layout(Layout* L, int fmt, int64_t N, int64_t K, int32_t g, bool zeros) {
  L->fmt = fmt;
  L->N = N;
  L->K = K;
  L->Kpad = round_up(K, kgrain_of(fmt));
  L->Npad = round_up(N, 256);
  L->NB = L->Npad / 16;
  L->nkb = L->Kpad / kb_of(fmt);
  L->group_size = g;
  L->G = g == 0 ? 0 : g < 0 ? 1 : K / g;
  // groups smaller than a superblock are indexed per 32-position piece up to Kpad
  L->G_store = g > 0 ? (L->Kpad + g - 1) / g : L->G;
  L->zeros = zeros;
  L->w_bytes = (size_t)L->nkb * (size_t)L->NB * 1024;
  L->s_offset = (size_t)round_up((int64_t)L->w_bytes, 256);
  L->s_bytes = (size_t)L->G_store * (size_t)L->Npad * (zeros ? 4 : 2);
  L->total = L->s_offset + L->s_bytes;
  return QGEMM_OK;
}

// formats (bit per format) whose GEMV runs on the matrix cores (int8, int2, fp16;
// fp16 M = 8: 77.2 against 82.0 us),
// for M in [MIN_M, MAX_M]: the matrix cores take up to 16 rows for the price of
// one (W2A8 M = 8: 13.9 us against 31.5 us with dot products; M = 16 / 24 / 32:
// 17.1 / 22.0 / 25.3 us against 30.9 / 31.9 / 31.4 us with the direct-load
// kernel), while at M = 1 the dot-product GEMV reads its activations through the
// scalar unit and stays ahead (12.6 against 13.2 us)
#ifndef QG_GEMV_MFMA_FMTS
#define QG_GEMV_MFMA_FMTS ((1 << FMT_I8) | (1 << FMT_I2) | (1 << FMT_F16))
#endif
#ifndef QG_GEMV_MFMA_MIN_M
#define QG_GEMV_MFMA_MIN_M 2
#endif
#ifndef QG_GEMV_MFMA_MAX_M
#define QG_GEMV_MFMA_MAX_M 32
#endif
// rows for which int4 / uint4 (groups of whole superblocks) take the matrix-core
// GEMV instead of the dot-product GEMV (M <= 8) or the direct-load kernel.
// Measured at N = K = 16384, g = 128: M = 4 / 8 / 16 / 32 ran 24.6 / 25.5 / 29.2 /
// 42.4 us against 35.8 / 64.5 / 67.8 / 69.7 us; M = 2 ties with the dot-product
// GEMV (24.5 us) and unscaled M = 2 is faster there (23.4 against 24.7 us); unscaled
// M = 24 / 32 ran 37.1 / 41.4 us against 53.4 / 53.6 us with the direct-load kernel.
#ifndef QG_GEMV4_MFMA_MIN_M
#define QG_GEMV4_MFMA_MIN_M 3
#endif
#ifndef QG_GEMV4_MFMA_MAX_M
#define QG_GEMV4_MFMA_MAX_M 32
#endif
#ifndef QG_GEMV4_MFMA_MAX_M_UNSCALED
#define QG_GEMV4_MFMA_MAX_M_UNSCALED 32
#endif

#ifndef QG_GEMV_TARGET_WAVES
#define QG_GEMV_TARGET_WAVES 2048
#endif

// M = 1 and so few 64-column blocks that they would occupy under half of the 256
// CUs (with more, the 64-column kernel is faster: measured at N = 4096 .. 32000)
#ifndef QG_GEMV_NARROW_BELOW
#define QG_GEMV_NARROW_BELOW 128
#endif
bool choose_gemv_narrow(const qgemm_plan* p, int64_t M, int kp) {
  return M == 1 && (p->N + 63) / 64 * kp < QG_GEMV_NARROW_BELOW;
}

int choose_gemv_waves(const qgemm_plan* p, int cols, int kp) {
  const int64_t rb = (p->N + cols - 1) / cols;
  const int64_t per_part = p->L.nkb / kp;
  int64_t want = (QG_GEMV_TARGET_WAVES + rb * kp - 1) / (rb * kp);
  int64_t maxw = per_part / 2;
  if (maxw < 1) maxw = 1;
  if (maxw > GEMV_MAX_WAVES) maxw = GEMV_MAX_WAVES;
  if (want > maxw) want = maxw;
  if (want < 1) want = 1;
  return (int)want;
}

// 16-column blocks per workgroup of the matrix-core GEMVs: the most (4, sharing each
// activation load) whose workgroups still occupy 60 % of the 256 CUs, else 1.  N =
// 4096 thus runs 256 workgroups of 16 columns instead of 64 of 64: W4A16 M = 8,
// K = 11008 in 10.0 against 16.4 us, fp16 M = 8, K = 4096 in 8.1 against 14.1 us.
int choose_gemv_cb(const qgemm_plan* p, int kp) {
  for (int cb : {4, 2}) {
    const int64_t wgs = (p->N + 16 * cb - 1) / (16 * cb) * kp;
    const int64_t waves = (wgs + 255) / 256;
    if (wgs * 10 >= waves * 256 * 6) return cb;
  }
  return 1;
}

// LDS-staged kernel: largest tile that still gives every CU a workgroup (256 CUs).
int choose_tile(const qgemm_plan* p, int64_t M, int kp) {
  if (M <= 32) return TILE_32x64;
  auto wgs = [&](int tile) {
    int bm, bn;
    tile_dims(p->L.fmt, tile, &bm, &bn);
    return ((M + bm - 1) / bm) * ((p->N + bn - 1) / bn) * kp;
  };
  if (M >= 256 && wgs(TILE_BIG) >= 256) return TILE_BIG;
  return wgs(TILE_128x128) >= 256 ? TILE_128x128 : TILE_64x64;
}

// Scale mode of a format and group size: per superblock (groups of whole
// superblocks, or one group over K), else per 32-position piece (groups that
// are not a multiple of the superblock depth, such as 32, 64, 96 or 160 for int4)
int scale_mode(int fmt, int32_t group_size) {
  const int KB = kb_of(fmt);
  if (group_size == 0) return SC_NONE;
  if (group_size > 0 && group_size % KB != 0) return SC_PIECE;
  return SC_BLOCK;
}

// Split-K reduction.  By default the parts add into one accumulator with global
// atomics (hidet issue #364, parallel-k with atomic reduction): fp32 atomics into
// a zero-filled workspace followed by a conversion pass for fp16 outputs, int32
// atomics straight into C.  QGEMM_DETERMINISTIC selects the fixed-order two-pass
// form (partials [k_parts][M][N], then one pass that sums them in part order).
// QGEMM_SPLIT_AUTO lets the library take whichever measured faster for the plan:
// the two-pass form for fp16 outputs, where zero-filling the accumulator plus
// contended fp32 atomics cost more than the partials (k_parts = 4: M = 1, LLaMA
// shapes 10.5 -> 9.5 us; M = 128, N = 32000, K = 4096 105 -> 74 us; M = 512,
// N = K = 16384 347 -> 291 us), and for int32 outputs from 128 rows (W8A8
// M = 512: 172 against 189 us; below that the atomics win, W2A8 M = 32: 34.2
// against 37.9 us), while the partials stay within 256 MiB; atomics otherwise.
#ifndef QG_TWO_PASS_MAX_BYTES
#define QG_TWO_PASS_MAX_BYTES ((size_t)256 << 20)
#endif
#ifndef QG_TWO_PASS_INT_MIN_M
#define QG_TWO_PASS_INT_MIN_M 128
#endif
bool two_pass_split(int64_t M, size_t partial_bytes, bool out_f16, uint32_t flags) {
  if (flags & QGEMM_DETERMINISTIC) return true;
  if (!(flags & QGEMM_SPLIT_AUTO)) return false;
  if (partial_bytes > QG_TWO_PASS_MAX_BYTES) return false;
  return out_f16 || M >= QG_TWO_PASS_INT_MIN_M;
}

// k-parts and reduction of a run of M rows: the plan's, or the library's own split
// (ordered partials) for the shapes it applies to
struct qg_split {
  int kp;
  bool two_pass;
};
qg_split split_of(const qgemm_plan* p, int64_t M) {
  if (p->auto_parts > 1 && M >= p->auto_min_m) return {p->auto_parts, true};
  return {p->k_parts, p->two_pass};
}

// The library's own K split (plans of k_parts 1), summed in part order (bitwise
// reproducible).  int4 / uint4 with 33 to 256 rows, N from 4096 and K from 8192, where
// the tiles that fill the CUs are few and long: as many parts (2, 4 or 8) as one wave
// of 256 workgroups of 128 x 128 tiles takes.  N = K = 16384, M = 128: 109 -> 91 us
// (two parts of 128 x 128 tiles instead of 64 x 128); N = 4096, K = 11008, M = 128:
// 51 -> 39 us with two parts, 31 us with eight.  fp16 and int8 ran slower split
// (122 / 68 against 120 / 64 us).
#ifndef QG_AUTO_SPLIT
#define QG_AUTO_SPLIT 1
#endif
// And the matrix-core int4 GEMV at 9 to 32 rows with N up to 4096 and K from 8192,
// whose 16-column workgroups would otherwise each read all of A: four parts from 17
// rows, two from 9, so 64-column workgroups fill the CUs (M = 32, N = 4096, K = 11008:
// 22.5 -> 15.3 us; M = 16: 13.3 -> 11.7 us; one part stayed fastest at the other
// LLaMA shapes and at N = K = 16384).
struct qg_auto {
  int parts, min_m;
};
qg_auto auto_parts_of(int fmt, int32_t group_size, int64_t M, int64_t N, int64_t Kpad, int k_parts,
                      int64_t n_units) {
  if (!QG_AUTO_SPLIT || k_parts != 1 || n_units < 2) return {0, 0};
  if (fmt != FMT_I4 && fmt != FMT_U4) return {0, 0};
  if (Kpad < 8192) return {0, 0};
  if (M > 8 && M <= 32 && N <= 4096 && scale_mode(fmt, group_size) != SC_PIECE && n_units >= 4)
    return M > 16 ? qg_auto{4, 17} : qg_auto{2, 9};
  if (M <= 32 || M > 256 || N < 4096) return {0, 0};
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  int kp = 2;
  while (kp < 8 && tiles * kp * 2 <= 256 && kp * 2 <= n_units) kp *= 2;
  return {kp, 33};
}

qg_choice choose(const qgemm_plan* p, int64_t M) {
  const int kp = split_of(p, M).kp;
  qg_choice c;
  c.path = M <= 8 ? QGEMM_PATH_GEMV : QGEMM_PATH_MFMA;
  c.tile = choose_tile(p, M, kp);
  c.dl_tile = c.path == QGEMM_PATH_MFMA ? choose_dl_tile(p->L.fmt, M, p->N, kp,
                                                          scale_mode(p->L.fmt, p->group_size))
                                        : -1;
  c.gemv_narrow = c.path == QGEMM_PATH_GEMV && choose_gemv_narrow(p, M, kp);
  c.gemv_mfma = !c.gemv_narrow && M >= QG_GEMV_MFMA_MIN_M && M <= QG_GEMV_MFMA_MAX_M &&
                ((QG_GEMV_MFMA_FMTS >> p->L.fmt) & 1);
  const int smode = scale_mode(p->L.fmt, p->group_size);
  // two rows as well when the matrix is narrow enough for 16- or 32-column
  // workgroups, which the dot-product GEMV does not have (N = 4096: 4.8 against
  // 7.8 us at K = 4096, 8.4 against 16.0 us at K = 11008)
  const int min_m4 = choose_gemv_cb(p, kp) < 4 ? 2 : QG_GEMV4_MFMA_MIN_M;
  c.gemv_mfma4 = (p->L.fmt == FMT_I4 || p->L.fmt == FMT_U4) && !c.gemv_narrow && smode != SC_PIECE &&
                 M >= min_m4 && M <= (smode == SC_NONE ? QG_GEMV4_MFMA_MAX_M_UNSCALED : QG_GEMV4_MFMA_MAX_M);
  c.gemv_cb = (c.gemv_mfma || c.gemv_mfma4) ? choose_gemv_cb(p, kp) : 4;
  c.gemv_waves = choose_gemv_waves(p, c.gemv_narrow ? 16 : (c.gemv_mfma || c.gemv_mfma4) ? 16 * c.gemv_cb : 64, kp);
  return c;
}

RunArgs make_args(const qgemm_plan* p, const qg_choice& ch, int64_t M, const void* A, const void* packed,
                  const void* bias, void* C, void* ws) {
  RunArgs a;
  a.A = A;
  a.bias = bias;
  a.row_scale = nullptr;
  a.col_scale = nullptr;
  a.epi_scale = nullptr;
  a.W = static_cast<const uint4*>(packed);
  a.S = p->L.G ? static_cast<const char*>(packed) + p->L.s_offset : nullptr;
  a.C = C;
  a.ws = ws;
  a.M = (int32_t)M;
  a.N = (int32_t)p->N;
  a.K = (int32_t)p->K;
  a.Npad = (int32_t)p->L.Npad;
  a.NB = (int32_t)p->L.NB;
  a.nkb = (int32_t)p->L.nkb;
  a.group_size = p->group_size;
  const int KB = kb_of(p->L.fmt);
  a.smode = scale_mode(p->L.fmt, p->group_size);
  // position -> group as a shift when the group size is a power of two (or one
  // group spans K), else -1 (divide)
  a.g_shift = -1;
  if (p->group_size < 0) a.g_shift = 31;
  else if (p->group_size > 0 && (p->group_size & (p->group_size - 1)) == 0) a.g_shift = __builtin_ctz(p->group_size);
  a.zeros = p->has_zeros;
  const qg_split sp = split_of(p, M);
  a.k_parts = sp.kp;
  a.unit_kb = p->unit_kb;
  a.n_units = p->n_units;
  a.waves = ch.gemv_waves;
  a.gemv_cb = ch.gemv_cb;
  a.sb_per_group = p->group_size > KB ? p->group_size / KB : p->group_size < 0 ? (int32_t)p->L.nkb : 1;
  a.out_mode = sp.kp == 1 ? OUT_STORE : sp.two_pass ? OUT_PARTIAL : OUT_ATOMIC;
  a.zr = nullptr;
  a.zp = nullptr;
  a.zr_gp = 0;
  a.zr_G = 0;
  return a;
}

}  // namespace

namespace {

// workspace of a run of M rows (the plan's workspace_bytes is this at its M): the
// split-K accumulator or partials, then (K not a multiple of the superblock depth)
// the activations zero-padded to Kpad, 256-byte aligned
size_t split_ws_bytes(const qgemm_plan* p, int64_t M) {
  const qg_split sp = split_of(p, M);
  if (sp.kp == 1) return 0;
  const size_t mn4 = (size_t)M * (size_t)p->N * 4;
  if (sp.two_pass) return mn4 * (size_t)sp.kp;
  return p->out_dtype == QGEMM_F16 ? mn4 : 0;
}
size_t a_esz(const qgemm_plan* p) { return p->a_dtype == QGEMM_F16 ? 2 : 1; }
size_t pad_offset(const qgemm_plan* p, int64_t M) { return (size_t)round_up((int64_t)split_ws_bytes(p, M), 256); }
size_t split_pad_bytes(const qgemm_plan* p, int64_t M) {
  if (p->L.Kpad == p->K) return split_ws_bytes(p, M);
  return pad_offset(p, M) + (size_t)M * (size_t)p->L.Kpad * a_esz(p);
}

// Zero-point folding: uint4 with zero points and groups of whole superblocks (or one
// over K) runs on the four-wave 256 x 256 tiles with the zero points taken out of the
// K loop, C = sum_k A q s - sum_g R[m, g] s z, after two passes that write the row sums
// of A over the groups (R) and P = -s z, each as two bf16 planes of round_up(G, 32)
// values per row or column, at the end of the workspace.  The eight-wave tile with
// the zero points in its loop measured 7.6-7.8 ms at M = N = K = 16384.
#ifndef QG_ZERO_FOLD
#define QG_ZERO_FOLD 1
#endif
// Signed int4 with groups of whole superblocks folds its offset 8 the same way (one
// group over K takes the column scale in the epilogue instead).
bool zero_fold_format(const qgemm_plan* p) {
  const bool u4z = p->L.fmt == FMT_U4 && p->L.zeros;
  const bool i4s = p->L.fmt == FMT_I4 && p->group_size > 0;
  return QG_ZERO_FOLD && QG_BIG4 && (u4z || i4s) && scale_mode(p->L.fmt, p->group_size) == SC_BLOCK &&
         p->L.Kpad / 32 <= ROWSUM_MAX_UNITS;
}
bool zero_fold(const qgemm_plan* p, const qg_choice& ch) {
  return zero_fold_format(p) && ch.path == QGEMM_PATH_MFMA && ch.dl_tile == DL_256x256;
}
int64_t zr_gp_of(const qgemm_plan* p) { return round_up(p->L.G, 32); }
size_t zr_offset(const qgemm_plan* p, int64_t M) { return (size_t)round_up((int64_t)split_pad_bytes(p, M), 256); }
size_t zp_offset(const qgemm_plan* p, int64_t M) {
  return zr_offset(p, M) + (size_t)round_up(M * zr_gp_of(p) * 2 * (int64_t)sizeof(uint16_t), 256);
}
size_t run_ws_bytes_for(const qgemm_plan* p, int64_t M, bool fold) {
  if (!fold) return split_pad_bytes(p, M);
  return zp_offset(p, M) + (size_t)p->L.Npad * (size_t)zr_gp_of(p) * 2 * sizeof(uint16_t);
}
// the workspace of a run of M rows with the kernels chosen for M
size_t run_ws_bytes(const qgemm_plan* p, int64_t M, const qg_choice& ch) { return run_ws_bytes_for(p, M, zero_fold(p, ch)); }
// The most rows of a run of this plan that takes the 256 x 256 tiles with the folding
// (0: none).  The tile choice depends on the rows only through the number of 256-row
// tiles (above 128 rows), so one run per tile count is checked, from the plan's down.
int64_t fold_rows(const qgemm_plan* p) {
  if (!zero_fold_format(p)) return 0;
  for (int64_t rt = (p->M + 255) / 256; rt >= 1; --rt) {
    const int64_t m = p->M < rt * 256 ? p->M : rt * 256;
    if (m <= 128) break;
    if (zero_fold(p, choose(p, m))) return m;
  }
  return 0;
}

// one run: the split-K fill, the kernel chosen for M rows, the finalize pass
qgemm_status run_impl(const qgemm_plan* plan, int64_t M, const void* A, const void* packed, const void* bias,
                      const float* row_scales, const float* col_scales, void* C, void* workspace,
                      size_t workspace_bytes, void* stream) {
  if (!plan || !A || !packed || !C) return QGEMM_ERR_INVALID_ARG;
  if (M < 1 || M > plan->M) return QGEMM_ERR_INVALID_ARG;
  const qg_choice ch = M == plan->M ? plan->ch : choose(plan, M);
  const bool fold = zero_fold(plan, ch);
  const size_t need = run_ws_bytes(plan, M, ch);
  if (need && (!workspace || workspace_bytes < need)) return QGEMM_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(packed) |
       reinterpret_cast<uintptr_t>(workspace)) & 15)
    return QGEMM_ERR_INVALID_ARG;
  const bool out_f16 = plan->out_dtype == QGEMM_F16;
  const bool acc_fp = plan->a_dtype == QGEMM_F16;
  if (reinterpret_cast<uintptr_t>(bias) & (out_f16 ? 1 : 3)) return QGEMM_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(row_scales) | reinterpret_cast<uintptr_t>(col_scales)) & 3)
    return QGEMM_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(stream);
  RunArgs a = make_args(plan, ch, M, A, packed, bias, C, workspace);
  a.row_scale = row_scales;
  a.col_scale = col_scales;
  (void)hipGetLastError();  // clear an error left by an unrelated earlier call on this thread
  hipError_t e = hipSuccess;
  if (plan->L.Kpad != plan->K) {
    // K is not a multiple of the superblock depth: the kernels read the activations
    // zero-padded to Kpad (the blob holds zero codes there)
    void* Ap = static_cast<char*>(workspace) + pad_offset(plan, M);
    e = launch_pad_rows(A, Ap, M, plan->K, plan->L.Kpad, (int)a_esz(plan), st);
    a.A = Ap;
    a.K = (int32_t)plan->L.Kpad;
  }
  if (e == hipSuccess && fold) {
    uint16_t* zr = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + zr_offset(plan, M));
    uint16_t* zp = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + zp_offset(plan, M));
    a.zr_gp = (int32_t)zr_gp_of(plan);
    a.zr_G = (int32_t)plan->L.G;
    e = launch_group_rowsum(a, zr, st);
    if (e == hipSuccess) e = launch_zero_planes(a, zp, st);
    a.zr = zr;
    a.zp = zp;
  }
  if (e == hipSuccess && a.out_mode == OUT_ATOMIC)
    e = out_f16 ? launch_fill_zero(workspace, (size_t)M * plan->N * 4, st)  // fp32 / int32 accumulator
        : bias  ? launch_fill_bias(a, st)
                : launch_fill_zero(C, (size_t)M * plan->N * 4, st);
  if (e == hipSuccess)
    e = ch.gemv_mfma4 ? launch_gemv_mfma4(plan->L.fmt, a, st)
        : ch.gemv_mfma ? launch_gemv_mfma(plan->L.fmt, a, st)
        : ch.path == QGEMM_PATH_GEMV ? (ch.gemv_narrow ? launch_gemv16(plan->L.fmt, a, st)
                                                       : launch_gemv(plan->L.fmt, a, st))
        : ch.dl_tile >= 0 ? launch_mfma_dl(plan->L.fmt, ch.dl_tile, a, st)
        : launch_mfma(plan->L.fmt, ch.tile, a, st);
  if (e == hipSuccess && (a.out_mode == OUT_PARTIAL || (a.out_mode == OUT_ATOMIC && out_f16)))
    e = launch_finalize(a, acc_fp, st);
  return e == hipSuccess ? QGEMM_OK : QGEMM_ERR_DEVICE;
}

bool dequant_plan(const qgemm_plan* p) { return p->a_dtype == QGEMM_I8 && p->out_dtype == QGEMM_F16; }

}  // namespace

// Scratch of qgemm_run_noalloc: a fixed array in device memory, one copy per GPU
// (each holds it until the process ends).  In host code `scratch` names only a
// stand-in for the symbol; the device address comes from hipGetSymbolAddress,
// taken once per device with that device current and kept in scratch_ptr.
static __device__ __align__(256) uint8_t scratch[QGEMM_NOALLOC_MAX_SCRATCH];

namespace {

constexpr int QG_MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[QG_MAX_DEVICES] = {};

// device address of the current device's scratch array (looked up on first use)
hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= QG_MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

qgemm_status qgemm_create(qgemm_plan** out, int64_t M, int64_t N, int64_t K, qgemm_dtype a_dtype,
                          qgemm_dtype w_dtype, qgemm_dtype out_dtype, qgemm_dtype accum_dtype,
                          int32_t group_size, int32_t has_zeros, int32_t k_parts, uint32_t flags,
                          size_t* packed_bytes, size_t* workspace_bytes) {
  if (!out) return QGEMM_ERR_INVALID_ARG;
  *out = nullptr;
  if (M < 1 || N < 1 || K < 1) return QGEMM_ERR_INVALID_ARG;
  if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return QGEMM_ERR_UNSUPPORTED;
  if (!known_dtype(a_dtype) || !known_dtype(w_dtype) || !known_dtype(out_dtype) || !known_dtype(accum_dtype))
    return QGEMM_ERR_INVALID_ARG;
  if (has_zeros != 0 && has_zeros != 1) return QGEMM_ERR_INVALID_ARG;
  if (k_parts < 1) return QGEMM_ERR_INVALID_ARG;
  if (flags & ~(QGEMM_DETERMINISTIC | QGEMM_SPLIT_AUTO)) return QGEMM_ERR_INVALID_ARG;
  if (group_size < -1) return QGEMM_ERR_INVALID_ARG;

  // legal format tuples
  const bool fp_tuple = a_dtype == QGEMM_F16 && out_dtype == QGEMM_F16 && accum_dtype == QGEMM_F32 &&
                        (w_dtype == QGEMM_I4 || w_dtype == QGEMM_U4 || w_dtype == QGEMM_F16);
  // int8 activations: int32 output, or fp16 output dequantised with per-row and
  // per-column scales (qgemm_run_scaled)
  const bool int_tuple = a_dtype == QGEMM_I8 && (out_dtype == QGEMM_I32 || out_dtype == QGEMM_F16) &&
                         accum_dtype == QGEMM_I32 && (w_dtype == QGEMM_I8 || w_dtype == QGEMM_I2);
  if (!fp_tuple && !int_tuple) return QGEMM_ERR_UNSUPPORTED;
  const int fmt = fmt_of(w_dtype);
  const int KB = kb_of(fmt);
  const bool scaled_fmt = fmt == FMT_I4 || fmt == FMT_U4;

  // scaling and zero points
  if (!scaled_fmt && group_size != 0) return QGEMM_ERR_UNSUPPORTED;
  if (has_zeros && (fmt != FMT_U4 || group_size == 0)) return QGEMM_ERR_UNSUPPORTED;
  if (group_size > 0 && (K % group_size != 0 || group_size % 32 != 0)) return QGEMM_ERR_UNSUPPORTED;
  // K: whole canonical words (8 int4, 16 int2 values); the kernels run on K padded
  // to whole superblocks
  if (K % pack_factor(fmt) != 0) return QGEMM_ERR_UNSUPPORTED;
  const int64_t Kpad = round_up(K, kgrain_of(fmt));
  if (Kpad > INT32_MAX) return QGEMM_ERR_UNSUPPORTED;

  // kernels index the blob with 32-bit uint4 offsets and the activations with
  // 32-bit byte offsets
  if ((N + 255) / 256 * 256 / 16 * (Kpad / KB) * 64 >= INT32_MAX) return QGEMM_ERR_UNSUPPORTED;
  if ((uint64_t)M * (uint64_t)Kpad * (a_dtype == QGEMM_F16 ? 2u : 1u) >= ((uint64_t)1 << 32))
    return QGEMM_ERR_UNSUPPORTED;

  // split unit: whole superblocks, and whole groups when groups are whole superblocks
  // (then K is a multiple of the group, so Kpad = K)
  const int64_t unit = scale_mode(fmt, group_size) == SC_BLOCK && group_size > KB ? group_size : kgrain_of(fmt);
  const int64_t n_units = Kpad / unit;
  if (k_parts > n_units) return QGEMM_ERR_INVALID_ARG;

  qgemm_plan* p = new (std::nothrow) qgemm_plan();
  if (!p) return QGEMM_ERR_NO_MEMORY;
  p->M = M;
  p->N = N;
  p->K = K;
  p->a_dtype = a_dtype;
  p->w_dtype = w_dtype;
  p->out_dtype = out_dtype;
  p->accum_dtype = accum_dtype;
  p->group_size = group_size;
  p->has_zeros = has_zeros;
  p->k_parts = k_parts;
  p->flags = flags;
  fill_layout(&p->L, fmt, N, K, group_size, has_zeros != 0);
  p->unit_kb = (int32_t)(unit / KB);
  p->n_units = (int32_t)n_units;
  const qg_auto au = auto_parts_of(fmt, group_size, M, N, Kpad, k_parts, n_units);
  p->auto_parts = au.parts;
  p->auto_min_m = au.min_m;
  const size_t mn4 = (size_t)M * (size_t)N * 4;
  p->two_pass = k_parts > 1 && two_pass_split(M, mn4 * (size_t)k_parts, out_dtype == QGEMM_F16, flags);
  p->ch = choose(p, M);
  // int32 output with atomics: none (straight into C).  With the folding, the planes
  // of the largest run that takes it, so that runs of fewer rows never need more than
  // the plan states
  p->ws_bytes = run_ws_bytes(p, M, p->ch);
  const int64_t mf = fold_rows(p);
  if (mf > 0 && run_ws_bytes_for(p, mf, true) > p->ws_bytes) p->ws_bytes = run_ws_bytes_for(p, mf, true);
  if (packed_bytes) *packed_bytes = p->L.total;
  if (workspace_bytes) *workspace_bytes = p->ws_bytes;
  *out = p;
  return QGEMM_OK;
}

qgemm_status qgemm_pack_weights(const qgemm_plan* plan, const void* w, const void* scales, const void* zeros,
                                void* packed, void* stream) {
  if (!plan || !w || !packed) return QGEMM_ERR_INVALID_ARG;
  if (plan->L.G && !scales) return QGEMM_ERR_INVALID_ARG;
  if (plan->L.zeros && !zeros) return QGEMM_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(packed)) & 15) return QGEMM_ERR_INVALID_ARG;
  (void)hipGetLastError();  // clear an error left by an unrelated earlier call on this thread
  hipError_t e = launch_pack(plan->L, w, scales, zeros, packed, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_ERR_DEVICE;
}

qgemm_status qgemm_run_ex(const qgemm_plan* plan, int64_t M, const void* A, const void* packed,
                          const void* bias, void* C, void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || dequant_plan(plan)) return QGEMM_ERR_INVALID_ARG;  // those need their scales
  return run_impl(plan, M, A, packed, bias, nullptr, nullptr, C, workspace, workspace_bytes, stream);
}

qgemm_status qgemm_run_noalloc(const qgemm_plan* plan, int64_t M, const void* A, const void* packed,
                               const void* bias, void* C, void* stream) {
  if (!plan || dequant_plan(plan)) return QGEMM_ERR_INVALID_ARG;
  if (M < 1 || M > plan->M) return QGEMM_ERR_INVALID_ARG;
  const size_t need = run_ws_bytes(plan, M, M == plan->M ? plan->ch : choose(plan, M));
  if (need > QGEMM_NOALLOC_MAX_SCRATCH) return QGEMM_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need) {
    (void)hipGetLastError();
    if (scratch_of_current_device(&ws) != hipSuccess) return QGEMM_ERR_DEVICE;
  }
  return run_impl(plan, M, A, packed, bias, nullptr, nullptr, C, ws, need, stream);
}

qgemm_status qgemm_run_scaled(const qgemm_plan* plan, int64_t M, const void* A, const void* packed,
                              const float* row_scales, const float* col_scales, const void* bias, void* C,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (!plan || !dequant_plan(plan) || !row_scales || !col_scales) return QGEMM_ERR_INVALID_ARG;
  return run_impl(plan, M, A, packed, bias, row_scales, col_scales, C, workspace, workspace_bytes, stream);
}

qgemm_status qgemm_quantize_rows(const void* A, int64_t M, int64_t K, void* Q, float* scales, void* stream) {
  if (!A || !Q || !scales || M < 1 || K < 8 || K % 8 != 0) return QGEMM_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(A) & 15) || (reinterpret_cast<uintptr_t>(Q) & 7) ||
      (reinterpret_cast<uintptr_t>(scales) & 3))
    return QGEMM_ERR_INVALID_ARG;
  (void)hipGetLastError();
  hipError_t e = launch_quantize_rows(A, M, K, Q, scales, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? QGEMM_OK : QGEMM_ERR_DEVICE;
}

qgemm_status qgemm_run(const qgemm_plan* plan, const void* A, const void* packed, void* C, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (!plan) return QGEMM_ERR_INVALID_ARG;
  return qgemm_run_ex(plan, plan->M, A, packed, nullptr, C, workspace, workspace_bytes, stream);
}

void qgemm_destroy(qgemm_plan* plan) { delete plan; }

int32_t qgemm_plan_path(const qgemm_plan* plan) { return plan ? plan->ch.path : -1; }

const char* qgemm_status_string(qgemm_status s) {
  switch (s) {
    case QGEMM_OK: return "ok";
    case QGEMM_ERR_INVALID_ARG: return "invalid argument";
    case QGEMM_ERR_UNSUPPORTED: return "unsupported format or shape";
    case QGEMM_ERR_NO_MEMORY: return "out of host memory";
    case QGEMM_ERR_DEVICE: return "device launch failed";
  }
  return "unknown status";
}

}  // extern "C"
