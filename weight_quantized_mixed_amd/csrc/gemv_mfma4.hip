// Skinny-M int4 / uint4 path on the matrix cores (3 <= M <= 32).
//
// Lane l of a wave works on column l % 16 of a 16-column superblock and K group
// g = l / 16 of every 32-position MFMA step.  In the packed blob, word g of the
// piece of step s holds exactly that group's eight positions (nibble slots 0..7 =
// positions 0,2,4,6,1,3,5,7).  A superblock is loaded as stored (one 16-byte load,
// piece l for lane l: step l / 16, column l % 16), and a 4 x 4 transpose of dwords
// across the four 16-lane rows (two permlane32 and two permlane16 swaps) hands
// lane (g, c) word g of the piece of every step; four v_and_or_b32 turn slot pairs
// (jj, jj + 4) into the fp16 pairs 1024 + b + q (b the offset of the code: 8 for
// signed int4, 0 for uint4) and one packed fp16 subtraction per pair takes
// 1024 + b off, exactly.  (Loading the words one dword per step instead,
// 16 loads of 256 bytes per wave for four superblocks, ran M = 8 in 40.9 against
// 25.5 us.)  The A operand is a row of activations
// (lane l: row l % 16 of the row block, positions 32 s + 8 g .. + 7), so one set
// of B operands serves up to 16 rows per MFMA, two row blocks up to 32.
//
// A workgroup owns CB superblock columns (16, 32 or 64 columns, the most that still
// gives the CUs enough workgroups) and a k-part; its waves take the part's
// superblock rows in turn and meet in LDS at the end.
//
// Without scales the MFMAs accumulate sum a q straight into the result.  With
// scales they accumulate T = sum a q per superblock and column block into a
// temporary, folded as acc += s * T; with zero points three more MFMAs per
// superblock against a B of fp16 ones give the row sums S = sum a, and the fold is
//   acc += s * (T - z * S)                                  (all in fp32)
// which is sum a (q - z) s for its scale group.  Products a q are exact in fp32
// and the partial sums stay as small as the result's own terms: keeping the
// 1024 + b offsets in the operands (and removing them once per superblock) would
// make T about a thousand times larger than the true sum, and its fp32 rounding
// alone exceeds a 1e-2 error at K = 16384 without scales.
// Groups of whole superblocks (or one group over K) only; 32- and 64-position
// groups take the dot-product GEMV.
#include "qgemm_internal.hpp"

namespace qg {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));

// (x & m) | c, left to the compiler (v_and_or_b32): its results feed an MFMA a few
// instructions later, and the compiler inserts the wait states that a VALU write
// followed by a matrix-core read of the same register needs, which it cannot do
// for an inline-assembly writer
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) { return (x & m) | c; }

__device__ __forceinline__ uint4 stream_load16(const uint4* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

// 4 x 4 transpose of dwords across the four 16-lane rows: lane (row r, column c)
// holds x[w] = word w of row r's piece; afterwards x[t] = word r of row t's piece
// (column c).  Two row-pair swaps, then two neighbouring-row swaps.
__device__ __forceinline__ void transpose_rows(uint32_t (&x)[4]) {
  auto a = __builtin_amdgcn_permlane32_swap(x[0], x[2], false, false);  // rows 2,3 of x0 <-> rows 0,1 of x2
  auto b = __builtin_amdgcn_permlane32_swap(x[1], x[3], false, false);
  auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);  // odd rows of x0 <-> even rows of x1
  auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  x[0] = c[0];
  x[1] = c[1];
  x[2] = d[0];
  x[3] = d[1];
}

__device__ __forceinline__ uint4 load16(const uint4* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u t = *reinterpret_cast<const v4u*>(p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ float4v mfma(const uint4& A, const uint4& B, const float4v& C) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8v, A), __builtin_bit_cast(half8v, B), C, 0, 0, 0);
}

// VAR: 0 unscaled, 1 scaled, 2 scaled with zero points
template <int FMT, int MB, int VAR, int CB>
__global__ __launch_bounds__(64 * GEMV_MAX_WAVES) void gemv_mfma4_kernel(RunArgs a) {
  constexpr int KB = 128, NS = 4;  // positions and 32-position MFMA steps per superblock
  constexpr bool SCALED = VAR >= 1, ZEROS = VAR == 2;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = blockIdx.x, part = blockIdx.y;
  const int g = lane >> 4, n16 = lane & 15;

  int u0, u1;
  part_units(a, part, u0, u1);
  const int kb0 = u0 * a.unit_kb, kb1 = u1 * a.unit_kb;
  const int cnt = __builtin_amdgcn_readfirstlane(kb1 - kb0 > wave ? (kb1 - kb0 - wave + a.waves - 1) / a.waves : 0);
  auto row_of = [&](int j) { return __builtin_amdgcn_readfirstlane(kb0 + wave + j * a.waves); };

  // activation rows of the lane (rows past M repeat row M - 1; results dropped)
  const uint4* __restrict__ Al[MB];
#pragma unroll
  for (int r = 0; r < MB; ++r)
    Al[r] = reinterpret_cast<const uint4*>(static_cast<const _Float16*>(a.A) + (size_t)min(r * 16 + n16, a.M - 1) * a.K) + g;

  // piece l of each superblock (16 bytes) for lane l, as stored
  const uint4* __restrict__ Wq = a.W + (size_t)rb * CB * 64 + lane;
  const uint32_t sbq_stride = (uint32_t)a.NB * 64u;  // uint4 per superblock row
  struct Stage {
    uint4 av[MB][NS];  // A operand of each row block and step
    uint4 wq[CB];       // piece (lane / 16, lane % 16) of each column block, as stored
    uint32_t sc[CB];    // raw scale (| zero << 16) of each column block
  };
  auto load = [&](Stage& s, int j) {
    const uint32_t kb = (uint32_t)row_of(min(j, cnt - 1));
#pragma unroll
    for (int r = 0; r < MB; ++r)
#pragma unroll
      for (int t = 0; t < NS; ++t) s.av[r][t] = load16(Al[r] + kb * (KB / 8) + t * 4);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) s.wq[cb] = stream_load16(Wq + kb * sbq_stride + cb * 64);
    if constexpr (SCALED) {
      const uint32_t grp = a.sb_per_group == 1 ? kb : kb / (uint32_t)a.sb_per_group;
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint32_t col = (uint32_t)((rb * CB + cb) * 16 + n16);
        if constexpr (ZEROS) s.sc[cb] = static_cast<const uint32_t*>(a.S)[grp * (uint32_t)a.Npad + col];
        else s.sc[cb] = static_cast<const uint16_t*>(a.S)[grp * (uint32_t)a.Npad + col];
      }
    }
  };

  float4v acc[MB][CB];
#pragma unroll
  for (int r = 0; r < MB; ++r)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) acc[r][cb] = float4v{0.f, 0.f, 0.f, 0.f};

  const uint4 ONES = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);
  // 1024 + b in both halves: (1024 + b + q) - (1024 + b) = q exactly in fp16
  const half2v OFS = __builtin_bit_cast(half2v, FMT == FMT_I4 ? 0x64086408u : 0x64006400u);
  auto code = [&](uint32_t x) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2v, and_or(x, 0x000F000Fu, 0x64006400u)) - OFS);
  };
  auto consume = [&](const Stage& s) {
    // packed word of each column block and step: word g of the piece of step t
    uint32_t w[CB][NS];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      uint32_t x[4] = {s.wq[cb].x, s.wq[cb].y, s.wq[cb].z, s.wq[cb].w};
      transpose_rows(x);
#pragma unroll
      for (int t = 0; t < NS; ++t) w[cb][t] = x[t];
    }
    // scaled: per-superblock sums T (and row sums S with zero points); unscaled:
    // straight into acc
    float4v T[MB][CB], S[MB];
#pragma unroll
    for (int r = 0; r < MB; ++r) {
      S[r] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) T[r][cb] = float4v{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int t = 0; t < NS; ++t) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const uint32_t wd = w[cb][t];
        const uint4 B = make_uint4(code(wd), code(wd >> 4), code(wd >> 8), code(wd >> 12));
#pragma unroll
        for (int r = 0; r < MB; ++r) {
          if constexpr (SCALED) T[r][cb] = mfma(s.av[r][t], B, T[r][cb]);
          else acc[r][cb] = mfma(s.av[r][t], B, acc[r][cb]);
        }
      }
      if constexpr (ZEROS) {
#pragma unroll
        for (int r = 0; r < MB; ++r) S[r] = mfma(s.av[r][t], ONES, S[r]);
      }
    }
    if constexpr (SCALED) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const float sc = (float)__builtin_bit_cast(_Float16, (uint16_t)(s.sc[cb] & 0xFFFFu));
        const float z = ZEROS ? (float)__builtin_bit_cast(_Float16, (uint16_t)(s.sc[cb] >> 16)) : 0.f;
#pragma unroll
        for (int r = 0; r < MB; ++r)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            if constexpr (ZEROS) acc[r][cb][i] += sc * (T[r][cb][i] - z * S[r][i]);
            else acc[r][cb][i] += sc * T[r][cb][i];
          }
      }
    }
  };

  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  Stage s0, s1;
  if (cnt > 0) {
    int j = 0;
    load(s0, 0);
    for (; j + 2 < cnt; j += 2) {
      fence();
      load(s1, j + 1);
      fence();
      consume(s0);
      fence();
      load(s0, j + 2);
      fence();
      consume(s1);
    }
    fence();
    if (j + 1 < cnt) {
      load(s1, j + 1);
      fence();
      consume(s0);
      fence();
      consume(s1);
    } else {
      consume(s0);
    }
  }

  // lane l holds rows 16 r + 4 (l / 16) + i of column l % 16 of each column block;
  // the waves meet in LDS
  __shared__ float red[GEMV_MAX_WAVES][MB][CB][4][64];
#pragma unroll
  for (int r = 0; r < MB; ++r)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][r][cb][i][lane] = acc[r][cb][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < MB * CB * 4 * 64; idx += blockDim.x) {
    const int r = idx / (CB * 256), cb = (idx >> 8) % CB, i = (idx >> 6) & 3, ln = idx & 63;
    const int row = r * 16 + 4 * (ln >> 4) + i, col = (rb * CB + cb) * 16 + (ln & 15);
    if (row >= a.M || col >= a.N) continue;
    float v = 0.f;
    for (int w = 0; w < a.waves; ++w) v += red[w][r][cb][i][ln];
    const size_t o = (size_t)row * a.N + col;
    if (a.out_mode == OUT_STORE) static_cast<_Float16*>(a.C)[o] = (_Float16)(v + bias_f(a, col));
    else if (a.out_mode == OUT_ATOMIC) unsafeAtomicAdd(static_cast<float*>(a.ws) + o, v);
    else static_cast<float*>(a.ws)[(size_t)part * a.M * a.N + o] = v;
  }
}

template <int FMT, int MB, int CB>
hipError_t launch_cb(const RunArgs& a, hipStream_t st) {
  const dim3 grid((a.N + 16 * CB - 1) / (16 * CB), a.k_parts), block(64 * a.waves);
  const int var = a.smode == SC_NONE ? 0 : a.zeros ? 2 : 1;
  if (var == 0) hipLaunchKernelGGL((gemv_mfma4_kernel<FMT, MB, 0, CB>), grid, block, 0, st, a);
  else if (var == 1) hipLaunchKernelGGL((gemv_mfma4_kernel<FMT, MB, 1, CB>), grid, block, 0, st, a);
  else if (FMT == FMT_U4) hipLaunchKernelGGL((gemv_mfma4_kernel<FMT_U4, MB, 2, CB>), grid, block, 0, st, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <int FMT, int MB>
hipError_t launch_mb(const RunArgs& a, hipStream_t st) {
  switch (a.gemv_cb) {
    case 1: return launch_cb<FMT, MB, 1>(a, st);
    case 2: return launch_cb<FMT, MB, 2>(a, st);
    case 4: return launch_cb<FMT, MB, 4>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemv_mfma4(int fmt, const RunArgs& a, hipStream_t st) {
  if (a.M < 1 || a.M > 32 || a.smode == SC_PIECE) return hipErrorInvalidValue;
  if (fmt == FMT_I4) return a.M <= 16 ? launch_mb<FMT_I4, 1>(a, st) : launch_mb<FMT_I4, 2>(a, st);
  if (fmt == FMT_U4) return a.M <= 16 ? launch_mb<FMT_U4, 1>(a, st) : launch_mb<FMT_U4, 2>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace qg
