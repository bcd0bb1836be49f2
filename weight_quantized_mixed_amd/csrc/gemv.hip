// Skinny-M path (M <= 8): wavefront dot products straight from HBM, no matrix cores.
//
// Each workgroup owns 64 output columns (four 16-column superblock columns)
// and one k-part; its waves take the part's superblock rows in turn and meet
// in LDS at the end (the intra-workgroup "block reduction" that the
// BitBLAS issue #252 discussion names as the cure for slow skinny dequantised
// shapes).  Lane l owns column n = 64*rb + l: for every superblock it loads
// the four 16-byte pieces of its column (one wave-wide load per quarter reads
// 4 x 256 contiguous bytes), unpacks them in registers (the packed-upcast
// trick of hidet issue #364) and dots them with the activation slice.  The
// loads of the next superblocks are issued before the current ones are
// consumed (two register stages), so every wave keeps 128 bytes per lane in
// flight while it computes.  All lanes of a wave need the same activations,
// so A is read through the scalar unit (constant address space).
//
// Bias folding.  The packed int4 nibble v (offset-binary) becomes the fp16
// 1024 + v with one and-or, and 1024 + 16v when taken from the upper nibble of
// a byte, so no per-element subtraction is needed: per superblock and row,
//   sum a*q = accE + accO/16 - (1024 + b)*SE - (64 + b)*SO,
// where accE / accO are the dot products of the two nibble classes, SE / SO the
// sums of the activations over the positions of each class, and b the
// offset (8 for signed, 0 for unsigned).  Without scales the offsets are taken
// off in fp16 instead (one exact packed subtraction per pair, so accE and accO sum
// a*q and a*16q): unscaled sums over K = 16384 reach about 600, and the folded
// accumulators, about a thousand times larger than the true sums, would round
// beyond a 1e-2 error on the results near zero; a scale (0.005..0.02) shrinks that
// error below it.  int2 crumbs are masked in place
// (byte values c, 4c, 16c, and the two's complement top crumb as 64q), dotted
// with int8 activations into four accumulators, and recombined exactly.  The
// activation sums come from one load per lane and a DPP reduction per
// superblock.  k-parts > 1 reduce across workgroups with global atomics or a
// two-pass partial store (hidet issue #364, parallel-k).
#include "qgemm_internal.hpp"

namespace qg {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) uint32_t* cptr;

__device__ __forceinline__ half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }
__device__ __forceinline__ float h2f(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

// (x & m) | c in one VALU op (the masks are not inline constants, so they are
// passed in registers)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// Weights are read exactly once: non-temporal loads keep them from displacing
// the activations and scales in the caches.
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

template <int CTRL, int ROW_MASK, typename T>
__device__ __forceinline__ T dpp_add(T v) {
  const int moved = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xF, true);
  return v + __builtin_bit_cast(T, moved);
}

// After this, lane 31 holds the sum over lanes 0..31 and lane 63 the sum over
// lanes 32..63 (in-row inclusive scans by row_shr 1, 2, 4, 8, then row_bcast15
// into rows 1 and 3).
template <typename T>
__device__ __forceinline__ T half_wave_sums(T v) {
  v = dpp_add<0x111, 0xF>(v);
  v = dpp_add<0x112, 0xF>(v);
  v = dpp_add<0x114, 0xF>(v);
  v = dpp_add<0x118, 0xF>(v);
  v = dpp_add<0x142, 0xA>(v);
  return v;
}

template <typename T>
__device__ __forceinline__ T lane_value(T v, int lane) {
  return __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// VAR (int4 only): 0 unscaled (offsets taken off exactly); 1 folded with one scale group per
// superblock; 2 as 1 with zero points; 3 exact per-element conversion with a
// scale group per 32-position piece (group size 32 or 64).  int2 is always folded.
template <int FMT, int MR, int VAR>
__global__ __launch_bounds__(64 * GEMV_MAX_WAVES) void gemv_kernel(RunArgs a) {
  constexpr bool FOLD = (FMT == FMT_I2) || ((FMT == FMT_I4 || FMT == FMT_U4) && VAR != 3);
  constexpr bool SCALED = VAR == 1 || VAR == 2;
  constexpr bool ZEROS = VAR == 2;
  constexpr bool FP = (FMT == FMT_I4 || FMT == FMT_U4 || FMT == FMT_F16);
  constexpr bool I4 = (FMT == FMT_I4 || FMT == FMT_U4);
  // unscaled int4: offsets taken off per pair (exact), no activation class sums
  constexpr bool EXACT = I4 && VAR == 0;
  constexpr bool SUMS = FOLD && !EXACT;  // per-superblock activation class sums
  typedef typename std::conditional<FP, float, int>::type acc_t;
  // dwords of A per row: fp16 -> K/2, int8 -> K/4; every superblock is 64 dwords of A per row
  const int a_row_dw = FP ? a.K / 2 : a.K / 4;
  constexpr int A_DW_SB = (FMT == FMT_F16) ? 16 : (FMT == FMT_I8) ? 16 : 64;

  const int lane = threadIdx.x & 63;
  // uniform within a wave: keeps the K range and activation addresses scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = blockIdx.x, part = blockIdx.y;
  const int n = rb * 64 + lane;

  int u0, u1;
  part_units(a, part, u0, u1);
  const int kb0 = u0 * a.unit_kb, kb1 = u1 * a.unit_kb;
  // The waves of a workgroup take the part's superblock rows in turn (wave w:
  // rows kb0 + w, kb0 + w + waves, ...), so at any moment the whole grid streams
  // one narrow band of consecutive 1 KiB superblock rows, which the memory system
  // serves much faster than one contiguous run per wave spread over the matrix.
  // (wave-uniform: readfirstlane keeps the loop counter and row index in scalar
  // registers, which the compiler does not infer by itself here)
  const int cnt = __builtin_amdgcn_readfirstlane(kb1 - kb0 > wave ? (kb1 - kb0 - wave + a.waves - 1) / a.waves : 0);
  auto row_of = [&](int j) { return __builtin_amdgcn_readfirstlane(kb0 + wave + j * a.waves); };

  cptr A = (cptr)a.A;
  const uint32_t* __restrict__ Av = static_cast<const uint32_t*>(a.A);
  const uint4* __restrict__ Wl = a.W + (size_t)(rb * 4 + (lane >> 4)) * 64 + (lane & 15);
  // 32-bit offsets: the blob is far below 2^31 uint4 and A below 2^31 dwords
  const uint32_t sb_stride = (uint32_t)a.NB * 64u;  // uint4 per superblock row (kb)
  const uint32_t a_row = (uint32_t)a_row_dw;
  // activation dword this lane feeds into the per-superblock class sums
  const int sum_dw = (FMT == FMT_I2) ? lane : (lane < 32 ? 2 * lane : 2 * (lane - 32) + 1);

  acc_t tot[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) tot[m] = 0;
  // int2: per-lane sums of the class 0..2 activations (lane l holds dword l of a
  // superblock's row, class l % 4) over the wave's superblocks; the column-independent
  // offset-binary correction is taken from them once, after the loop
  int sacc[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) sacc[m] = 0;
  const int ones012 = (lane & 3) == 3 ? 0 : 0x01010101;

  constexpr int UNR = FMT == FMT_I2 ? QG_GEMV_UNR_I2 : QG_GEMV_UNR;
  struct Stage {
    uint4 w[UNR][4];
    uint32_t as[UNR][MR];
    uint32_t sc[UNR];  // raw scale (or scale | zero << 16) of the superblock's group
  };

  // Every stage issues the same loads (in a partial stage, superblocks past the
  // wave's range re-read its last one and are not used), so the compiler can count
  // outstanding loads exactly and never has to drain the next stage to use this one.
  auto load = [&](Stage& s, int j) {
#pragma unroll
    for (int u = 0; u < UNR; ++u) {
      const uint32_t kbl = (uint32_t)row_of(min(j + u, cnt - 1));
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) s.w[u][kq] = stream_load(&Wl[kbl * sb_stride + kq * 16]);
      if constexpr (SUMS) {
#pragma unroll
        for (int m = 0; m < MR; ++m) s.as[u][m] = Av[m * a_row + kbl * A_DW_SB + sum_dw];
      }
      if constexpr (SCALED) {
        // group of the superblock: sb_per_group = g / 128 (nkb when one group spans K)
        const uint32_t grp = a.sb_per_group == 1 ? kbl : kbl / (uint32_t)a.sb_per_group;
        if constexpr (ZEROS) s.sc[u] = static_cast<const uint32_t*>(a.S)[grp * (uint32_t)a.Npad + n];
        else s.sc[u] = static_cast<const uint16_t*>(a.S)[grp * (uint32_t)a.Npad + n];
      } else {
        s.sc[u] = 0x3C00u;  // 1.0
      }
    }
  };

  auto scale_of = [&](int grp, float& s, float& z) {
    if (a.zeros) {
      const uint32_t sz = static_cast<const uint32_t*>(a.S)[(size_t)grp * a.Npad + n];
      s = h2f((uint16_t)(sz & 0xFFFF));
      z = h2f((uint16_t)(sz >> 16));
    } else {
      s = h2f(static_cast<const uint16_t*>(a.S)[(size_t)grp * a.Npad + n]);
      z = 0.f;
    }
  };

  // offsets of the even (1024 + b) and odd (1024 + 16 b) nibble classes as fp16 pairs
  const half2v OFS_E = as_h2(FMT == FMT_I4 ? 0x64086408u : 0x64006400u);
  const half2v OFS_O = as_h2(FMT == FMT_I4 ? 0x64806480u : 0x64006400u);
  auto exact = [&](half2v x, half2v o) { return EXACT ? x - o : x; };

  // adds a superblock's nibble-class sums to the result: exact sums directly;
  // folded ones less the offsets times the activation class sums, scaled
  auto fold = [&](const float (&accE)[MR], const float (&accO)[MR], const uint32_t (&as)[MR], uint32_t sc) {
    if constexpr (EXACT) {
#pragma unroll
      for (int m = 0; m < MR; ++m) tot[m] += accE[m] + accO[m] * 0.0625f;
    } else {
      constexpr float cE = (FMT == FMT_I4) ? 1032.f : 1024.f, cO = (FMT == FMT_I4) ? 72.f : 64.f;
      const float s = h2f((uint16_t)(sc & 0xFFFFu)), z = h2f((uint16_t)(sc >> 16));
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        const float h = half_wave_sums(__builtin_amdgcn_fdot2(as_h2(as[m]), as_h2(0x3C003C00u), 0.f, false));
        const float SE = lane_value(h, 31), SO = lane_value(h, 63);
        float v = accE[m] + accO[m] * 0.0625f - cE * SE - cO * SO;
        if constexpr (ZEROS) v -= z * (SE + SO);
        tot[m] += SCALED ? s * v : v;
      }
    }
  };

  auto do_block = [&](const uint4 (&wv)[4], const uint32_t (&as)[MR], uint32_t sc, int kb) {
    if constexpr (I4 && FOLD) {
      const uint32_t MASK_E = 0x000F000Fu, MASK_O = 0x00F000F0u, EXP16 = 0x64006400u;
      float accE[MR], accO[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) { accE[m] = 0.f; accO[m] = 0.f; }
      // the superblock's activations first (64 scalar dwords per row), so their
      // latency overlaps the nibble unpacking below
      uint32_t av[MR][64];
#pragma unroll
      for (int m = 0; m < MR; ++m)
#pragma unroll
        for (int i = 0; i < 64; ++i) av[m][i] = A[m * a_row + kb * 64 + i];
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const uint32_t wd[4] = {wv[kq].x, wv[kq].y, wv[kq].z, wv[kq].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint32_t w = wd[t], w8 = w >> 8;
          const half2v e0 = exact(as_h2(and_or(w, MASK_E, EXP16)), OFS_E);
          const half2v o0 = exact(as_h2(and_or(w, MASK_O, EXP16)), OFS_O);
          const half2v e1 = exact(as_h2(and_or(w8, MASK_E, EXP16)), OFS_E);
          const half2v o1 = exact(as_h2(and_or(w8, MASK_O, EXP16)), OFS_O);
          const int base = kq * 16 + 4 * t;  // activation dword of positions 8t, 8t+1
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            accE[m] = __builtin_amdgcn_fdot2(e0, as_h2(av[m][base + 0]), accE[m], false);
            accO[m] = __builtin_amdgcn_fdot2(o0, as_h2(av[m][base + 1]), accO[m], false);
            accE[m] = __builtin_amdgcn_fdot2(e1, as_h2(av[m][base + 2]), accE[m], false);
            accO[m] = __builtin_amdgcn_fdot2(o1, as_h2(av[m][base + 3]), accO[m], false);
          }
        }
      }
      fold(accE, accO, as, sc);
    } else if constexpr (I4) {
      // exact per-element conversion, used when a superblock holds several groups
      constexpr uint32_t bias = (FMT == FMT_I4) ? 0x64086408u : 0x64006400u;  // 1032 or 1024
      const half2v hb = as_h2(bias);
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const uint32_t wd[4] = {wv[kq].x, wv[kq].y, wv[kq].z, wv[kq].w};
        const int k0 = kb * 128 + kq * 32;
        float pq[MR], pa[MR];
#pragma unroll
        for (int m = 0; m < MR; ++m) { pq[m] = 0.f; pa[m] = 0.f; }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t h = ((wd[t] >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
            const half2v q = as_h2(h) - hb;  // exact small integers
#pragma unroll
            for (int m = 0; m < MR; ++m) {
              const uint32_t av = A[m * a_row + (k0 >> 1) + 4 * t + j];
              pq[m] = __builtin_amdgcn_fdot2(q, as_h2(av), pq[m], false);
              if (FMT == FMT_U4 && a.zeros)
                pa[m] = __builtin_amdgcn_fdot2(as_h2(0x3C003C00u), as_h2(av), pa[m], false);
            }
          }
        float s, z;
        scale_of(k0 / a.group_size, s, z);
#pragma unroll
        for (int m = 0; m < MR; ++m) tot[m] += s * (pq[m] - z * pa[m]);
      }
    } else if constexpr (FMT == FMT_F16) {
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const uint32_t wd[4] = {wv[kq].x, wv[kq].y, wv[kq].z, wv[kq].w};
        const int k0 = kb * 32 + kq * 8;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            const uint32_t av = A[m * a_row + (k0 >> 1) + t];
            tot[m] = __builtin_amdgcn_fdot2(as_h2(wd[t]), as_h2(av), tot[m], false);
          }
      }
    } else if constexpr (FMT == FMT_I8) {
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const uint32_t wd[4] = {wv[kq].x, wv[kq].y, wv[kq].z, wv[kq].w};
        const int k0 = kb * 64 + kq * 16;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            const uint32_t av = A[m * a_row + (k0 >> 2) + t];
            tot[m] = __builtin_amdgcn_sdot4((int)wd[t], (int)av, tot[m], false);
          }
      }
    } else {  // FMT_I2
      int acc[4][MR];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[j][m] = 0;
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const uint32_t wd[4] = {wv[kq].x, wv[kq].y, wv[kq].z, wv[kq].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          // byte b of (w & mask_j) is position 4j + b scaled by 4^j; the top crumb is
          // stored two's complement, so its byte is exactly 64q as a signed int8
          const int q0 = (int)(wd[t] & 0x03030303u), q1 = (int)(wd[t] & 0x0C0C0C0Cu);
          const int q2 = (int)(wd[t] & 0x30303030u), q3 = (int)(wd[t] & 0xC0C0C0C0u);
          const int base = kq * 16 + 4 * t;
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            cptr Am = A + (m * a_row + kb * 64 + base);
            const uint4 a4 = make_uint4(Am[0], Am[1], Am[2], Am[3]);
            acc[0][m] = __builtin_amdgcn_sdot4(q0, (int)a4.x, acc[0][m], false);
            acc[1][m] = __builtin_amdgcn_sdot4(q1, (int)a4.y, acc[1][m], false);
            acc[2][m] = __builtin_amdgcn_sdot4(q2, (int)a4.z, acc[2][m], false);
            acc[3][m] = __builtin_amdgcn_sdot4(q3, (int)a4.w, acc[3][m], false);
          }
        }
      }
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        sacc[m] = __builtin_amdgcn_sdot4((int)as[m], ones012, sacc[m], false);
        tot[m] += acc[0][m] + (acc[1][m] >> 2) + (acc[2][m] >> 4) + (acc[3][m] >> 6);
      }
    }
  };

  // Several activation rows: the superblock's activations stream through the
  // scalar unit in 16-dword chunks (one piece of one row at a time), and each
  // chunk is requested right after the previous one has landed, so at most two
  // chunks occupy scalar registers whatever the number of rows (loading a whole
  // superblock for every row at once would overflow them).  Scalar loads can
  // complete out of order, hence the full lgkmcnt wait before each request.
  auto do_block_rows = [&](const uint4 (&wv)[4], const uint32_t (&as)[MR], uint32_t sc, int kb) {
    constexpr int NC = (FMT == FMT_F16 || FMT == FMT_I8) ? 1 : 4;  // chunks per row and superblock
    struct Chunk { uint32_t d[16]; };
    auto fetch = [&](int c, int m) {
      Chunk ch;
      uint32_t off = __builtin_amdgcn_readfirstlane(m * a_row + kb * A_DW_SB + c * 16);  // uniform
      // constant-space loads count as invariant and could be hoisted past the
      // wait below; passing the offset through an (empty) volatile asm pins
      // the request after it
      asm volatile("; chunk %0" : "+s"(off));
      cptr p = A + off;
#pragma unroll
      for (int i = 0; i < 16; ++i) ch.d[i] = p[i];
      return ch;
    };
    // runs body(c, m, chunk) over every (piece c, row m), prep(c) before the rows of piece c
    auto sweep = [&](auto&& prep, auto&& body) {
      Chunk cur = fetch(0, 0);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        prep(c);
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): cur has landed
          const bool more = !(c == NC - 1 && m == MR - 1);
          Chunk nxt;
          if (more) nxt = fetch(m == MR - 1 ? c + 1 : c, m == MR - 1 ? 0 : m + 1);
          __builtin_amdgcn_sched_barrier(0);
          body(c, m, cur);
          __builtin_amdgcn_sched_barrier(0);
          if (more) cur = nxt;
        }
      }
    };

    if constexpr (I4 && FOLD) {
      const uint32_t MASK_E = 0x000F000Fu, MASK_O = 0x00F000F0u, EXP16 = 0x64006400u;
      float accE[MR], accO[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) { accE[m] = 0.f; accO[m] = 0.f; }
      half2v e0[4], o0[4], e1[4], o1[4];
      sweep(
          [&](int c) {
            const uint32_t wd[4] = {wv[c].x, wv[c].y, wv[c].z, wv[c].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const uint32_t w = wd[t], w8 = w >> 8;
              e0[t] = exact(as_h2(and_or(w, MASK_E, EXP16)), OFS_E);
              o0[t] = exact(as_h2(and_or(w, MASK_O, EXP16)), OFS_O);
              e1[t] = exact(as_h2(and_or(w8, MASK_E, EXP16)), OFS_E);
              o1[t] = exact(as_h2(and_or(w8, MASK_O, EXP16)), OFS_O);
            }
          },
          [&](int c, int m, const Chunk& ch) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              accE[m] = __builtin_amdgcn_fdot2(e0[t], as_h2(ch.d[4 * t + 0]), accE[m], false);
              accO[m] = __builtin_amdgcn_fdot2(o0[t], as_h2(ch.d[4 * t + 1]), accO[m], false);
              accE[m] = __builtin_amdgcn_fdot2(e1[t], as_h2(ch.d[4 * t + 2]), accE[m], false);
              accO[m] = __builtin_amdgcn_fdot2(o1[t], as_h2(ch.d[4 * t + 3]), accO[m], false);
            }
          });
      fold(accE, accO, as, sc);
    } else if constexpr (I4) {
      constexpr uint32_t bias = (FMT == FMT_I4) ? 0x64086408u : 0x64006400u;  // 1032 or 1024
      const half2v hb = as_h2(bias);
      half2v qv[4][4];
      float gsv[4], gzv[4];  // scale (and zero point) of each piece's group
#pragma unroll
      for (int c = 0; c < 4; ++c) scale_of((kb * 128 + c * 32) / a.group_size, gsv[c], gzv[c]);
      float pq[MR], pa[MR];
      sweep(
          [&](int c) {
            const uint32_t wd[4] = {wv[c].x, wv[c].y, wv[c].z, wv[c].w};
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
              for (int j = 0; j < 4; ++j) qv[t][j] = as_h2(((wd[t] >> (4 * j)) & 0x000F000Fu) | 0x64006400u) - hb;
          },
          [&](int c, int m, const Chunk& ch) {
            pq[m] = 0.f;
            pa[m] = 0.f;
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                pq[m] = __builtin_amdgcn_fdot2(qv[t][j], as_h2(ch.d[4 * t + j]), pq[m], false);
                if (FMT == FMT_U4 && a.zeros)
                  pa[m] = __builtin_amdgcn_fdot2(as_h2(0x3C003C00u), as_h2(ch.d[4 * t + j]), pa[m], false);
              }
            tot[m] += gsv[c] * (pq[m] - gzv[c] * pa[m]);
          });
    } else if constexpr (FMT == FMT_F16 || FMT == FMT_I8) {
      sweep([](int) {},
            [&](int, int m, const Chunk& ch) {
#pragma unroll
              for (int kq = 0; kq < 4; ++kq) {
                const uint32_t wd[4] = {wv[kq].x, wv[kq].y, wv[kq].z, wv[kq].w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                  if constexpr (FMT == FMT_F16)
                    tot[m] = __builtin_amdgcn_fdot2(as_h2(wd[t]), as_h2(ch.d[kq * 4 + t]), tot[m], false);
                  else
                    tot[m] = __builtin_amdgcn_sdot4((int)wd[t], (int)ch.d[kq * 4 + t], tot[m], false);
                }
              }
            });
    } else {  // FMT_I2
      int acc[4][MR];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[j][m] = 0;
      int q[4][4];
      sweep(
          [&](int c) {
            const uint32_t wd[4] = {wv[c].x, wv[c].y, wv[c].z, wv[c].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              q[t][0] = (int)(wd[t] & 0x03030303u);
              q[t][1] = (int)(wd[t] & 0x0C0C0C0Cu);
              q[t][2] = (int)(wd[t] & 0x30303030u);
              q[t][3] = (int)(wd[t] & 0xC0C0C0C0u);
            }
          },
          [&](int, int m, const Chunk& ch) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                acc[j][m] = __builtin_amdgcn_sdot4(q[t][j], (int)ch.d[4 * t + j], acc[j][m], false);
          });
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        sacc[m] = __builtin_amdgcn_sdot4((int)as[m], ones012, sacc[m], false);
        tot[m] += acc[0][m] + (acc[1][m] >> 2) + (acc[2][m] >> 4) + (acc[3][m] >> 6);
      }
    }
  };

  auto block = [&](const uint4 (&wv)[4], const uint32_t (&as)[MR], uint32_t sc, int kb) {
    if constexpr (MR == 1) do_block(wv, as, sc, kb);
    else do_block_rows(wv, as, sc, kb);
  };

  // Two register stages (one for int8 / fp16 at M = 1): the loads of the next UNR
  // superblocks fly while these are consumed.
  Stage s0, s1;
  // keeps the machine scheduler from sinking a stage's loads below the block
  // code that follows them, which it does for the unscaled int4 variant (draining
  // the prefetch); the other variants are scheduled better without it
  auto fence = [] {
    if constexpr (I4 && VAR == 0) __builtin_amdgcn_sched_barrier(0);
  };
  auto consume = [&](const Stage& s, int j) {
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      if (j + u < cnt) block(s.w[u], s.as[u], s.sc[u], row_of(j + u));
  };
  if constexpr (MR == 1 && (FMT == FMT_I8 || FMT == FMT_F16)) {
    // One superblock in flight per wave: the int8 and fp16 blocks are light enough
    // that the other waves of the SIMD keep loads going while one computes, and
    // this measured faster than a prefetched stage (1.3 us at int8 and 2.5 us at
    // fp16 for N = K = 16384).
    for (int j = 0; j < cnt; j += UNR) {
      load(s0, j);
      consume(s0, j);
    }
  } else if constexpr (MR == 1 && !I4) {
    // The steady loop runs while two more stages remain, so it never loads past
    // the wave's rows; the last one or two stages follow it (faster for the
    // int2 blocks, whose code can be repeated).
    if (cnt > 0) {
      int j = 0;
      load(s0, 0);
      for (; j + 2 * UNR < cnt; j += 2 * UNR) {
        load(s1, j + UNR);
        fence();
        consume(s0, j);
        load(s0, j + 2 * UNR);
        fence();
        consume(s1, j + UNR);
      }
      if (j + UNR < cnt) {
        load(s1, j + UNR);
        fence();
        consume(s0, j);
        consume(s1, j + UNR);
      } else {
        consume(s0, j);
      }
    }
  } else {
    // one copy of each stage's block code: the last stage loads a clamped copy
    // of the wave's last superblock that is never used
    int j = 0;
    if (j < cnt) load(s0, j);
    while (j < cnt) {
      load(s1, j + UNR);
      fence();
      consume(s0, j);
      j += UNR;
      if (j >= cnt) break;
      load(s0, j + UNR);
      fence();
      consume(s1, j);
      j += UNR;
    }
  }

  if constexpr (FMT == FMT_I2) {
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      // classes 0..2 are offset-binary (q + 2): subtract 2 * (their activation sum)
      const int h = half_wave_sums(sacc[m]);
      tot[m] -= 2 * (lane_value(h, 31) + lane_value(h, 63));
    }
  }

  // block reduction across the waves of the workgroup
  __shared__ acc_t red[GEMV_MAX_WAVES][MR][64];
#pragma unroll
  for (int m = 0; m < MR; ++m) red[wave][m][lane] = tot[m];
  __syncthreads();
  for (int idx = threadIdx.x; idx < MR * 64; idx += blockDim.x) {
    const int m = idx >> 6, ln = idx & 63;
    acc_t s = 0;
    for (int w = 0; w < a.waves; ++w) s += red[w][m][ln];
    const int col = rb * 64 + ln;
    if (col >= a.N) continue;
    const size_t o = (size_t)m * a.N + col;
    if (a.out_mode == OUT_STORE) {
      if constexpr (FP) static_cast<_Float16*>(a.C)[o] = (_Float16)(s + bias_f(a, col));
      else if (a.row_scale) static_cast<_Float16*>(a.C)[o] = dq_out(a, m, col, s);
      else static_cast<int*>(a.C)[o] = s + bias_i(a, col);
    } else if (a.out_mode == OUT_ATOMIC) {
      if constexpr (FP) unsafeAtomicAdd(static_cast<float*>(a.ws) + o, s);
      else atomicAdd(int_atomic_target(a) + o, s);
    } else {
      static_cast<acc_t*>(a.ws)[(size_t)part * a.M * a.N + o] = s;
    }
  }
}

template <int FMT, int VAR>
hipError_t launch_fmt(const RunArgs& a, hipStream_t st) {
  dim3 grid((a.N + 63) / 64, a.k_parts), block(64 * a.waves);
  switch (a.M) {
#define QG_CASE(R) \
  case R: hipLaunchKernelGGL((gemv_kernel<FMT, R, VAR>), grid, block, 0, st, a); break;
    QG_CASE(1) QG_CASE(2) QG_CASE(3) QG_CASE(4) QG_CASE(5) QG_CASE(6) QG_CASE(7) QG_CASE(8)
#undef QG_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(int fmt, const RunArgs& a, hipStream_t st) {
  const int var = a.smode == SC_PIECE ? 3 : a.smode == SC_NONE ? 0 : a.zeros ? 2 : 1;
  switch (fmt) {
    case FMT_I4:
      return var == 3 ? launch_fmt<FMT_I4, 3>(a, st) : var == 0 ? launch_fmt<FMT_I4, 0>(a, st)
                                                               : launch_fmt<FMT_I4, 1>(a, st);
    case FMT_U4:
      return var == 3 ? launch_fmt<FMT_U4, 3>(a, st) : var == 0 ? launch_fmt<FMT_U4, 0>(a, st)
           : var == 1 ? launch_fmt<FMT_U4, 1>(a, st) : launch_fmt<FMT_U4, 2>(a, st);
    case FMT_F16: return launch_fmt<FMT_F16, 0>(a, st);
    case FMT_I8: return launch_fmt<FMT_I8, 0>(a, st);
    case FMT_I2: return launch_fmt<FMT_I2, 0>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
