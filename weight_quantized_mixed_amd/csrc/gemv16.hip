// Narrow skinny-M path (M = 1 when the matrix has fewer than 128 blocks of 64
// columns): a workgroup owns 16 output columns (one superblock column) and lane
// l takes piece l of every superblock -- K quarter l / 16, column l % 16, the
// blob's own piece order -- so a superblock is a single wave-wide 16-byte load
// and four times as many workgroups share the CUs as with one 64-column block
// per workgroup.  The waves take the part's superblock rows in turn; every lane
// accumulates its quarter, and the four quarters and the waves of a column meet
// in LDS at the end (the intra-workgroup block reduction of the BitBLAS issue
// #252 discussion).
//
// Each lane needs the activations of its own quarter (32 positions for int4,
// 64 for int2, 16 for int8, 8 for fp16), loaded as vectors beside the weights.
// int4 is converted exactly in registers (or-ing 0x6400, subtracting the bias
// and the zero point in fp16, as the MFMA path does) and dotted with
// v_dot2_f32_f16; the group scale multiplies the piece's partial sum, so group
// sizes 32 and 64 (one or two pieces per group) need no special case.  int2 is
// masked in place (byte values c, 4c, 16c and the two's complement top crumb as
// 64q) and corrected by the lane's own sum of the offset-binary classes.
#include "qgemm_internal.hpp"

namespace qg {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }
__device__ __forceinline__ float h2f(uint32_t x) { return (float)__builtin_bit_cast(_Float16, (uint16_t)x); }

__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

// VAR: 0 unscaled, 1 scaled, 2 scaled with zero points (int4 formats only)
template <int FMT, int VAR>
__global__ __launch_bounds__(64 * GEMV_MAX_WAVES) void gemv16_kernel(RunArgs a) {
  constexpr bool FP = (FMT == FMT_I4 || FMT == FMT_U4 || FMT == FMT_F16);
  constexpr bool I4 = (FMT == FMT_I4 || FMT == FMT_U4);
  constexpr bool SCALED = VAR >= 1, ZEROS = VAR == 2;
  constexpr int KB = kb_of(FMT);
  constexpr int PQ = KB / 4;                       // positions per piece
  constexpr int ADW = FP ? PQ / 2 : PQ / 4;        // activation dwords per piece (16 or 4)
  constexpr int AV = ADW / 4;                      // ... as 16-byte vectors
  constexpr int A_DW_SB = FP ? KB / 2 : KB / 4;    // activation dwords per superblock
  typedef typename std::conditional<FP, float, int>::type acc_t;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = blockIdx.x, part = blockIdx.y;
  const int kq = lane >> 4;
  const int n = nb * 16 + (lane & 15);

  int u0, u1;
  part_units(a, part, u0, u1);
  const int kb0 = u0 * a.unit_kb, kb1 = u1 * a.unit_kb;
  // superblock rows of this wave, in turn with the other waves (wave-uniform)
  const int cnt = __builtin_amdgcn_readfirstlane(kb1 - kb0 > wave ? (kb1 - kb0 - wave + a.waves - 1) / a.waves : 0);
  auto row_of = [&](int j) { return __builtin_amdgcn_readfirstlane(kb0 + wave + j * a.waves); };

  const uint4* __restrict__ Wl = a.W + (size_t)nb * 64 + lane;
  const uint32_t sb_stride = (uint32_t)a.NB * 64u;  // uint4 per superblock row
  const uint4* __restrict__ Al = reinterpret_cast<const uint4*>(static_cast<const uint32_t*>(a.A) + kq * ADW);

  struct Stage {
    uint4 w;
    uint4 av[AV];
    uint32_t sc;  // raw scale (or scale | zero << 16) of the piece's group
  };
  auto load = [&](Stage& s, int j) {
    const uint32_t kb = (uint32_t)row_of(min(j, cnt - 1));
    s.w = stream_load(Wl + kb * sb_stride);
#pragma unroll
    for (int i = 0; i < AV; ++i) s.av[i] = Al[(kb * A_DW_SB) / 4 + i];
    if constexpr (SCALED) {
      const int pos = (int)kb * KB + kq * PQ;
      const uint32_t grp = a.group_size > 0 ? (uint32_t)(pos / a.group_size) : 0u;
      if constexpr (ZEROS) s.sc = static_cast<const uint32_t*>(a.S)[grp * (uint32_t)a.Npad + n];
      else s.sc = static_cast<const uint16_t*>(a.S)[grp * (uint32_t)a.Npad + n];
    } else {
      s.sc = 0;
    }
  };

  acc_t tot = 0;
  int acc2[4] = {0, 0, 0, 0}, s012 = 0;  // int2: class accumulators and offset-binary sum

  auto consume = [&](const Stage& s) {
    const uint32_t wd[4] = {s.w.x, s.w.y, s.w.z, s.w.w};
    if constexpr (I4) {
      constexpr uint32_t bias = (FMT == FMT_I4) ? 0x64086408u : 0x64006400u;  // 1032 or 1024
      const uint32_t zz = ZEROS ? (s.sc >> 16) * 0x10001u : 0u;
      float p = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t ad[4] = {s.av[t].x, s.av[t].y, s.av[t].z, s.av[t].w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          // slots jj and jj + 4 of word t hold positions 8t + 2jj and 8t + 2jj + 1
          half2v q = as_h2(and_or(wd[t] >> (4 * jj), 0x000F000Fu, 0x64006400u)) - as_h2(bias);
          if constexpr (ZEROS) q = q - as_h2(zz);
          p = __builtin_amdgcn_fdot2(q, as_h2(ad[jj]), p, false);
        }
      }
      tot += SCALED ? h2f(s.sc & 0xFFFFu) * p : p;
    } else if constexpr (FMT == FMT_I2) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        // word t holds positions 16t..16t+15; class j = positions 16t + 4j .. + 3
        const uint32_t ad[4] = {s.av[t].x, s.av[t].y, s.av[t].z, s.av[t].w};
        acc2[0] = __builtin_amdgcn_sdot4((int)(wd[t] & 0x03030303u), (int)ad[0], acc2[0], false);
        acc2[1] = __builtin_amdgcn_sdot4((int)(wd[t] & 0x0C0C0C0Cu), (int)ad[1], acc2[1], false);
        acc2[2] = __builtin_amdgcn_sdot4((int)(wd[t] & 0x30303030u), (int)ad[2], acc2[2], false);
        acc2[3] = __builtin_amdgcn_sdot4((int)(wd[t] & 0xC0C0C0C0u), (int)ad[3], acc2[3], false);
#pragma unroll
        for (int j = 0; j < 3; ++j) s012 = __builtin_amdgcn_sdot4((int)ad[j], 0x01010101, s012, false);
      }
    } else if constexpr (FMT == FMT_I8) {
      const uint32_t ad[4] = {s.av[0].x, s.av[0].y, s.av[0].z, s.av[0].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) tot = __builtin_amdgcn_sdot4((int)wd[t], (int)ad[t], tot, false);
    } else {  // FMT_F16
      const uint32_t ad[4] = {s.av[0].x, s.av[0].y, s.av[0].z, s.av[0].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) tot = __builtin_amdgcn_fdot2(as_h2(wd[t]), as_h2(ad[t]), tot, false);
    }
  };

  // two register stages; the steady loop never loads past the wave's rows
  Stage s0, s1;
  if (cnt > 0) {
    int j = 0;
    load(s0, 0);
    for (; j + 2 < cnt; j += 2) {
      load(s1, j + 1);
      consume(s0);
      load(s0, j + 2);
      consume(s1);
    }
    if (j + 1 < cnt) {
      load(s1, j + 1);
      consume(s0);
      consume(s1);
    } else {
      consume(s0);
    }
  }
  if constexpr (FMT == FMT_I2)  // classes 0..2 are offset-binary (q + 2)
    tot = acc2[0] + (acc2[1] >> 2) + (acc2[2] >> 4) + (acc2[3] >> 6) - 2 * s012;

  // the four quarters of each column and the waves meet in LDS
  __shared__ acc_t red[GEMV_MAX_WAVES][64];
  red[wave][lane] = tot;
  __syncthreads();
  if (threadIdx.x < 16) {
    const int col = nb * 16 + threadIdx.x;
    acc_t s = 0;
    for (int w = 0; w < a.waves; ++w)
#pragma unroll
      for (int q = 0; q < 4; ++q) s += red[w][q * 16 + threadIdx.x];
    if (col < a.N) {
      if (a.out_mode == OUT_STORE) {
        if constexpr (FP) static_cast<_Float16*>(a.C)[col] = (_Float16)(s + bias_f(a, col));
        else if (a.row_scale) static_cast<_Float16*>(a.C)[col] = dq_out(a, 0, col, s);
        else static_cast<int*>(a.C)[col] = s + bias_i(a, col);
      } else if (a.out_mode == OUT_ATOMIC) {
        if constexpr (FP) unsafeAtomicAdd(static_cast<float*>(a.ws) + col, s);
        else atomicAdd(int_atomic_target(a) + col, s);
      } else {
        static_cast<acc_t*>(a.ws)[(size_t)part * a.N + col] = s;
      }
    }
  }
}

template <int FMT, int VAR>
hipError_t launch16(const RunArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((gemv16_kernel<FMT, VAR>), dim3((a.N + 15) / 16, a.k_parts), dim3(64 * a.waves), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv16(int fmt, const RunArgs& a, hipStream_t st) {
  if (a.M != 1) return hipErrorInvalidValue;
  const int var = a.smode == SC_NONE ? 0 : a.zeros ? 2 : 1;
  switch (fmt) {
    case FMT_I4: return var == 0 ? launch16<FMT_I4, 0>(a, st) : launch16<FMT_I4, 1>(a, st);
    case FMT_U4:
      return var == 0 ? launch16<FMT_U4, 0>(a, st) : var == 1 ? launch16<FMT_U4, 1>(a, st) : launch16<FMT_U4, 2>(a, st);
    case FMT_F16: return launch16<FMT_F16, 0>(a, st);
    case FMT_I8: return launch16<FMT_I8, 0>(a, st);
    case FMT_I2: return launch16<FMT_I2, 0>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
