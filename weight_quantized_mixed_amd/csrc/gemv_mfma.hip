// Skinny-M int8 / int2 / fp16 path on the matrix cores (M <= 32).
//
// The packed blob already holds every 16-column superblock in the lane order of
// a gfx950 16x16 MFMA B operand (lane l: column l % 16, K group l / 16), so one
// wave-wide 16-byte load of a superblock is an MFMA operand as it stands
// (int8), or four of them after masking (int2): no LDS, no transposition.  A
// workgroup owns CB superblock columns (16, 32 or 64 columns: the most that
// still gives the CUs enough workgroups; each activation load then serves CB
// MFMAs) and a k-part; its waves take the part's superblock rows in turn (as the
// VALU GEMV does) and meet in LDS at the end.  The activation rows ride in the A operand: lane l loads the
// K group l / 16 of row l % 16 (rows past M repeat row M - 1, and their results
// are dropped), so up to 16 rows cost the same instructions as one; a second row
// block of 16 reuses every B operand.
//
// int8: one v_mfma_i32_16x16x64_i8 per superblock and column block; fp16 the same
// with v_mfma_f32_16x16x32_f16 (a 32-position superblock, fp32 accumulation).
// int2: word t of piece g holds positions 64 g + 16 t + 4 j + b (class j, byte b);
// masking word t with 0x03, 0x0C, 0x30 or 0xC0 per byte keeps class j as the byte
// value 4^j c (the top class two's complement, so 64 q as a signed byte), and the
// four masked words of a piece are the B operand of class j.  The matching A
// operand is dword 4 t + j of the lane's 64-byte activation slice, a choice of
// registers.  Classes 0-2 are offset-binary (c = q + 2): one more MFMA per class
// against a B of ones gives the activation sums that the correction subtracts.
// Per word this is four VALU masks, where the dot-product GEMV needs four masks
// and four dot products.
#include <type_traits>

#include "qgemm_internal.hpp"

namespace qg {
namespace {

typedef int int4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u t = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ int4v as_i4(const uint4& v) { return int4v{(int)v.x, (int)v.y, (int)v.z, (int)v.w}; }

// one 16-byte load as a vector (kept whole)
__device__ __forceinline__ uint4 load16(const uint4* p) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u t = *reinterpret_cast<const v4u*>(p);
  return make_uint4(t.x, t.y, t.z, t.w);
}

// a register copy the compiler cannot fold into a vector shuffle (which it lowers
// through scratch memory when building the transposed activation operands): an
// identity DPP move, which unlike inline assembly stays visible to the pass that
// inserts the wait states between a VALU write and the MFMA that reads it
__device__ __forceinline__ int mv(uint32_t x) { return __builtin_amdgcn_mov_dpp((int)x, 0xE4, 0xF, 0xF, false); }

__device__ __forceinline__ int4v masked(const uint4& w, uint32_t m) {
  return int4v{(int)(w.x & m), (int)(w.y & m), (int)(w.z & m), (int)(w.w & m)};
}

__device__ __forceinline__ int4v shifted_masked(const uint4& w, int sh, uint32_t m) {
  return int4v{(int)((w.x >> sh) & m), (int)((w.y >> sh) & m), (int)((w.z >> sh) & m), (int)((w.w >> sh) & m)};
}

__device__ __forceinline__ int4v mfma(const int4v& A, const int4v& B, const int4v& C) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(A, B, C, 0, 0, 0);
}

// fp16 weights: 16x16x32 with fp32 accumulation
__device__ __forceinline__ float4v mfma(const int4v& A, const int4v& B, const float4v& C) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8v, A), __builtin_bit_cast(half8v, B), C, 0, 0, 0);
}

// MB row blocks of 16 (M <= 16 MB)
template <int FMT, int MB, int CB>
__global__ __launch_bounds__(64 * GEMV_MAX_WAVES) void gemv_mfma_kernel(RunArgs a) {
  constexpr bool I2 = FMT == FMT_I2, FP = FMT == FMT_F16;
  constexpr int KB = kb_of(FMT);   // positions per superblock: 256 (int2), 64 (int8), 32 (fp16)
  constexpr int ESZ = FP ? 2 : 1;  // activation bytes
  constexpr int AV = KB * ESZ / 64;  // 16-byte activation vectors per lane and superblock
  typedef typename std::conditional<FP, float4v, int4v>::type acc_v;
  typedef typename std::conditional<FP, float, int>::type acc_t;
  // accumulators per column block: int2 keeps the four classes apart (values 4^j c)
  // with one row block; with two (registers) it shifts classes 1 and 2 down to c
  // and sums classes 0-2 in one accumulator, the two's complement class in another
  constexpr int NC = !I2 ? 1 : MB == 1 ? 4 : 2;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rb = blockIdx.x, part = blockIdx.y;
  const int g = lane >> 4, r16 = lane & 15;

  int u0, u1;
  part_units(a, part, u0, u1);
  const int kb0 = u0 * a.unit_kb, kb1 = u1 * a.unit_kb;
  // superblock rows of this wave, in turn with the other waves (wave-uniform)
  const int cnt = __builtin_amdgcn_readfirstlane(kb1 - kb0 > wave ? (kb1 - kb0 - wave + a.waves - 1) / a.waves : 0);
  auto row_of = [&](int j) { return __builtin_amdgcn_readfirstlane(kb0 + wave + j * a.waves); };

  const uint4* __restrict__ Wl = a.W + (size_t)rb * CB * 64 + lane;  // column block rb*CB + cb at + cb*64
  const uint32_t sb_stride = (uint32_t)a.NB * 64u;                   // uint4 per superblock row
  // this lane's activation slice: row r16, K group g of each superblock.  Lanes of
  // rows past M read row M - 1 (results dropped): the loads stay unconditional,
  // since masking them off makes the compiler drain every load in flight at the
  // end of the masked block.
  const uint4* __restrict__ Al[MB];
#pragma unroll
  for (int r = 0; r < MB; ++r)
    Al[r] = reinterpret_cast<const uint4*>(static_cast<const int8_t*>(a.A) +
                                           (size_t)min(r * 16 + r16, a.M - 1) * a.K * ESZ) +
            g * AV;

  // A is loaded before the weights, so that waiting for a stage's activations
  // never waits for the weight loads of the stage after it
  struct Stage {
    uint4 av[MB][AV];
    uint4 w[CB];
  };
  auto load = [&](Stage& s, int j) {
    const uint32_t kb = (uint32_t)row_of(min(j, cnt - 1));
#pragma unroll
    for (int r = 0; r < MB; ++r)
#pragma unroll
      for (int i = 0; i < AV; ++i) s.av[r][i] = load16(Al[r] + kb * (KB * ESZ / 16) + i);
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) s.w[cb] = stream_load(Wl + kb * sb_stride + cb * 64);
  };

  acc_v acc[MB][CB][NC];
  int4v accS[MB];  // int2: activation sums of classes 0-2
#pragma unroll
  for (int r = 0; r < MB; ++r) {
    accS[r] = int4v{0, 0, 0, 0};
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[r][cb][c] = acc_v{0, 0, 0, 0};
  }

  auto consume = [&](const Stage& s) {
#pragma unroll
    for (int r = 0; r < MB; ++r) {
      if constexpr (I2) {
        // the A operand of class j takes dword 4 t + j of the lane's 64-byte slice as
        // its dword t
        int4v A[4];
        A[0] = int4v{mv(s.av[r][0].x), mv(s.av[r][1].x), mv(s.av[r][2].x), mv(s.av[r][3].x)};
        A[1] = int4v{mv(s.av[r][0].y), mv(s.av[r][1].y), mv(s.av[r][2].y), mv(s.av[r][3].y)};
        A[2] = int4v{mv(s.av[r][0].z), mv(s.av[r][1].z), mv(s.av[r][2].z), mv(s.av[r][3].z)};
        A[3] = int4v{mv(s.av[r][0].w), mv(s.av[r][1].w), mv(s.av[r][2].w), mv(s.av[r][3].w)};
        if constexpr (NC == 4) {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) {
            const uint4 w = s.w[cb];
            acc[r][cb][0] = mfma(A[0], masked(w, 0x03030303u), acc[r][cb][0]);
            acc[r][cb][1] = mfma(A[1], masked(w, 0x0C0C0C0Cu), acc[r][cb][1]);
            acc[r][cb][2] = mfma(A[2], masked(w, 0x30303030u), acc[r][cb][2]);
            acc[r][cb][3] = mfma(A[3], masked(w, 0xC0C0C0C0u), acc[r][cb][3]);
          }
        } else {
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[r][cb][0] = mfma(A[0], masked(s.w[cb], 0x03030303u), acc[r][cb][0]);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[r][cb][0] = mfma(A[1], shifted_masked(s.w[cb], 2, 0x03030303u), acc[r][cb][0]);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb)
            acc[r][cb][0] = mfma(A[2], shifted_masked(s.w[cb], 4, 0x03030303u), acc[r][cb][0]);
#pragma unroll
          for (int cb = 0; cb < CB; ++cb) acc[r][cb][1] = mfma(A[3], masked(s.w[cb], 0xC0C0C0C0u), acc[r][cb][1]);
        }
        const int4v ones = int4v{0x01010101, 0x01010101, 0x01010101, 0x01010101};
        accS[r] = mfma(A[0], ones, accS[r]);
        accS[r] = mfma(A[1], ones, accS[r]);
        accS[r] = mfma(A[2], ones, accS[r]);
      } else {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb) acc[r][cb][0] = mfma(as_i4(s.av[r][0]), as_i4(s.w[cb]), acc[r][cb][0]);
      }
    }
  };

  // two register stages; the steady loop never loads past the wave's rows.  The
  // fences keep each stage's loads ahead of the other stage's MFMAs, so that the
  // wait for one stage never covers the loads of the next.
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

  // lane l holds rows 16 rb + 4 (l / 16) + i of column l % 16 of each column block;
  // the waves meet in LDS
  __shared__ acc_t red[GEMV_MAX_WAVES][MB][CB][4][64];
#pragma unroll
  for (int r = 0; r < MB; ++r)
#pragma unroll
    for (int cb = 0; cb < CB; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc_t v = acc[r][cb][0][i];
        if constexpr (NC == 4)  // classes 0..2 are offset-binary (q + 2)
          v += (acc[r][cb][1][i] >> 2) + (acc[r][cb][2][i] >> 4) + (acc[r][cb][3][i] >> 6) - 2 * accS[r][i];
        else if constexpr (NC == 2)
          v += (acc[r][cb][1][i] >> 6) - 2 * accS[r][i];
        red[wave][r][cb][i][lane] = v;
      }
  __syncthreads();
  for (int idx = threadIdx.x; idx < MB * CB * 4 * 64; idx += blockDim.x) {
    const int r = idx / (CB * 256), cb = (idx >> 8) % CB, i = (idx >> 6) & 3, ln = idx & 63;
    const int row = r * 16 + 4 * (ln >> 4) + i, col = (rb * CB + cb) * 16 + (ln & 15);
    if (row >= a.M || col >= a.N) continue;
    acc_t s = 0;
    for (int w = 0; w < a.waves; ++w) s += red[w][r][cb][i][ln];
    const size_t o = (size_t)row * a.N + col;
    if constexpr (FP) {
      if (a.out_mode == OUT_STORE) static_cast<_Float16*>(a.C)[o] = (_Float16)(s + bias_f(a, col));
      else if (a.out_mode == OUT_ATOMIC) unsafeAtomicAdd(static_cast<float*>(a.ws) + o, s);
      else static_cast<float*>(a.ws)[(size_t)part * a.M * a.N + o] = s;
    } else {
      if (a.out_mode == OUT_STORE) {
        if (a.row_scale) static_cast<_Float16*>(a.C)[o] = dq_out(a, row, col, s);
        else static_cast<int*>(a.C)[o] = s + bias_i(a, col);
      } else if (a.out_mode == OUT_ATOMIC) {
        atomicAdd(int_atomic_target(a) + o, s);
      } else {
        static_cast<int*>(a.ws)[(size_t)part * a.M * a.N + o] = s;
      }
    }
  }
}

template <int FMT, int MB, int CB>
void launch_cb(const RunArgs& a, hipStream_t st) {
  const dim3 grid((a.N + 16 * CB - 1) / (16 * CB), a.k_parts), block(64 * a.waves);
  hipLaunchKernelGGL((gemv_mfma_kernel<FMT, MB, CB>), grid, block, 0, st, a);
}

template <int FMT, int MB>
hipError_t launch_mb(const RunArgs& a, hipStream_t st) {
  switch (a.gemv_cb) {
    case 1: launch_cb<FMT, MB, 1>(a, st); break;
    case 2: launch_cb<FMT, MB, 2>(a, st); break;
    case 4: launch_cb<FMT, MB, 4>(a, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_mfma(int fmt, const RunArgs& a, hipStream_t st) {
  if (a.M < 1 || a.M > 32) return hipErrorInvalidValue;
  const bool two = a.M > 16;
  if (fmt == FMT_I8) return two ? launch_mb<FMT_I8, 2>(a, st) : launch_mb<FMT_I8, 1>(a, st);
  if (fmt == FMT_I2) return two ? launch_mb<FMT_I2, 2>(a, st) : launch_mb<FMT_I2, 1>(a, st);
  if (fmt == FMT_F16) return two ? launch_mb<FMT_F16, 2>(a, st) : launch_mb<FMT_F16, 1>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace qg
