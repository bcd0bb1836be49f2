// Skinny-M path (M <= 8): wavefront dot products straight from HBM, no matrix cores.
//
// Each workgroup owns 64 output columns (four 16-column superblock columns)
// and one k-part; its waves split the part's superblocks into contiguous runs
// and meet in LDS at the end (the intra-workgroup "block reduction" whose
// absence the BitBLAS issue #252 split-K discussion blames for the slow
// M = 32/128 dequantised rows).  Lane l owns column n = 64*rb + l: for every
// superblock it loads the four 16-byte pieces of its column (one wave-wide load
// per quarter reads 4 x 256 contiguous bytes), unpacks them in registers (the
// packed-upcast trick of hidet issue #364) and dots them with the activation
// slice.  All lanes of a wave need the same activations, so A is read through
// the scalar unit (constant address space) and never occupies vector memory
// bandwidth.  k-parts > 1 reduce across workgroups with global atomics or a
// two-pass partial store (hidet issue #364, parallel-k with atomic reduction).
#include "qgemm_internal.hpp"

namespace qg {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(4))) uint32_t* cptr;

__device__ __forceinline__ half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }
__device__ __forceinline__ float h2f(uint16_t x) { return (float)__builtin_bit_cast(_Float16, x); }

template <int FMT, int MR>
__global__ __launch_bounds__(1024) void gemv_kernel(RunArgs a) {
  constexpr bool FP = (FMT == FMT_I4 || FMT == FMT_U4 || FMT == FMT_F16);
  typedef typename std::conditional<FP, float, int>::type acc_t;
  constexpr int KB = kb_of(FMT);
  // dwords of A per row: fp16 -> K/2, int8 -> K/4
  const int a_row_dw = FP ? a.K / 2 : a.K / 4;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int rb = blockIdx.x, part = blockIdx.y;
  const int n = rb * 64 + lane;

  const int u0 = (int)((int64_t)part * a.n_units / a.k_parts);
  const int u1 = (int)((int64_t)(part + 1) * a.n_units / a.k_parts);
  const int kb0 = u0 * a.unit_kb, kb1 = u1 * a.unit_kb;
  const int per = (kb1 - kb0 + a.waves - 1) / a.waves;
  const int my0 = min(kb0 + wave * per, kb1);
  const int my1 = min(my0 + per, kb1);

  cptr A = (cptr)a.A;
  const uint4* __restrict__ Wl = a.W + (size_t)(rb * 4 + (lane >> 4)) * 64 + (lane & 15);
  const size_t sb_stride = (size_t)a.NB * 64;  // uint4 per superblock row (kb)

  acc_t tot[MR];
#pragma unroll
  for (int m = 0; m < MR; ++m) tot[m] = 0;

  auto do_block = [&](const uint4 (&wv)[4], int kb) {
    if constexpr (FMT == FMT_I4 || FMT == FMT_U4) {
      constexpr uint32_t bias = (FMT == FMT_I4) ? 0x64086408u : 0x64006400u;  // 1032 or 1024
      const half2v hb = as_h2(bias);
      float pq[MR], pa[MR];
#pragma unroll
      for (int m = 0; m < MR; ++m) { pq[m] = 0.f; pa[m] = 0.f; }
      auto flush = [&](int grp) {
        if (a.smode == SC_NONE) {
#pragma unroll
          for (int m = 0; m < MR; ++m) tot[m] += pq[m];
        } else if (a.zeros) {
          const uint32_t sz = static_cast<const uint32_t*>(a.S)[(size_t)grp * a.Npad + n];
          const float s = h2f((uint16_t)(sz & 0xFFFF)), z = h2f((uint16_t)(sz >> 16));
#pragma unroll
          for (int m = 0; m < MR; ++m) tot[m] += s * (pq[m] - z * pa[m]);
        } else {
          const float s = h2f(static_cast<const uint16_t*>(a.S)[(size_t)grp * a.Npad + n]);
#pragma unroll
          for (int m = 0; m < MR; ++m) tot[m] += s * pq[m];
        }
#pragma unroll
        for (int m = 0; m < MR; ++m) { pq[m] = 0.f; pa[m] = 0.f; }
      };
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const uint32_t wd[4] = {wv[kq].x, wv[kq].y, wv[kq].z, wv[kq].w};
        const int k0 = kb * 128 + kq * 32;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t h = ((wd[t] >> (4 * j)) & 0x000F000Fu) | 0x64006400u;
            const half2v q = as_h2(h) - hb;  // exact small integers
#pragma unroll
            for (int m = 0; m < MR; ++m) {
              const uint32_t av = A[(size_t)m * a_row_dw + (k0 >> 1) + 4 * t + j];
              pq[m] = __builtin_amdgcn_fdot2(q, as_h2(av), pq[m], false);
              if (FMT == FMT_U4 && a.zeros)
                pa[m] = __builtin_amdgcn_fdot2(as_h2(0x3C003C00u), as_h2(av), pa[m], false);
            }
          }
        }
        if (a.smode == SC_PIECE) flush(k0 / a.group_size);
      }
      if (a.smode != SC_PIECE) flush(a.group_size > 0 ? (kb * 128) / a.group_size : 0);
    } else if constexpr (FMT == FMT_F16) {
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const uint32_t wd[4] = {wv[kq].x, wv[kq].y, wv[kq].z, wv[kq].w};
        const int k0 = kb * 32 + kq * 8;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int m = 0; m < MR; ++m) {
            const uint32_t av = A[(size_t)m * a_row_dw + (k0 >> 1) + t];
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
            const uint32_t av = A[(size_t)m * a_row_dw + (k0 >> 2) + t];
            tot[m] = __builtin_amdgcn_sdot4((int)wd[t], (int)av, tot[m], false);
          }
      }
    } else {  // FMT_I2
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const uint32_t wd[4] = {wv[kq].x, wv[kq].y, wv[kq].z, wv[kq].w};
        const int k0 = kb * 256 + kq * 64;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            // offset-binary crumbs 0..3 -> signed bytes -2..1 through a byte-permute table
            const uint32_t sel = (wd[t] >> (2 * j)) & 0x03030303u;
            const int qv = (int)__builtin_amdgcn_perm(0u, 0x0100FFFEu, sel);
#pragma unroll
            for (int m = 0; m < MR; ++m) {
              const uint32_t av = A[(size_t)m * a_row_dw + (k0 >> 2) + 4 * t + j];
              tot[m] = __builtin_amdgcn_sdot4(qv, (int)av, tot[m], false);
            }
          }
      }
    }
  };

  constexpr int UNR = 2;
  int kb = my0;
  for (; kb + UNR <= my1; kb += UNR) {
    uint4 wv[UNR][4];
#pragma unroll
    for (int u = 0; u < UNR; ++u)
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) wv[u][kq] = Wl[(size_t)(kb + u) * sb_stride + kq * 16];
#pragma unroll
    for (int u = 0; u < UNR; ++u) do_block(wv[u], kb + u);
  }
  for (; kb < my1; ++kb) {
    uint4 wv[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) wv[kq] = Wl[(size_t)kb * sb_stride + kq * 16];
    do_block(wv, kb);
  }

  // block reduction across the waves of the workgroup
  __shared__ acc_t red[16][MR][64];
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
      if constexpr (FP) static_cast<_Float16*>(a.C)[o] = (_Float16)s;
      else static_cast<int*>(a.C)[o] = s;
    } else if (a.out_mode == OUT_ATOMIC) {
      if constexpr (FP) unsafeAtomicAdd(static_cast<float*>(a.ws) + o, s);
      else atomicAdd(static_cast<int*>(a.C) + o, s);
    } else {
      static_cast<acc_t*>(a.ws)[(size_t)part * a.M * a.N + o] = s;
    }
  }
}

template <int FMT>
hipError_t launch_fmt(const RunArgs& a, hipStream_t st) {
  dim3 grid((a.N + 63) / 64, a.k_parts), block(64 * a.waves);
  switch (a.M) {
#define QG_CASE(R) \
  case R: hipLaunchKernelGGL((gemv_kernel<FMT, R>), grid, block, 0, st, a); break;
    QG_CASE(1) QG_CASE(2) QG_CASE(3) QG_CASE(4) QG_CASE(5) QG_CASE(6) QG_CASE(7) QG_CASE(8)
#undef QG_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(int fmt, const RunArgs& a, hipStream_t st) {
  switch (fmt) {
    case FMT_I4: return launch_fmt<FMT_I4>(a, st);
    case FMT_U4: return launch_fmt<FMT_U4>(a, st);
    case FMT_F16: return launch_fmt<FMT_F16>(a, st);
    case FMT_I8: return launch_fmt<FMT_I8>(a, st);
    case FMT_I2: return launch_fmt<FMT_I2>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
