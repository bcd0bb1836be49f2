// Split-K helpers: zeroing of the atomic accumulator (a fill kernel rather than
// a memset so that callers may capture qgemm_run in a HIP graph) or, for int32
// outputs with a bias, its filling with the bias rows; the fp32 -> fp16
// conversion after atomic accumulation, and the fixed-order two-pass reduction
// of per-part partials (the deterministic alternative to the atomic reduction
// of hidet issue #364's parallel-k), each adding the bias if there is one; the
// activation row sums by scale group that fold uint4 zero points out of the
// large tiles' K loop.
#include "qgemm_internal.hpp"

namespace qg {
namespace {

__global__ void fill_zero_kernel(uint4* __restrict__ p, size_t n16, uint32_t* __restrict__ tail,
                                 size_t n4tail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && threadIdx.x < n4tail) tail[threadIdx.x] = 0;
}

// C = fp16(sum over parts of ws[p]) (fp16 output) or int32 sum; parts = 1 for the
// conversion after atomics.  Parts are added in order 0, 1, ..., so the result
// does not depend on scheduling.
template <bool FP>
__global__ void finalize_kernel(const void* __restrict__ ws, void* __restrict__ C, size_t mn, int parts,
                                RunArgs a) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < mn; i += stride) {
    const int col = (a.bias || a.row_scale) ? (int)(i % (size_t)a.N) : 0;
    if constexpr (FP) {
      const float* w = static_cast<const float*>(ws);
      float s = w[i];
      for (int p = 1; p < parts; ++p) s += w[(size_t)p * mn + i];
      static_cast<_Float16*>(C)[i] = (_Float16)(s + bias_f(a, col));
    } else {
      const int* w = static_cast<const int*>(ws);
      int s = w[i];
      for (int p = 1; p < parts; ++p) s += w[(size_t)p * mn + i];
      if (a.row_scale) static_cast<_Float16*>(C)[i] = dq_out(a, (int)(i / (size_t)a.N), col, s);
      else static_cast<int*>(C)[i] = s + bias_i(a, col);
    }
  }
}

// int32 C[m, n] = bias[n], rows of N elements
__global__ void fill_bias_kernel(int* __restrict__ C, const int* __restrict__ bias, int M, int N) {
  for (int m = blockIdx.y; m < M; m += gridDim.y)
    for (int n = blockIdx.x * blockDim.x + threadIdx.x; n < N; n += gridDim.x * blockDim.x)
      C[(size_t)m * N + n] = bias[n];
}

// one 16-byte chunk of a padded row per thread, its elements read one by one (the
// source rows need not be 16-byte aligned)
template <typename T>
__global__ void pad_rows_kernel(const T* __restrict__ A, uint4* __restrict__ dst, int64_t M, int64_t K,
                                int64_t Kpad) {
  constexpr int E = 16 / sizeof(T);
  const int64_t chunks_row = Kpad / E, total = M * chunks_row;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t m = i / chunks_row, k0 = (i - m * chunks_row) * E;
    union { T v[E]; uint4 u; } c;
#pragma unroll
    for (int e = 0; e < E; ++e) c.v[e] = k0 + e < K ? A[m * K + k0 + e] : (T)0;
    dst[i] = c.u;
  }
}

// fp32 -> bf16, rounded to nearest even (finite values)
__device__ __forceinline__ uint16_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// sum of the 8 fp16 values of a 16-byte chunk in fp32, in position order
__device__ __forceinline__ float sum8_f16(uint4 v) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] & 0xFFFFu));
    s += (float)__builtin_bit_cast(_Float16, (uint16_t)(w[i] >> 16));
  }
  return s;
}

// Row sums of A over the scale groups (zero-point folding of the 256 x 256 tiles):
// one workgroup per row.  A lane sums a 16-byte chunk (8 positions) in fp32, four
// neighbouring lanes combine theirs into the sum of a 32-position unit by a fixed
// butterfly, so every run rounds alike, and after a barrier lane g adds the units of
// group g in order.  Row length K (a multiple of 32, at most 32 * ROWSUM_MAX_UNITS);
// units: K / 32 floats of dynamic LDS.
constexpr int ROWSUM_BATCH = 8;  // chunks per lane in flight
__global__ __launch_bounds__(256) void group_rowsum_kernel(const uint4* __restrict__ A, uint16_t* __restrict__ zr,
                                                           int K, int upg, int G, int gp) {
  extern __shared__ float unit[];
  const int chunks = K / 8;
  const uint4* row = A + (size_t)blockIdx.x * chunks;
  for (int c0 = 0; c0 < chunks; c0 += 256 * ROWSUM_BATCH) {
    uint4 v[ROWSUM_BATCH];
#pragma unroll
    for (int b = 0; b < ROWSUM_BATCH; ++b) {
      const int c = c0 + b * 256 + (int)threadIdx.x;
      v[b] = c < chunks ? row[c] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < ROWSUM_BATCH; ++b) {
      // chunks is a multiple of 4, so the four lanes of a unit are all in range or all out
      const int c = c0 + b * 256 + (int)threadIdx.x;
      float s = sum8_f16(v[b]);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      if (c < chunks && (threadIdx.x & 3) == 0) unit[c >> 2] = s;
    }
  }
  __syncthreads();
  uint16_t* out = zr + (size_t)blockIdx.x * 2 * gp;
  for (int g = threadIdx.x; g < gp; g += 256) {
    float r = 0.f;
    if (g < G)
      for (int u = g * upg; u < (g + 1) * upg; ++u) r += unit[u];
    const uint16_t hi = bf16_rne(r);
    out[g] = hi;
    out[gp + g] = bf16_rne(r - __uint_as_float((uint32_t)hi << 16));
  }
}

// The zero-point term of the 256 x 256 tiles for each column and scale group, as bf16
// hi + lo planes, [Npad][hi gp | lo gp], from the (scale, zero) pairs [G][Npad]; groups
// G .. gp - 1 zero.  Those tiles upcast a weight q of the group as one fp16 fma,
// (1024 + q) s + c with b = fp16(1024 + z) = 1024 + r and c = fp16(-b s), which is
// (q - r) s + d rounded once, d = c + b s (exact in fp32, as is b s); the term is
// P = -(z - r) s - d, so that adding sum_g R[m, g] P[g, n] leaves (q - z) s.
// Consecutive threads take consecutive columns of one group, so the pairs are read
// in order.  Signed int4 (pairs false: fp16 scales [G][Npad]) takes its offset 8 as
// the zero point: b = 1032, r = 8, P = -d.
__global__ void zero_planes_kernel(const void* __restrict__ S, uint16_t* __restrict__ zp, int Npad, int G, int gp,
                                   bool pairs) {
  // a thread takes 8 consecutive groups of one column (16 bytes of each plane); the
  // threads of a run take consecutive columns, so each group's reads stay in order
  const int64_t total = (int64_t)Npad * (gp / 8);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int gb = (int)(i / Npad), col = (int)(i - (int64_t)gb * Npad);
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int g = gb * 8 + e;
      float p = 0.f;
      if (g < G) {
        const uint32_t u = pairs ? static_cast<const uint32_t*>(S)[(size_t)g * Npad + col]
                                 : static_cast<const uint16_t*>(S)[(size_t)g * Npad + col] | 0x48000000u;  // z = 8
        const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xFFFFu));
        const float z = (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16));
        const float b = (float)(_Float16)(z + 1024.f);  // z + 1024 is exact in fp32
        const float bs = b * s;                         // exact: 11 x 11 significant bits
        const float d = (float)(_Float16)(-bs) + bs;    // the rounding of c, exact
        p = -(z - (b - 1024.f)) * s - d;
      }
      const uint32_t h = bf16_rne(p);
      const uint32_t l = bf16_rne(p - __uint_as_float(h << 16));
      if (e & 1) {
        hi[e / 2] |= h << 16;
        lo[e / 2] |= l << 16;
      } else {
        hi[e / 2] = h;
        lo[e / 2] = l;
      }
    }
    uint4* o = reinterpret_cast<uint4*>(zp + (size_t)col * 2 * gp + gb * 8);  // 16-byte aligned: gp % 32 == 0
    o[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    o[gp / 8] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  }
}

int grid_for(size_t items, int threads) {
  size_t b = (items + threads - 1) / threads;
  if (b > 8192) b = 8192;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t st) {
  // bytes is a multiple of 4 (fp32 / int32 elements)
  const size_t n16 = bytes / 16, n4tail = (bytes % 16) / 4;
  uint32_t* tail = reinterpret_cast<uint32_t*>(static_cast<char*>(p) + n16 * 16);
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n16 ? n16 : 1, 256)), dim3(256), 0, st,
                     static_cast<uint4*>(p), n16, tail, n4tail);
  return hipGetLastError();
}

hipError_t launch_pad_rows(const void* A, void* dst, int64_t M, int64_t K, int64_t Kpad, int esz,
                           hipStream_t st) {
  const size_t chunks = (size_t)M * (size_t)(Kpad * esz / 16);
  if (esz == 2)
    hipLaunchKernelGGL(pad_rows_kernel<uint16_t>, dim3(grid_for(chunks, 256)), dim3(256), 0, st,
                       static_cast<const uint16_t*>(A), static_cast<uint4*>(dst), M, K, Kpad);
  else
    hipLaunchKernelGGL(pad_rows_kernel<uint8_t>, dim3(grid_for(chunks, 256)), dim3(256), 0, st,
                       static_cast<const uint8_t*>(A), static_cast<uint4*>(dst), M, K, Kpad);
  return hipGetLastError();
}

hipError_t launch_group_rowsum(const RunArgs& a, uint16_t* zr, hipStream_t st) {
  if (a.K % 32 != 0 || a.K / 32 > ROWSUM_MAX_UNITS || a.zr_gp % 32 != 0 || a.zr_G > a.zr_gp)
    return hipErrorInvalidValue;
  const int upg = a.group_size > 0 ? a.group_size / 32 : a.K / 32;
  hipLaunchKernelGGL(group_rowsum_kernel, dim3(a.M), dim3(256), (size_t)(a.K / 32) * sizeof(float), st,
                     static_cast<const uint4*>(a.A), zr, a.K, upg, a.zr_G, a.zr_gp);
  return hipGetLastError();
}

hipError_t launch_zero_planes(const RunArgs& a, uint16_t* zp, hipStream_t st) {
  if (!a.S || a.zr_gp % 32 != 0 || a.zr_G > a.zr_gp) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_planes_kernel, dim3(grid_for((size_t)a.Npad * (a.zr_gp / 8), 256)), dim3(256), 0, st, a.S, zp,
                     a.Npad, a.zr_G, a.zr_gp, a.zeros != 0);
  return hipGetLastError();
}

hipError_t launch_finalize(const RunArgs& a, int acc_fp, hipStream_t st) {
  const size_t mn = (size_t)a.M * a.N;
  const int parts = a.out_mode == OUT_PARTIAL ? a.k_parts : 1;
  if (acc_fp)
    hipLaunchKernelGGL(finalize_kernel<true>, dim3(grid_for(mn, 256)), dim3(256), 0, st, a.ws, a.C, mn, parts, a);
  else
    hipLaunchKernelGGL(finalize_kernel<false>, dim3(grid_for(mn, 256)), dim3(256), 0, st, a.ws, a.C, mn, parts, a);
  return hipGetLastError();
}

hipError_t launch_fill_bias(const RunArgs& a, hipStream_t st) {
  const int gx = (a.N + 255) / 256 < 64 ? (a.N + 255) / 256 : 64;
  const int gy = a.M < 1024 ? a.M : 1024;
  hipLaunchKernelGGL(fill_bias_kernel, dim3(gx, gy), dim3(256), 0, st, static_cast<int*>(a.C),
                     static_cast<const int*>(a.bias), a.M, a.N);
  return hipGetLastError();
}

}  // namespace qg
