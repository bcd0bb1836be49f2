// Split-K helpers: zeroing of the atomic accumulator (a fill kernel rather than
// a memset so that callers may capture qgemm_run in a HIP graph) or, for int32
// outputs with a bias, its filling with the bias rows; the fp32 -> fp16
// conversion after atomic accumulation, and the fixed-order two-pass reduction
// of per-part partials (the deterministic alternative to the atomic reduction
// of hidet issue #364's parallel-k), each adding the bias if there is one.
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
