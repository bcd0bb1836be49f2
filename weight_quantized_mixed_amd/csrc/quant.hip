// Dynamic per-token int8 quantisation of fp16 activations, the step in front of
// the int8 x int8 / int8 x int2 products in the int8 dynamic-activation
// configurations of torchao issue #2752 (Int8DynamicActivationInt8WeightConfig,
// Int8DynamicActivationIntxWeightConfig).  Symmetric, one scale per row:
//   scale[m] = max_k |a[m, k]| / 127            (fp32, rounded to nearest)
//   q[m, k]  = clamp(rint(a[m, k] / scale[m]), -127, 127)
// with the division in fp32, correctly rounded, and rint to nearest even; a row
// of zeros gets scale 0 and codes 0.  The products then dequantise with
// acc * scale[m] * weight_scale[n].
//
// One workgroup per row (grid-stride over rows).  Rows up to 32768 values are
// loaded once into registers (all loads in flight together), reduced to their
// largest magnitude (wave shuffles, then LDS across the four waves) and turned
// into codes eight at a time; longer rows take a second pass from cache.
#include "qgemm_internal.hpp"

namespace qg {
namespace {

constexpr int QT = 256;   // threads per workgroup
constexpr int RMAX = 16;  // 16-byte groups a thread keeps in registers (K <= 32768)

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ float group_amax(const uint4& v, float amax) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    amax = fmaxf(amax, fabsf((float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] & 0xFFFFu))));
    amax = fmaxf(amax, fabsf((float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] >> 16))));
  }
  return amax;
}

// eight codes of eight fp16 values
__device__ __forceinline__ uint2 group_codes(const uint4& v, float scale) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  uint32_t out[2] = {0u, 0u};
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float x = (float)__builtin_bit_cast(_Float16, (uint16_t)(w[j / 2] >> (16 * (j & 1))));
    const float c = scale > 0.f ? fminf(fmaxf(rintf(__fdiv_rn(x, scale)), -127.f), 127.f) : 0.f;
    out[j / 4] |= ((uint32_t)(int32_t)c & 0xFFu) << (8 * (j & 3));
  }
  return make_uint2(out[0], out[1]);
}

// the row maximum of every thread's amax (all threads get it)
__device__ __forceinline__ float block_max(float amax, float* part) {
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
  __syncthreads();  // part is rewritten for the next row
  return amax;
}

__global__ __launch_bounds__(QT) void quantize_rows_kernel(const uint4* __restrict__ A, int64_t M, int64_t K,
                                                           uint2* __restrict__ Q, float* __restrict__ S) {
  __shared__ float part[QT / 64];
  const int64_t k8 = K / 8;  // groups of eight values
  for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
    const uint4* a = A + m * k8;
    uint2* q = Q + m * k8;
    if (k8 <= (int64_t)QT * RMAX) {
      // the row stays in registers: every load is issued before the first use
      uint4 v[RMAX];
      float amax = 0.f;
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        const int64_t i = threadIdx.x + (int64_t)r * QT;
        v[r] = i < k8 ? a[i] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < RMAX; ++r) amax = group_amax(v[r], amax);
      const float scale = __fdiv_rn(block_max(amax, part), 127.f);
      if (threadIdx.x == 0) S[m] = scale;
#pragma unroll
      for (int r = 0; r < RMAX; ++r) {
        const int64_t i = threadIdx.x + (int64_t)r * QT;
        if (i < k8) q[i] = group_codes(v[r], scale);
      }
    } else {
      // longer rows: a pass for the maximum, a second one (from cache) for the codes
      float amax = 0.f;
      for (int64_t i = threadIdx.x; i < k8; i += QT) amax = group_amax(a[i], amax);
      const float scale = __fdiv_rn(block_max(amax, part), 127.f);
      if (threadIdx.x == 0) S[m] = scale;
      for (int64_t i = threadIdx.x; i < k8; i += QT) q[i] = group_codes(a[i], scale);
    }
  }
}

}  // namespace

hipError_t launch_quantize_rows(const void* A, int64_t M, int64_t K, void* Q, float* scales, hipStream_t st) {
  const int64_t blocks = M < 65536 ? M : 65536;
  hipLaunchKernelGGL(quantize_rows_kernel, dim3((unsigned)blocks), dim3(QT), 0, st, static_cast<const uint4*>(A), M,
                     K, static_cast<uint2*>(Q), scales);
  return hipGetLastError();
}

}  // namespace qg
