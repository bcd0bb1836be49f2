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
// One workgroup per row (grid-stride over rows): a pass that finds the row's
// largest magnitude (wave shuffles, then LDS across the four waves), and a
// second pass, from cache, that writes the codes eight at a time.
#include "qgemm_internal.hpp"

namespace qg {
namespace {

constexpr int QT = 256;  // threads per workgroup

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__global__ __launch_bounds__(QT) void quantize_rows_kernel(const uint4* __restrict__ A, int64_t M, int64_t K,
                                                           uint2* __restrict__ Q, float* __restrict__ S) {
  __shared__ float part[QT / 64];
  const int64_t k8 = K / 8;  // groups of eight values
  for (int64_t m = blockIdx.x; m < M; m += gridDim.x) {
    const uint4* a = A + m * k8;
    float amax = 0.f;
    for (int64_t i = threadIdx.x; i < k8; i += QT) {
      const uint4 v = a[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        amax = fmaxf(amax, fabsf((float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] & 0xFFFFu))));
        amax = fmaxf(amax, fabsf((float)__builtin_bit_cast(_Float16, (uint16_t)(w[j] >> 16))));
      }
    }
    amax = wave_max(amax);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    __syncthreads();  // part is rewritten for the next row
    const float scale = __fdiv_rn(amax, 127.f);
    if (threadIdx.x == 0) S[m] = scale;
    uint2* q = Q + m * k8;
    for (int64_t i = threadIdx.x; i < k8; i += QT) {
      const uint4 v = a[i];
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      uint32_t out[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint16_t h = (uint16_t)(w[j / 2] >> (16 * (j & 1)));
        float c = 0.f;
        if (scale > 0.f) c = fminf(fmaxf(rintf(__fdiv_rn((float)__builtin_bit_cast(_Float16, h), scale)), -127.f), 127.f);
        out[j / 4] |= ((uint32_t)(int32_t)c & 0xFFu) << (8 * (j & 3));
      }
      q[i] = make_uint2(out[0], out[1]);
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
