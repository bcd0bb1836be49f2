// One-time repacking of canonical "nt" weights into the gfx950 superblock blob
// (K padded with zero codes to whole superblocks), and of the [N, G] scale / zero
// tables into [G_store][Npad] rows.  The storage
// format is the problem statement's transposed weight (BitBLAS issue #252,
// reproduction script, layout "nt"); the pre-shuffled, backend-specific packed
// tensor follows the "dtype + packing_format" structure of torchao issue #2752.
#include "qgemm_internal.hpp"

namespace qg {
namespace {

// slot (0..7) of a word that receives position p (0..7): evens first, then odds
__device__ __forceinline__ int i4_slot(int p) { return (p & 1) ? 4 + (p >> 1) : (p >> 1); }

// The 16 canonical bytes of column n from reduction position k0 on (one piece):
// four words of 8 int4 / 16 int2 values, 16 int8 values or 8 fp16 values.
// Positions at or past K read as zero codes; rows that are not 16-byte aligned
// (K not a multiple of 32 int4 / 64 int2 / 16 int8 / 8 fp16 values) are read
// word by word or element by element.
__device__ __forceinline__ uint4 canonical_piece(int fmt, const void* __restrict__ w, int64_t n, int64_t K,
                                                 int64_t k0) {
  const int pf = pack_factor(fmt);
  const int per16 = pf == 1 ? (fmt == FMT_I8 ? 16 : 8) : 4 * pf;  // values per 16 bytes
  const int64_t row_elems = pf == 1 ? K : K / pf;                  // elements (words) per row
  const bool aligned = K % per16 == 0 && k0 + per16 <= K;
  if (aligned) {
    if (pf == 1) {
      const size_t esz = fmt == FMT_I8 ? 1 : 2;
      return *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(w) + ((size_t)n * K + k0) * esz);
    }
    return reinterpret_cast<const uint4*>(w)[((size_t)n * row_elems + k0 / pf) / 4];
  }
  union { uint32_t d[4]; uint8_t b[16]; uint16_t h[8]; uint4 u; } r;
  r.u = make_uint4(0, 0, 0, 0);
  if (pf > 1) {
    const uint32_t* src = static_cast<const uint32_t*>(w) + (size_t)n * row_elems;
    for (int t = 0; t < 4; ++t)
      if (k0 + (int64_t)t * pf < K) r.d[t] = src[k0 / pf + t];  // K is a multiple of pf
  } else if (fmt == FMT_I8) {
    const uint8_t* src = static_cast<const uint8_t*>(w) + (size_t)n * K;
    for (int e = 0; e < 16; ++e)
      if (k0 + e < K) r.b[e] = src[k0 + e];
  } else {
    const uint16_t* src = static_cast<const uint16_t*>(w) + (size_t)n * K;
    for (int e = 0; e < 8; ++e)
      if (k0 + e < K) r.h[e] = src[k0 + e];
  }
  return r.u;
}

__global__ void pack_weights_kernel(int fmt, const void* __restrict__ w, uint4* __restrict__ out,
                                    int64_t N, int64_t K, int64_t NB, int64_t n_pieces) {
  const int KB = kb_of(fmt);
  for (int64_t p = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; p < n_pieces;
       p += (int64_t)gridDim.x * blockDim.x) {
    const int64_t sb = p >> 6;
    const int within = (int)(p & 63);
    const int kq = within >> 4, nn = within & 15;
    const int64_t kb = sb / NB, nb = sb - kb * NB;
    const int64_t n = nb * 16 + nn;
    const int64_t k0 = kb * KB + (int64_t)kq * (KB / 4);
    uint4 r = make_uint4(0, 0, 0, 0);
    if (n < N) {
      const uint4 src = canonical_piece(fmt, w, n, K, k0);
      if (fmt == FMT_I4 || fmt == FMT_U4) {
        const uint32_t in[4] = {src.x, src.y, src.z, src.w};
        uint32_t o[4];
        for (int t = 0; t < 4; ++t) {
          uint32_t acc = 0;
          for (int i = 0; i < 8; ++i) {
            uint32_t v = (in[t] >> (4 * i)) & 0xFu;
            if (fmt == FMT_I4) v ^= 0x8u;  // two's complement -> offset-binary (q + 8)
            acc |= v << (4 * i4_slot(i));
          }
          o[t] = acc;
        }
        r = make_uint4(o[0], o[1], o[2], o[3]);
      } else if (fmt == FMT_I2) {
        const uint32_t in[4] = {src.x, src.y, src.z, src.w};
        uint32_t o[4];
        for (int t = 0; t < 4; ++t) {
          uint32_t acc = 0;
          for (int e = 0; e < 16; ++e) {
            // crumb classes 0..2 offset-binary (q + 2), class 3 (the top bits of
            // each byte) two's complement
            uint32_t c = (in[t] >> (2 * e)) & 0x3u;
            if ((e >> 2) < 3) c ^= 0x2u;
            acc |= c << (8 * (e & 3) + 2 * (e >> 2));
          }
          o[t] = acc;
        }
        r = make_uint4(o[0], o[1], o[2], o[3]);
      } else {  // FMT_I8, FMT_F16: stored as they are
        r = src;
      }
    }
    out[p] = r;
  }
}

// rows g >= G (groups wholly past K, whose positions read zero activations) get
// zero scales and zero points
__global__ void pack_scales_kernel(const uint16_t* __restrict__ s, const uint16_t* __restrict__ z,
                                   void* __restrict__ out, int64_t N, int64_t Npad, int64_t G, int64_t G_store) {
  const int64_t total = G_store * Npad;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t g = i / Npad, n = i - g * Npad;
    const bool in = n < N && g < G;
    const uint16_t sv = in ? s[n * G + g] : 0;
    if (z) {
      const uint16_t zv = in ? z[n * G + g] : 0;
      static_cast<uint32_t*>(out)[i] = (uint32_t)sv | ((uint32_t)zv << 16);
    } else {
      static_cast<uint16_t*>(out)[i] = sv;
    }
  }
}

int grid_for(int64_t items, int threads) {
  int64_t b = (items + threads - 1) / threads;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (int)b;
}

}  // namespace

hipError_t launch_pack(const Layout& L, const void* w, const void* s, const void* z, void* packed,
                       hipStream_t st) {
  const int64_t n_pieces = L.nkb * L.NB * 64;
  hipLaunchKernelGGL(pack_weights_kernel, dim3(grid_for(n_pieces, 256)), dim3(256), 0, st, L.fmt, w,
                     static_cast<uint4*>(packed), L.N, L.K, L.NB, n_pieces);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || L.G == 0) return e;
  void* sdst = static_cast<char*>(packed) + L.s_offset;
  hipLaunchKernelGGL(pack_scales_kernel, dim3(grid_for(L.G_store * L.Npad, 256)), dim3(256), 0, st,
                     static_cast<const uint16_t*>(s), L.zeros ? static_cast<const uint16_t*>(z) : nullptr,
                     sdst, L.N, L.Npad, L.G, L.G_store);
  return hipGetLastError();
}

}  // namespace qg
