// M > 8 path: LDS-staged tiles on the gfx950 matrix cores.
//
// fp16 activations use v_mfma_f32_16x16x32_f16 (fp32 accumulation); int8
// activations use v_mfma_i32_16x16x64_i8 (exact int32 accumulation, the int8
// product semantics of Triton PR #3595).  Every stage moves a BM-row activation
// slab and BN/16 x KSTEP weight superblocks from HBM into one of two LDS
// buffers while the other is consumed (the multi-stage software pipelining of
// hidet issue #364; the depth is two, the tile and stage depth depend on the
// problem size).  Packed weights are upcast in registers right before the
// MFMA: int4 nibbles become fp16 by or-ing the 0x6400 exponent and subtracting
// the bias exactly, then the group scale (and zero point) is applied in fp16;
// int2 crumbs become int8 through a byte-permute table.  Since the pack kernel
// stores each 16-byte weight piece in the lane order of the B operand (lane l:
// column l%16, K slice l/16), a B fragment is one conflict-free 16-byte LDS read
// per lane; the A fragment of lane l reads row l%16 at the matching K slice, so
// A and B agree on the K order by construction.
//
// Workgroups are numbered so that each of the 8 XCDs (which receive workgroups
// round-robin) owns a contiguous band of output tiles, swept in column-major
// groups of 8 tile rows: the A row-blocks and B column-blocks that concurrently
// running workgroups share then stay in that XCD's L2 (the traversal / L2
// reuse point made in the mKernel AG-GEMM PR #41 discussion).
#include "qgemm_internal.hpp"

namespace qg {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }
__device__ __forceinline__ uint32_t as_u32(half2v x) { return __builtin_bit_cast(uint32_t, x); }

template <int FMT> struct FmtTraits;
// E: elements per lane per MFMA; STEPS: MFMA K-steps per superblock
template <> struct FmtTraits<FMT_I4> { static constexpr int E = 8, STEPS = 4; static constexpr bool FP = true; };
template <> struct FmtTraits<FMT_U4> { static constexpr int E = 8, STEPS = 4; static constexpr bool FP = true; };
template <> struct FmtTraits<FMT_F16> { static constexpr int E = 8, STEPS = 1; static constexpr bool FP = true; };
template <> struct FmtTraits<FMT_I8> { static constexpr int E = 16, STEPS = 1; static constexpr bool FP = false; };
template <> struct FmtTraits<FMT_I2> { static constexpr int E = 16, STEPS = 4; static constexpr bool FP = false; };

// superblocks per stage: 256 activation bytes per row, 128 for the 256-row tiles
// of the fp16 and int8 weight formats (keeps two stages within LDS)
constexpr int kstep_of(int fmt, int bm) {
  return (fmt == FMT_I4 || fmt == FMT_U4 || fmt == FMT_I2) ? 1 : (bm >= 256 ? 2 : 4);
}

template <int FMT, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void mfma_kernel(RunArgs a) {
  using T = FmtTraits<FMT>;
  constexpr bool FP = T::FP;
  constexpr int KB = kb_of(FMT);
  constexpr int KSTEP = kstep_of(FMT, BM), E = T::E, STEPS = T::STEPS;
  constexpr int ESZ = FP ? 2 : 1;             // activation element bytes
  constexpr int ROWB = KSTEP * KB * ESZ;      // activation bytes per row per stage
  constexpr int PITCH = ROWB + 16;            // padded LDS row pitch (conflict-free fragment reads)
  constexpr int NT = WM * WN * 64;
  constexpr int WTM = BM / WM / 16, WTN = BN / WN / 16;
  constexpr int NBT = BN / 16;                // superblock columns per tile
  constexpr int CPR = ROWB / 16;              // 16-byte chunks per activation row
  constexpr int A_CHUNKS = BM * CPR;          // 16-byte chunks per stage
  constexpr int B_CHUNKS = KSTEP * NBT * 64;
  constexpr int A_PER = (A_CHUNKS + NT - 1) / NT;
  constexpr int B_PER = (B_CHUNKS + NT - 1) / NT;
  static_assert(ROWB == 128 || ROWB == 256, "activation slab of 128 or 256 bytes per row");
  typedef typename std::conditional<FP, float4v, int4v>::type acc_v;

  __shared__ __attribute__((aligned(16))) uint8_t lds_a[2][BM * PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t lds_b[2][B_CHUNKS * 16];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int kq = lane >> 4, l16 = lane & 15;

  // ---- tile of this workgroup (1-D grid: tiles x k-parts)
  const int tiles_n = (a.N + BN - 1) / BN, tiles_m = (a.M + BM - 1) / BM;
  const int tiles = tiles_m * tiles_n;
  int w = blockIdx.x;
  const int part = w / tiles;
  w -= part * tiles;
  if ((tiles & 7) == 0) w = (w & 7) * (tiles >> 3) + (w >> 3);  // contiguous band per XCD
  constexpr int GROUP_M = 8;
  const int group = w / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_group = w - group * GROUP_M * tiles_n;
  const int m0 = (first_m + in_group % gsz) * BM, n0 = (in_group / gsz) * BN;

  int u0, u1;
  part_units(a, part, u0, u1);
  const int kb0 = u0 * a.unit_kb, kb1 = u1 * a.unit_kb;
  const int nst = (kb1 - kb0 + KSTEP - 1) / KSTEP;

  const uint8_t* __restrict__ Ab = static_cast<const uint8_t*>(a.A);
  const size_t a_row_bytes = (size_t)a.K * ESZ;

  uint4 ra[A_PER], rb[B_PER];
#pragma unroll
  for (int i = 0; i < A_PER; ++i) ra[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < B_PER; ++i) rb[i] = make_uint4(0, 0, 0, 0);
  // scale (and zero) of this lane's weight column for each n-subtile of the
  // wave, for the stage being staged: half2 (s, s) and (z, z)
  uint32_t rs[WTN], rz[WTN];
#pragma unroll
  for (int j = 0; j < WTN; ++j) { rs[j] = 0x3C003C00u; rz[j] = 0; }

  // Stage loads are branch-free: a superblock past the part's end (only in a
  // partial last stage) is clamped to the last one and never consumed, so the
  // compiler sees a fixed number of loads and never drains them early.
  auto g_load = [&](int st) {
    const int kbs = kb0 + st * KSTEP;
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      if (A_CHUNKS % NT == 0 || c < A_CHUNKS) {
        const int r = c / CPR, cc = c % CPR;
        const int row = min(m0 + r, a.M - 1);
        const int kk = (cc * 16) / (KB * ESZ);  // superblock of this chunk within the stage
        const int kbl = min(kbs + kk, kb1 - 1);
        ra[i] = *reinterpret_cast<const uint4*>(Ab + (size_t)row * a_row_bytes + (size_t)kbl * KB * ESZ +
                                                (cc * 16) % (KB * ESZ));
      }
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = tid + i * NT;
      if (B_CHUNKS % NT == 0 || c < B_CHUNKS) {
        const int sbi = c >> 6, piece = c & 63;
        const int kk = sbi / NBT, nbl = sbi % NBT;
        const int kbl = min(kbs + kk, kb1 - 1);
        rb[i] = a.W[((size_t)kbl * a.NB + (n0 >> 4) + nbl) * 64 + piece];
      }
    }
    if constexpr (FMT == FMT_I4 || FMT == FMT_U4) {
      if (a.smode != SC_NONE) {
        const int kpos = kbs * KB + (a.smode == SC_PIECE ? kq * 32 : 0);
        const int grp = a.group_size > 0 ? kpos / a.group_size : 0;
#pragma unroll
        for (int j = 0; j < WTN; ++j) {
          const int col = n0 + (wn * WTN + j) * 16 + l16;
          if (a.zeros) {
            const uint32_t sz = static_cast<const uint32_t*>(a.S)[(size_t)grp * a.Npad + col];
            rs[j] = (sz & 0xFFFFu) * 0x10001u;
            rz[j] = (sz >> 16) * 0x10001u;
          } else {
            const uint32_t s = static_cast<const uint16_t*>(a.S)[(size_t)grp * a.Npad + col];
            rs[j] = s * 0x10001u;
          }
        }
      }
    }
  };
  auto s_store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int c = tid + i * NT;
      if (A_CHUNKS % NT == 0 || c < A_CHUNKS)
        *reinterpret_cast<uint4*>(&lds_a[buf][(c / CPR) * PITCH + (c % CPR) * 16]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int c = tid + i * NT;
      if (B_CHUNKS % NT == 0 || c < B_CHUNKS)
        *reinterpret_cast<uint4*>(&lds_b[buf][c * 16]) = rb[i];
    }
  };

  acc_v acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = acc_v{0, 0, 0, 0};

  uint32_t cs[WTN], cz[WTN];  // scales of the stage being computed

  g_load(0);
  s_store(0);
#pragma unroll
  for (int j = 0; j < WTN; ++j) { cs[j] = rs[j]; cz[j] = rz[j]; }
  __syncthreads();

  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) g_load(st + 1);
    const int kbs = kb0 + st * KSTEP;
    const int kvalid = min(KSTEP, kb1 - kbs);  // superblocks of this stage inside the part
#pragma unroll
    for (int kk = 0; kk < KSTEP; ++kk) {
      if (KSTEP > 1 && kk >= kvalid) break;
      uint4 bp[WTN];
#pragma unroll
      for (int j = 0; j < WTN; ++j)
        bp[j] = *reinterpret_cast<const uint4*>(&lds_b[buf][((kk * NBT) + wn * WTN + j) * 1024 + lane * 16]);
#pragma unroll
      for (int t = 0; t < STEPS; ++t) {
        const int kbyte = (kk * KB + kq * (KB / 4) + t * E) * ESZ;
        uint4 af[WTM];
#pragma unroll
        for (int i = 0; i < WTM; ++i)
          af[i] = *reinterpret_cast<const uint4*>(&lds_a[buf][((wm * WTM + i) * 16 + l16) * PITCH + kbyte]);
        uint4 bf[WTN];
#pragma unroll
        for (int j = 0; j < WTN; ++j) {
          const uint32_t wd = t == 0 ? bp[j].x : t == 1 ? bp[j].y : t == 2 ? bp[j].z : bp[j].w;
          if constexpr (FMT == FMT_I4 || FMT == FMT_U4) {
            constexpr uint32_t bias = (FMT == FMT_I4) ? 0x64086408u : 0x64006400u;
            uint32_t o[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
              half2v q = as_h2(((wd >> (4 * jj)) & 0x000F000Fu) | 0x64006400u) - as_h2(bias);
              if (a.smode != SC_NONE) {
                if (FMT == FMT_U4 && a.zeros) q = q - as_h2(cz[j]);
                q = q * as_h2(cs[j]);
              }
              o[jj] = as_u32(q);
            }
            bf[j] = make_uint4(o[0], o[1], o[2], o[3]);
          } else if constexpr (FMT == FMT_I2) {
            uint32_t o[4];
#pragma unroll
            for (int jj = 0; jj < 3; ++jj)  // offset-binary classes: 0,1,2,3 -> -2,-1,0,1
              o[jj] = __builtin_amdgcn_perm(0u, 0x0100FFFEu, (wd >> (2 * jj)) & 0x03030303u);
            // two's complement class: 0,1,2,3 -> 0,1,-2,-1
            o[3] = __builtin_amdgcn_perm(0u, 0xFFFE0100u, (wd >> 6) & 0x03030303u);
            bf[j] = make_uint4(o[0], o[1], o[2], o[3]);
          } else {
            bf[j] = bp[j];
          }
        }
#pragma unroll
        for (int i = 0; i < WTM; ++i)
#pragma unroll
          for (int j = 0; j < WTN; ++j) {
            if constexpr (FP)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  __builtin_bit_cast(half8v, af[i]), __builtin_bit_cast(half8v, bf[j]), acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
                  __builtin_bit_cast(int4v, af[i]), __builtin_bit_cast(int4v, bf[j]), acc[i][j], 0, 0, 0);
          }
      }
    }
    if (st + 1 < nst) {
      s_store(buf ^ 1);
#pragma unroll
      for (int j = 0; j < WTN; ++j) { cs[j] = rs[j]; cz[j] = rz[j]; }
    }
    __syncthreads();
  }

  // epilogue: lane l holds rows 4*(l/16) + r, column l%16 of each 16x16 sub-tile
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int col = n0 + (wn * WTN + j) * 16 + l16;
      if (col >= a.N) continue;
      const float bf = FP && a.out_mode == OUT_STORE ? bias_f(a, col) : 0.f;
      const int bi = !FP && a.out_mode == OUT_STORE ? bias_i(a, col) : 0;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + (wm * WTM + i) * 16 + kq * 4 + r;
        if (row >= a.M) continue;
        const size_t o = (size_t)row * a.N + col;
        const auto v = acc[i][j][r];
        if (a.out_mode == OUT_STORE) {
          if constexpr (FP) static_cast<_Float16*>(a.C)[o] = (_Float16)(v + bf);
          else if (a.row_scale) static_cast<_Float16*>(a.C)[o] = dq_out(a, row, col, v);
          else static_cast<int*>(a.C)[o] = v + bi;
        } else if (a.out_mode == OUT_ATOMIC) {
          if constexpr (FP) unsafeAtomicAdd(static_cast<float*>(a.ws) + o, v);
          else atomicAdd(int_atomic_target(a) + o, v);
        } else {
          if constexpr (FP) static_cast<float*>(a.ws)[(size_t)part * a.M * a.N + o] = v;
          else static_cast<int*>(a.ws)[(size_t)part * a.M * a.N + o] = v;
        }
      }
    }
}

template <int FMT, int BM, int BN, int WM, int WN>
hipError_t launch_t(const RunArgs& a, hipStream_t st) {
  const int tiles = ((a.M + BM - 1) / BM) * ((a.N + BN - 1) / BN);
  hipLaunchKernelGGL((mfma_kernel<FMT, BM, BN, WM, WN>), dim3(tiles * a.k_parts), dim3(WM * WN * 64), 0, st, a);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(int tile, const RunArgs& a, hipStream_t st) {
  constexpr int BIG_N = (FMT == FMT_F16 || FMT == FMT_I8) ? 256 : 128;
  switch (tile) {
    case TILE_32x64: return launch_t<FMT, 32, 64, 2, 2>(a, st);
    case TILE_64x64: return launch_t<FMT, 64, 64, 2, 2>(a, st);
    case TILE_128x128: return launch_t<FMT, 128, 128, 2, 2>(a, st);
    case TILE_BIG: return launch_t<FMT, 256, BIG_N, 2, 4>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

void tile_dims(int fmt, int tile, int* bm, int* bn) {
  switch (tile) {
    case TILE_32x64: *bm = 32; *bn = 64; return;
    case TILE_64x64: *bm = 64; *bn = 64; return;
    case TILE_128x128: *bm = 128; *bn = 128; return;
    default: *bm = 256; *bn = 256; return;
  }
}

hipError_t launch_mfma(int fmt, int tile, const RunArgs& a, hipStream_t st) {
  switch (fmt) {
    case FMT_I4: return launch_fmt<FMT_I4>(tile, a, st);
    case FMT_U4: return launch_fmt<FMT_U4>(tile, a, st);
    case FMT_F16: return launch_fmt<FMT_F16>(tile, a, st);
    case FMT_I8: return launch_fmt<FMT_I8>(tile, a, st);
    case FMT_I2: return launch_fmt<FMT_I2>(tile, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
