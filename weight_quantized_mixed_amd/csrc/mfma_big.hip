// Large-M path: 256 x 256 output tiles, 8 waves (2 x 4, 128 x 64 each), a ring of
// NSTAGE LDS stages filled by direct global -> LDS loads (global_load_lds_dwordx4:
// lane l's 16 bytes land at the instruction's LDS base + 16 l, so no registers or
// LDS-store instructions carry the staging) — the multi-stage software pipelining
// of hidet issue #364 with num_stages = NSTAGE.
//
// One stage covers 32 (fp16 weights), 64 (int8 / int4) or 128 (int2) reduction
// positions.  For int4 and int2 a stage is half a superblock (pieces kq = 2h and
// 2h + 1) and takes two MFMA K-steps; lane group q then uses piece 2h + (q & 1),
// word 2t + (q >> 1) in step t, and the activation fragment reads the same
// positions, so A and B agree on the K order by construction.
//
// Activation rows sit unpadded in LDS with their 16-byte chunks XOR-swizzled
// (chunk c of row r at position c ^ swz(r)), which keeps the fragment reads
// free of bank conflicts with either 32 or 64 LDS banks; the swizzle is applied
// on the global side of the direct loads.  Group scales (and zero points) of the
// stage ride along as one more direct load into LDS.
//
// Workgroups are numbered so each XCD owns a contiguous band of tiles, swept in
// column-major groups of 8 tile rows (L2 reuse of the shared A / B blocks, the
// traversal point of the mKernel AG-GEMM PR #41 discussion).
#include "qgemm_internal.hpp"

#ifndef QG_BIG_WM
#define QG_BIG_WM 2
#endif
#ifndef QG_BIG_WN
#define QG_BIG_WN 4
#endif

namespace qg {
namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }
__device__ __forceinline__ uint32_t as_u32(half2v x) { return __builtin_bit_cast(uint32_t, x); }

// s_waitcnt vmcnt(n), leaving the other counters alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt vmcnt(n) lgkmcnt(0)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (0 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ uint32_t lds_off(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// 16-byte direct global -> LDS load of this lane (gfx950 global_load_lds_dwordx4:
// lane l's bytes land at LDS address m0 + 16 l).  Written as inline assembly so
// that the compiler, which cannot tell the ring slots apart, does not make every
// later LDS read wait for all of these loads; m0 is saved and restored inside.
// Completion is waited for explicitly (s_waitcnt vmcnt + s_barrier) before a
// slot is read.  No register receives data from these loads.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g), "s"(lds_base)
      : "memory");
}

// (x & m) | c in one VALU op (masks that are not inline constants go in registers)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t c) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(c));
  return r;
}

template <int FMT> struct BigCfg;
// SPOS: positions per stage; ROWB: activation bytes per row per stage; BSB: weight
// bytes per 16 columns per stage; NSTAGE: ring depth
template <> struct BigCfg<FMT_F16> { static constexpr int SPOS = 32, ROWB = 64, BSB = 1024, NSTAGE = 4; };
template <> struct BigCfg<FMT_I8> { static constexpr int SPOS = 64, ROWB = 64, BSB = 1024, NSTAGE = 4; };
template <> struct BigCfg<FMT_I4> { static constexpr int SPOS = 64, ROWB = 128, BSB = 512, NSTAGE = 3; };
template <> struct BigCfg<FMT_U4> { static constexpr int SPOS = 64, ROWB = 128, BSB = 512, NSTAGE = 3; };
template <> struct BigCfg<FMT_I2> { static constexpr int SPOS = 128, ROWB = 128, BSB = 512, NSTAGE = 3; };

// position (in 16-byte units) of chunk c of activation row r.  Only r mod 16
// enters, so rows that are 16 apart share one pattern and a fragment read's lane
// addresses differ between sub-tiles by a constant offset; any 16 consecutive rows
// (and any 8 aligned ones) spread over distinct 16-byte bank groups.
template <int ROWB>
__device__ __forceinline__ int swz(int r, int c) {
  r &= 15;
  if constexpr (ROWB == 64) return c ^ (((r >> 1) ^ (r >> 2)) & 3);
  else return c ^ ((r ^ (r >> 3)) & 7);
}

template <int FMT, bool SCALED, bool ZEROS, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void mfma_big_kernel(RunArgs a) {
  using C = BigCfg<FMT>;
  constexpr bool FP = (FMT == FMT_F16 || FMT == FMT_I4 || FMT == FMT_U4);
  constexpr bool I4 = (FMT == FMT_I4 || FMT == FMT_U4);
  constexpr bool HALF = I4 || FMT == FMT_I2;  // stage = half a superblock, two MFMA steps
  constexpr int BM = 256, BN = 256, NT = WM * WN * 64;
  constexpr int WTM = BM / WM / 16, WTN = BN / WN / 16;  // 16 x 16 sub-tiles per wave
  constexpr int SPOS = C::SPOS, ROWB = C::ROWB, BSB = C::BSB, NSTAGE = C::NSTAGE;
  constexpr int KB = kb_of(FMT);
  constexpr int ESZ = FP ? 2 : 1;
  constexpr int A_BYTES = BM * ROWB, B_BYTES = (BN / 16) * BSB;
  constexpr int S_BYTES = SCALED ? BN * (ZEROS ? 4 : 2) : 0;
  constexpr int S_PAD = SCALED ? 1024 : 0;  // a whole 1 KiB direct-load slot
  constexpr int STAGE_BYTES = A_BYTES + B_BYTES + S_PAD;
  constexpr int A_LOADS = A_BYTES / 1024 / (NT / 64), B_LOADS = B_BYTES / 1024 / (NT / 64);
  static_assert(A_BYTES % (1024 * NT / 64) == 0 && B_BYTES % (1024 * NT / 64) == 0, "whole loads per wave");
  // direct loads issued per wave per stage; wave 0 also loads the scale slot
  constexpr int LOADS = A_LOADS + B_LOADS;
  typedef typename std::conditional<FP, float4v, int4v>::type acc_v;

  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int q = lane >> 4, l16 = lane & 15;

  // ---- tile of this workgroup
  const int tiles_n = (a.N + BN - 1) / BN, tiles_m = (a.M + BM - 1) / BM;
  const int tiles = tiles_m * tiles_n;
  int w = blockIdx.x;
  const int part = w / tiles;
  w -= part * tiles;
  if ((tiles & 7) == 0) w = (w & 7) * (tiles >> 3) + (w >> 3);
  constexpr int GROUP_M = 8;
  const int group = w / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_group = w - group * GROUP_M * tiles_n;
  const int m0 = (first_m + in_group % gsz) * BM, n0 = (in_group / gsz) * BN;

  // ---- stages of this k-part (a stage = SPOS positions)
  constexpr int SPB = KB / SPOS;  // stages per superblock (int4: 2, int2: 4, else 1)
  const int u0 = (int)((int64_t)part * a.n_units / a.k_parts);
  const int u1 = (int)((int64_t)(part + 1) * a.n_units / a.k_parts);
  const int s0 = u0 * a.unit_kb * SPB, s1 = u1 * a.unit_kb * SPB;  // global stage indices
  const int nst = s1 - s0;

  const uint8_t* __restrict__ Ab = static_cast<const uint8_t*>(a.A);
  const size_t a_row_bytes = (size_t)a.K * ESZ;
  const uint8_t* __restrict__ Wb = reinterpret_cast<const uint8_t*>(a.W);

  // Per-lane global source of each direct load (the stage-dependent part is added
  // at issue time).  A: wave-instruction i covers 1 KiB = 1024 / ROWB rows.
  constexpr int ROWS_PER_LOAD = 1024 / ROWB, CPR = ROWB / 16;
  int a_row_off[A_LOADS];
  int a_chunk[A_LOADS];
#pragma unroll
  for (int i = 0; i < A_LOADS; ++i) {
    const int slot = (wave * A_LOADS + i) * 64 + lane;  // 16-byte slot in the stage's A area
    const int r = slot / CPR, p = slot % CPR;
    a_row_off[i] = min(m0 + r, a.M - 1);
    a_chunk[i] = swz<ROWB>(r, p);  // chunk whose data belongs at position p of row r
  }
  // B: wave-instruction i covers 1024 / BSB column blocks of 16
  int b_off[B_LOADS];
#pragma unroll
  for (int i = 0; i < B_LOADS; ++i) {
    const int slot = (wave * B_LOADS + i) * 64 + lane;
    const int byte = slot * 16;
    const int nbl = byte / BSB, within = byte % BSB;
    b_off[i] = ((n0 >> 4) + nbl) * 1024 + within;  // + kb * NB * 1024 + piece offset of the stage
  }

  auto issue = [&](int st) {  // stage st of this part into ring slot st % NSTAGE
    const int gs = s0 + min(st, nst - 1);  // clamped: stages past the end are never consumed
    const int kb = gs / SPB, sub = gs % SPB;
    uint8_t* base = lds + (st % NSTAGE) * STAGE_BYTES;
    const size_t kpos_bytes = (size_t)gs * SPOS * ESZ;
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
      const uint8_t* g = Ab + (size_t)a_row_off[i] * a_row_bytes + kpos_bytes + a_chunk[i] * 16;
      dma16(g, lds_off(base) + (wave * A_LOADS + i) * 1024);
    }
    const size_t sb_row = (size_t)kb * a.NB * 1024 + (size_t)sub * BSB;
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i)
      dma16(Wb + sb_row + b_off[i], lds_off(base) + A_BYTES + (wave * B_LOADS + i) * 1024);
    if constexpr (SCALED) {
      if (wave == 0) {
        // (scale[, zero]) of columns n0 .. n0 + 255: 512 or 1024 bytes (lanes past
        // the end re-read the last 16 bytes into the unused half of the slot)
        const int grp = (kb * KB) / (a.group_size > 0 ? a.group_size : a.K);
        const int bytes_per = ZEROS ? 4 : 2;
        const int off = min(lane * 16, S_BYTES - 16);
        const uint8_t* src = static_cast<const uint8_t*>(a.S) + ((size_t)grp * a.Npad + n0) * bytes_per + off;
        dma16(src, lds_off(base) + A_BYTES + B_BYTES);
      }
    }
  };

  acc_v acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = acc_v{0, 0, 0, 0};

  // Register double buffering: the fragments of the next MFMA step are read from
  // LDS (and, for int4 / int2, upcast) while the MFMAs of the current step run, so
  // LDS reads, dequantisation and matrix-core work overlap instead of alternating.
  struct Frag {
    uint4 a[WTM];  // activation fragments (16 rows each)
    uint4 b[WTN];  // MFMA-ready weight fragments (16 columns each)
  };
  // int4 / int2: the one packed word (8 int4 or 16 int2 values) that a lane feeds
  // to an MFMA step, per column block, and the block's scale / zero point pair
  uint32_t rw[WTN];
  uint32_t sc[WTN], zc[WTN];

  auto slot = [&](int s) -> const uint8_t* { return lds + (s % NSTAGE) * STAGE_BYTES; };

  // stage sn becomes readable: this wave's loads of it are done when at most
  // NSTAGE - 2 later stages of loads are outstanding, and lgkmcnt(0) retires this
  // wave's LDS reads of the stage held in registers, whose ring slot the load
  // issued after the barrier overwrites.  A bare s_barrier (a compiler memory
  // barrier through the clobber) instead of __syncthreads, whose fence would
  // drain the loads still in flight.
  auto sync_stage = [&](int sn) {
    if (SCALED && wave == 0) wait_vm_lgkm0<(NSTAGE - 2) * (LOADS + 1)>();
    else wait_vm_lgkm0<(NSTAGE - 2) * LOADS>();
    asm volatile("s_barrier" ::: "memory");
    issue(sn + NSTAGE - 1);
  };

  // keeps the machine scheduler from moving instructions across it, so that the
  // reads of the next fragments issue before the MFMAs of the current ones and no
  // MFMA of the next step is hoisted above the barrier that guards its data
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  // fragments of step t of stage s: activation rows, and the weight pieces of this
  // wave's column blocks (straight into the fragment for fp16 / int8; for int4 /
  // int2 the packed word, plus the stage's scales on its first step)
  auto read_step = [&](Frag& f, int s, int t) {
    const uint8_t* base = slot(s);
    int chunk;
    if constexpr (HALF) chunk = (q & 1) * 4 + (2 * t + (q >> 1));  // piece q & 1, word 2t + (q >> 1)
    else chunk = q;                                                  // 8 fp16 / 16 int8 per lane group
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      const int r = (wm * WTM + i) * 16 + l16;
      f.a[i] = *reinterpret_cast<const uint4*>(base + r * ROWB + swz<ROWB>(r, chunk) * 16);
    }
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const uint8_t* lb = base + A_BYTES + (wn * WTN + j) * BSB;
      if constexpr (HALF)
        rw[j] = *reinterpret_cast<const uint32_t*>(lb + ((q & 1) * 16 + l16) * 16 + (2 * t + (q >> 1)) * 4);
      else
        f.b[j] = *reinterpret_cast<const uint4*>(lb + lane * 16);  // whole superblock, piece = lane
      if constexpr (SCALED) {
        if (t == 0) {
          const int col = (wn * WTN + j) * 16 + l16;
          if constexpr (ZEROS) {
            const uint32_t u = *reinterpret_cast<const uint32_t*>(base + A_BYTES + B_BYTES + col * 4);
            sc[j] = (u & 0xFFFFu) * 0x10001u;
            zc[j] = (u >> 16) * 0x10001u;
          } else {
            const uint32_t u = *reinterpret_cast<const uint16_t*>(base + A_BYTES + B_BYTES + col * 2);
            sc[j] = u * 0x10001u;
            zc[j] = 0;
          }
        }
      }
    }
  };

  // upcast of column block j from its packed word (int4 / int2 only)
  auto make_b = [&](Frag& f, int j) {
    if constexpr (HALF) {
      const uint32_t wd = rw[j];
      uint32_t o[4];
      if constexpr (I4) {
        constexpr uint32_t bias = (FMT == FMT_I4) ? 0x64086408u : 0x64006400u;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          half2v v = as_h2(and_or(wd >> (4 * jj), 0x000F000Fu, 0x64006400u)) - as_h2(bias);
          if constexpr (ZEROS) v = v - as_h2(zc[j]);
          if constexpr (SCALED) v = v * as_h2(sc[j]);
          o[jj] = as_u32(v);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 3; ++jj)
          o[jj] = __builtin_amdgcn_perm(0u, 0x0100FFFEu, (wd >> (2 * jj)) & 0x03030303u);
        o[3] = __builtin_amdgcn_perm(0u, 0xFFFE0100u, (wd >> 6) & 0x03030303u);
      }
      f.b[j] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };

  auto mma = [&](const Frag& f, int j) {
#pragma unroll
    for (int i = 0; i < WTM; ++i) {
      if constexpr (FP)
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            __builtin_bit_cast(half8v, f.a[i]), __builtin_bit_cast(half8v, f.b[j]), acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
            __builtin_bit_cast(int4v, f.a[i]), __builtin_bit_cast(int4v, f.b[j]), acc[i][j], 0, 0, 0);
    }
  };

  // one MFMA step on cur while nxt (already read) is upcast, block by block
  auto compute = [&](const Frag& cur, Frag& nxt) {
    fence();
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      mma(cur, j);
      make_b(nxt, j);
    }
    fence();
  };

  // prologue: NSTAGE stages in flight, then the fragments of step 0
#pragma unroll
  for (int st = 0; st < NSTAGE; ++st) issue(st);
  if (SCALED && wave == 0) wait_vm_lgkm0<(NSTAGE - 1) * (LOADS + 1)>();
  else wait_vm_lgkm0<(NSTAGE - 1) * LOADS>();
  asm volatile("s_barrier" ::: "memory");

  Frag X, Y;
  read_step(X, 0, 0);
#pragma unroll
  for (int j = 0; j < WTN; ++j) make_b(X, j);

  if constexpr (HALF) {
    // two MFMA steps per stage: X holds step 0 of stage s, Y step 1
    for (int s = 0; s < nst; ++s) {
      fence();
      read_step(Y, s, 1);
      compute(X, Y);
      sync_stage(s + 1);  // past the last stage this reads clamped copies that are never used
      fence();
      read_step(X, s + 1, 0);
      compute(Y, X);
    }
  } else {
    // one MFMA step per stage, two stages per iteration
    int s = 0;
    for (; s + 1 < nst; s += 2) {
      sync_stage(s + 1);
      fence();
      read_step(Y, s + 1, 0);
      compute(X, Y);
      sync_stage(s + 2);
      fence();
      read_step(X, s + 2, 0);
      compute(Y, X);
    }
    if (s < nst) compute(X, Y);
  }
  wait_vmcnt<0>();  // drain the clamped tail loads before the workgroup's LDS is released

  // epilogue: lane l holds rows 4 (l / 16) + r, column l % 16 of each 16 x 16 sub-tile
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int col = n0 + (wn * WTN + j) * 16 + l16;
      if (col >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + (wm * WTM + i) * 16 + q * 4 + r;
        if (row >= a.M) continue;
        const size_t o = (size_t)row * a.N + col;
        const auto v = acc[i][j][r];
        if (a.out_mode == OUT_STORE) {
          if constexpr (FP) static_cast<_Float16*>(a.C)[o] = (_Float16)v;
          else static_cast<int*>(a.C)[o] = v;
        } else if (a.out_mode == OUT_ATOMIC) {
          if constexpr (FP) unsafeAtomicAdd(static_cast<float*>(a.ws) + o, v);
          else atomicAdd(static_cast<int*>(a.C) + o, v);
        } else {
          if constexpr (FP) static_cast<float*>(a.ws)[(size_t)part * a.M * a.N + o] = v;
          else static_cast<int*>(a.ws)[(size_t)part * a.M * a.N + o] = v;
        }
      }
    }
}

template <int FMT, bool SCALED, bool ZEROS>
hipError_t launch_big_t(const RunArgs& a, hipStream_t st) {
  using C = BigCfg<FMT>;
  constexpr int STAGE_BYTES = 256 * C::ROWB + 16 * C::BSB + (SCALED ? 1024 : 0);
  static_assert((size_t)STAGE_BYTES * C::NSTAGE <= 160 * 1024, "LDS budget");
  const int tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  hipLaunchKernelGGL((mfma_big_kernel<FMT, SCALED, ZEROS, QG_BIG_WM, QG_BIG_WN>), dim3(tiles * a.k_parts),
                     dim3(QG_BIG_WM * QG_BIG_WN * 64), 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool big_tile_supported(int fmt, const RunArgs& a) {
  // whole groups per stage pair and no per-piece scales
  if ((fmt == FMT_I4 || fmt == FMT_U4) && a.smode == SC_PIECE) return false;
  return true;
}

hipError_t launch_mfma_big(int fmt, const RunArgs& a, hipStream_t st) {
  const bool sc = a.smode != SC_NONE;
  switch (fmt) {
    case FMT_F16: return launch_big_t<FMT_F16, false, false>(a, st);
    case FMT_I8: return launch_big_t<FMT_I8, false, false>(a, st);
    case FMT_I2: return launch_big_t<FMT_I2, false, false>(a, st);
    case FMT_I4: return sc ? launch_big_t<FMT_I4, true, false>(a, st) : launch_big_t<FMT_I4, false, false>(a, st);
    case FMT_U4:
      return !sc ? launch_big_t<FMT_U4, false, false>(a, st)
           : a.zeros ? launch_big_t<FMT_U4, true, true>(a, st) : launch_big_t<FMT_U4, true, false>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
