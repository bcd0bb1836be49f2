// Large-tile matrix-core path for fp16 and int4 / uint4 weights: 256 x 256 output
// tiles computed by four waves, each owning a 128 x 128
// quadrant (64 MFMA tiles of 16 x 16, whose accumulators live in the accumulation
// registers), from a ring of two LDS stages that global_load_lds_dwordx4 fills
// straight from memory.  This is the shape of the large-M products in the BitBLAS
// issue #252 benchmark table (M = 16384 rows): every fragment read from LDS feeds 8
// MFMAs, so a wave reads 64 KiB of fragments per 32 positions of a tile instead of
// the 96 KiB of eight 128 x 64 waves (the 256 x 256 tile of mfma_dl.hip, which the
// other formats keep), and one barrier per stage serves 128 MFMAs per wave.
//
// The stage geometry is that of the direct-load tiles (mfma_dl.hip): 128-byte
// activation rows per stage (64 fp16 or 128 int8 positions) with swizzled 16-byte
// chunks, two superblock rows of fp16 / int8 weights or half a superblock row of
// int4 / int2 weights, and for scaled int4 one slot of the stage's group scales.
// Each wave issues the same number of direct loads per stage (the scale slot is
// split four ways by lane), so a fixed vmcnt says when a stage has landed.
//
// Per stage a wave runs two MFMA steps.  The first computes with fragments read
// during the previous step, while it reads (and for int4 upcasts) the second
// step's fragments from the same slot; then one barrier; the second step computes
// while the wave issues its direct loads of the stage NSTAGE ahead into the slot
// just released and reads the next stage's first-step fragments.  With one wave per
// SIMD nothing covers a stall of that wave, so the side operations are spread over
// the 64 MFMAs of a step in a fixed order: the direct loads evenly over the whole
// step (issued as a burst after the barrier they filled the texture path's queue and
// held the matrix cores 47 % idle), the fragment reads after every other MFMA of the
// first half, the upcasts from the 16th MFMA on.
//
// Scaled uint4 is upcast and scaled by one packed fp16 fma per pair, (1024 + q) s +
// c; with zero points the fma's addend holds the zero point rounded to an integer,
// and what it leaves (the fraction of z and the rounding of the addend, a constant
// per column and group) is added after the loop as sum_g R[m, g] P[g, n] by bf16
// MFMAs over the groups (R the row sums of A over each group, both R and P written
// by passes before the kernel), so the loop costs what unscaled int4 costs.
//
// Tiles are numbered as in mfma_dl.hip: each XCD owns a contiguous band of tiles,
// swept in column-major groups of tile rows.
#include "dl_common.hpp"

namespace qg {
namespace {
using namespace dl;

#ifndef QG_BIG_GROUP_M
#define QG_BIG_GROUP_M 2
#endif
// LDS ring depth (stages in flight + 1).  The int4 loop runs two stages per iteration,
// and a depth of two keeps each of them on a fixed slot, so their fragment addresses
// are constants (a depth of three or four recomputed them: 16384^3 uint4 g = 128 6.84 ->
// 6.53 ms, int4 unscaled 6.03-6.06 -> 5.88-5.89 ms); fp16 stages (64 KiB) fit only two.
#ifndef QG_BIG_MAXST
#define QG_BIG_MAXST 2
#endif
#ifndef QG_BIG_U0
#define QG_BIG_U0 16
#endif
#ifndef QG_BIG_RSTEP
#define QG_BIG_RSTEP 2
#endif
#ifndef QG_BIG_DSPAN
#define QG_BIG_DSPAN 64
#endif

template <int FMT, bool SCALED>
struct BigGeo {
  static constexpr bool FP = FMT != FMT_I8 && FMT != FMT_I2;  // fp16 activations
  static constexpr bool PACKED = FMT == FMT_I4 || FMT == FMT_U4 || FMT == FMT_I2;
  static constexpr int KB = kb_of(FMT);
  static constexpr int ESZ = FP ? 2 : 1;
  static constexpr int ROWB = 128;                // activation bytes per row per stage
  static constexpr int SPOS = ROWB / ESZ;         // positions per stage
  static constexpr int BSB = SPOS * 1024 / KB;    // weight bytes per 16 columns per stage
  static constexpr int A_BYTES = 256 * ROWB, B_BYTES = 16 * BSB;
  static constexpr int S_BYTES = SCALED ? 1024 : 0;
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  static constexpr int FIT = 160 * 1024 / STAGE;
  static constexpr int NSTAGE = FIT < QG_BIG_MAXST ? FIT : QG_BIG_MAXST;
  // direct loads of a wave per stage: slots wave, wave + 4, ... of A and of B,
  // and a quarter of the scale slot
  static constexpr int LA = A_BYTES / 1024 / 4, LB = B_BYTES / 1024 / 4;
  static constexpr int L = LA + LB + (SCALED ? 1 : 0);
  static_assert(BSB == 512 || BSB == 2048, "half a superblock or two superblocks per stage");
  static_assert(B_BYTES % 4096 == 0, "B slots split evenly over the waves");
  static_assert(NSTAGE >= 2 && (NSTAGE - 1) * L < 64, "ring depth and the 6-bit load counter");
  static_assert(!SCALED || (FMT == FMT_I4 || FMT == FMT_U4), "scales only with int4 weights");
  static_assert(!PACKED || FMT == FMT_I2 || KB == 2 * SPOS, "an int4 superblock is two stages (two per iteration)");
};

// FOLD: a correction after the loop takes what the loop leaves of the weights' offset,
// the zero points of uint4 (whose scale slot then holds (scale, zero) pairs) or the
// offset 8 of signed int4; see nc below
template <int FMT, bool SCALED, bool FOLD>
__global__ __launch_bounds__(256) void mfma_big_kernel(RunArgs a) {
  using G = BigGeo<FMT, SCALED>;
  constexpr bool FP = G::FP, PACKED = G::PACKED;
  constexpr bool I4 = FMT == FMT_I4 || FMT == FMT_U4;
  // scaled uint4, and folded signed int4: the upcast and scale fold into one packed fma
  // (its addend, -1024 s, -fp16(1024 + z) s or -1032 s, must be finite in fp16:
  // |s| < 63, |s (1024 + z)| < 65504)
  constexpr bool U4S = SCALED && (FMT == FMT_U4 || (FMT == FMT_I4 && FOLD));
  constexpr bool ZEROS = FOLD && FMT == FMT_U4;  // (scale, zero) pairs in the scale slot
  constexpr int KB = G::KB, ESZ = G::ESZ, ROWB = G::ROWB, SPOS = G::SPOS, BSB = G::BSB;
  constexpr int A_BYTES = G::A_BYTES, B_BYTES = G::B_BYTES, STAGE = G::STAGE, NSTAGE = G::NSTAGE;
  constexpr int LA = G::LA, LB = G::LB, L = G::L;
  constexpr int bytes_per_scale = ZEROS ? 4 : 2;
  typedef typename std::conditional<FP, float4v, int4v>::type acc_v;

  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;  // quadrant rows wm * 128.., columns wn * 128..
  const int q = lane >> 4, l16 = lane & 15;

  // ---- tile of this workgroup
  const int tiles_n = (a.N + 255) / 256, tiles_m = (a.M + 255) / 256;
  const int tiles = tiles_m * tiles_n;
  int w = blockIdx.x;
  const int part = w / tiles;
  w -= part * tiles;
  if ((tiles & 7) == 0) w = (w & 7) * (tiles >> 3) + (w >> 3);
  const int group = w / (QG_BIG_GROUP_M * tiles_n);
  const int first_m = group * QG_BIG_GROUP_M;
  const int gsz = min(tiles_m - first_m, QG_BIG_GROUP_M);
  const int in_group = w - group * QG_BIG_GROUP_M * tiles_n;
  const int m0 = (first_m + in_group % gsz) * 256, n0 = (in_group / gsz) * 256;

  // ---- stages of this k-part (a split unit is a whole number of stages)
  int u0, u1;
  part_units(a, part, u0, u1);
  const int s0 = u0 * a.unit_kb * KB / SPOS;
  const int nst = u1 * a.unit_kb * KB / SPOS - s0;

  acc_v acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = acc_v{0, 0, 0, 0};

  if (nst > 0) {
    const uint8_t* __restrict__ Ab = static_cast<const uint8_t*>(a.A);
    const uint32_t a_row_bytes = (uint32_t)a.K * ESZ;  // the plan keeps M * K * ESZ below 4 GiB
    const uint8_t* __restrict__ Wb = reinterpret_cast<const uint8_t*>(a.W);

    // Per-lane 32-bit offsets of this wave's direct loads from their stage's
    // wave-uniform sources.  A slot e covers rows 8 (wave + 4 e) .. + 7, chunk
    // swz(r, p) of row r landing at position p.
    uint32_t a_off[LA];
#pragma unroll
    for (int e = 0; e < LA; ++e) {
      const int c16 = (wave + 4 * e) * 64 + lane;
      const int r = c16 >> 3, p = c16 & 7;
      a_off[e] = (uint32_t)min(m0 + r, a.M - 1) * a_row_bytes + (uint32_t)swz<ROWB, PACKED>(r, p) * 16;
    }
    // B: byte o of the stage's weight area is column block o / BSB, byte o % BSB of
    // it; with two superblocks per stage the second is the next superblock row
    uint32_t b_off[LB];
#pragma unroll
    for (int e = 0; e < LB; ++e) {
      const int o = ((wave + 4 * e) * 64 + lane) * 16;
      const int cb = (n0 >> 4) + o / BSB, wo = o % BSB;
      b_off[e] = BSB == 512 ? (uint32_t)(cb * 1024 + wo)
                            : (uint32_t)(cb * 1024 + (wo >> 10) * a.NB * 1024 + (wo & 1023));
    }
    // scales of columns n0 .. n0 + 255 (lanes past them re-read the last 16 bytes
    // into the unused rest of the slot); wave w loads lanes 16 w .. 16 w + 15
    const uint32_t s_off = (uint32_t)min(lane * 16, 256 * bytes_per_scale - 16);

    // the next stage to issue: ring slot and sources, advanced by constant strides;
    // past the part's last stage the sources stay put (copies never consumed)
    const uint32_t lds0 = lds_off(lds), lds_end = lds0 + NSTAGE * STAGE;
    uint32_t nx_dst = lds0;
    int nx_i = 0;
    const int64_t pos0 = (int64_t)s0 * SPOS;
    const uint8_t* nx_a = Ab + pos0 * ESZ;
    const uint8_t* nx_w = Wb + (pos0 / KB) * a.NB * 1024 + (pos0 % KB) * 1024 / KB;
    const uint8_t* nx_s = nullptr;
    int grp_left = 0;  // stages from the next one to the end of its scale group
    if constexpr (SCALED) {
      int64_t grp = 0;
      grp_left = 1 << 30;  // one group over K
      if (a.group_size > 0) {
        grp = pos0 / a.group_size;
        grp_left = (int)((a.group_size - pos0 % a.group_size) / SPOS);
      }
      nx_s = static_cast<const uint8_t*>(a.S) + ((size_t)grp * a.Npad + n0) * bytes_per_scale;
    }
    auto advance = [&]() {
      nx_dst = nx_dst + STAGE == lds_end ? lds0 : nx_dst + STAGE;
      if (nx_i < nst - 1) {
        nx_a += SPOS * ESZ;
        if constexpr (BSB == 512) nx_w += ((s0 + nx_i) & 1) ? (size_t)a.NB * 1024 - 512 : (size_t)512;
        else nx_w += (size_t)2 * a.NB * 1024;
        if constexpr (SCALED) {
          if (--grp_left == 0) {
            nx_s += (size_t)a.Npad * bytes_per_scale;
            grp_left = a.group_size / SPOS;
          }
        }
      }
      ++nx_i;
    };
    // direct load e of the next stage (A slots, then B slots, then the scale quarter)
    auto dma = [&](auto E) {
      constexpr int e = decltype(E)::value;
      if constexpr (e < LA) {
        dma16s(nx_a, a_off[e], nx_dst + (wave + 4 * e) * 1024);
      } else if constexpr (e < LA + LB) {
        dma16s(nx_w, b_off[e - LA], nx_dst + A_BYTES + (wave + 4 * (e - LA)) * 1024);
      } else {
        if (q == wave) dma16s(nx_s, s_off, nx_dst + A_BYTES + B_BYTES);
      }
      if constexpr (e == L - 1) advance();
    };
    auto issue_all = [&]() { static_for(std::make_integer_sequence<int, L>{}, [&](auto E) { dma(E); }); };

    struct Frag {
      uint4 a[8];  // activation fragments (16 rows each)
      uint4 b[8];  // MFMA-ready weight fragments (16 columns each)
    };
    // int4 upcast constants held in registers (an SGPR mask and a VGPR exponent),
    // so (w & mask) | exponent is one v_and_or_b32
    const uint32_t k_nib = __builtin_amdgcn_readfirstlane(0x000F000Fu);
    uint32_t k_exp;
    asm("v_mov_b32 %0, 0x64006400" : "=v"(k_exp));
    uint32_t rw[8];          // int4 / int2: packed word of column block j
    uint32_t sc[8];          // scale of column block j, both halves
    uint32_t nc[8];          // uint4: the fma's addend, -1024 s (with zero points -fp16(1024 + z) s)
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

    auto read_a = [&](Frag& f, const uint8_t* base, auto T, auto I) {
      constexpr int t = decltype(T)::value, i = decltype(I)::value;
      int chunk;
      if constexpr (PACKED) chunk = (q & 1) * 4 + (2 * t + (q >> 1));  // piece q & 1, word 2t + (q >> 1)
      else chunk = t * 4 + q;
      const int r = wm * 128 + i * 16 + l16;
      f.a[i] = *reinterpret_cast<const uint4*>(base + r * ROWB + swz<ROWB, PACKED>(r, chunk) * 16);
    };
    // SCL: the stage's scales are read as well (at step 0 of a stage whose scales may
    // differ from the previous stage's)
    auto read_b = [&](Frag& f, const uint8_t* base, auto T, auto J, auto SCL) {
      constexpr int t = decltype(T)::value, j = decltype(J)::value;
      constexpr bool scl = decltype(SCL)::value;
      const uint8_t* lb = base + A_BYTES + (wn * 8 + j) * BSB;
      if constexpr (PACKED)
        rw[j] = *reinterpret_cast<const uint32_t*>(lb + ((q & 1) * 16 + l16) * 16 + (2 * t + (q >> 1)) * 4);
      else
        f.b[j] = *reinterpret_cast<const uint4*>(lb + t * 1024 + lane * 16);  // superblock t, piece = lane
      if constexpr (SCALED && t == 0 && scl) {
        const int col = (wn * 8 + j) * 16 + l16;
        // with zero points the slot holds (scale, zero) pairs; the zero points (and
        // the offset of folded signed int4) are applied after the loop
        const uint32_t u = ZEROS ? *reinterpret_cast<const uint32_t*>(base + A_BYTES + B_BYTES + col * 4)
                                 : *reinterpret_cast<const uint16_t*>(base + A_BYTES + B_BYTES + col * 2);
        sc[j] = __builtin_amdgcn_perm(u, u, 0x01000100u);  // low half in both halves
        if constexpr (ZEROS) {
          // b = fp16(1024 + z) = 1024 + r with r = rne(z) for 0 <= z < 1024 (the fp16
          // spacing there is 1), and c = fp16(-b s): the fma below then gives
          // (q - r) s + d rounded once, with d = c + b s the rounding of c, and
          // -(z - r) s - d goes with the zero points after the loop
          const uint32_t b = as_u32(as_h2(__builtin_amdgcn_perm(u, u, 0x03020302u)) + as_h2(k_exp));
          nc[j] = as_u32(as_h2(b) * -as_h2(sc[j]));
        } else if constexpr (FMT == FMT_I4 && U4S) {
          // signed int4, stored q + 8: its offset as a zero point z = 8, b = 1032, c =
          // fp16(-1032 s); -d goes after the loop
          nc[j] = as_u32(as_h2(sc[j]) * as_h2(0xE408E408u));
        } else if constexpr (U4S) {
          nc[j] = as_u32(as_h2(sc[j]) * as_h2(0xE400E400u));  // -1024 s, exact
        }
      }
    };
    // word jj of column block j's MFMA operand from its packed word
    auto make_b_part = [&](Frag& f, auto J, auto JJ) {
      constexpr int j = decltype(J)::value, jj = decltype(JJ)::value;
      if constexpr (PACKED) {
        const uint32_t wd = rw[j];
        uint32_t o;
        if constexpr (I4) {
          const half2v x = as_h2(((wd >> (4 * jj)) & k_nib) | k_exp);  // 1024 + the stored nibble
          half2v v;
          if constexpr (U4S) {
            // (1024 + q) s - 1024 s with one rounding: q s rounded to nearest, as the
            // subtraction and product would give it, in one instruction (with zero
            // points (q - r) s + d, see nc)
            v = __builtin_elementwise_fma(x, as_h2(sc[j]), as_h2(nc[j]));
          } else {
            v = x - as_h2((FMT == FMT_I4) ? 0x64086408u : 0x64006400u);
            if constexpr (SCALED) v = v * as_h2(sc[j]);
          }
          o = as_u32(v);
        } else if constexpr (jj < 3) {
          o = __builtin_amdgcn_perm(0u, 0x0100FFFEu, (wd >> (2 * jj)) & 0x03030303u);  // 0..3 -> -2..1
        } else {
          o = __builtin_amdgcn_perm(0u, 0xFFFE0100u, (wd >> 6) & 0x03030303u);  // 0..3 -> 0, 1, -2, -1
        }
        if constexpr (jj == 0) f.b[j].x = o;
        else if constexpr (jj == 1) f.b[j].y = o;
        else if constexpr (jj == 2) f.b[j].z = o;
        else f.b[j].w = o;
      }
    };
    // The MFMA with its accumulator as a tied operand in the accumulation registers:
    // the builtin lets the allocator give each product a fresh destination and copy
    // all 256 accumulators back at every loop iteration.  The fragments reach an
    // MFMA through LDS reads (waited for by the compiler) or upcasts at least eight
    // MFMAs earlier; the epilogue's reads of the accumulators wait explicitly.
    auto mma = [&acc](const Frag& f, auto K) {  // explicit: asm operands do not capture implicitly
      constexpr int k = decltype(K)::value, i = k % 8, j = k / 8;
      if constexpr (FP)
        asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0"
                     : "+a"(acc[i][j])
                     : "v"(__builtin_bit_cast(half8v, f.a[i])), "v"(__builtin_bit_cast(half8v, f.b[j])));
      else
        asm volatile("v_mfma_i32_16x16x64_i8 %0, %1, %2, %0"
                     : "+a"(acc[i][j])
                     : "v"(__builtin_bit_cast(int4v, f.a[i])), "v"(__builtin_bit_cast(int4v, f.b[j])));
    };

    // One MFMA step on cur with, between its MFMAs: (DMA) this wave's direct loads of
    // the next stage, spread evenly over the step (a burst of them after the barrier
    // fills the texture path's queue, and the wave, alone on its SIMD, stalls with
    // the matrix core idle); the reads of step T of the slot at rb into nxt, after
    // every other MFMA of the first half; and nxt's upcasts in the second half.
    constexpr int NR = 16, NU = PACKED ? 32 : 0;
    auto step = [&](const Frag& cur, Frag& nxt, const uint8_t* rb, auto T, auto DMA, auto SCL) {
      constexpr bool D = decltype(DMA)::value;
      constexpr int ND = D ? L : 0;
      constexpr int DSTEP = ND > 0 ? QG_BIG_DSPAN / (ND > 0 ? ND : 1) : 64;  // loads over the first DSPAN MFMAs
      constexpr int U0 = QG_BIG_U0;    // first MFMA followed by an upcast
      constexpr int RS = QG_BIG_RSTEP; // MFMAs between two fragment reads
      fence();
      static_for(std::make_integer_sequence<int, 64>{}, [&](auto K) {
        constexpr int k = decltype(K)::value;
        mma(cur, K);
        fence();
        if constexpr (D && k % DSTEP == 0 && k / DSTEP < ND) {
          dma(std::integral_constant<int, k / DSTEP>{});
          fence();
        }
        if constexpr (k % RS == 1 % RS && k / RS < 8) {
          read_b(nxt, rb, T, std::integral_constant<int, k / RS>{}, SCL);
          fence();
        } else if constexpr (k % RS == 1 % RS && k / RS < NR) {
          read_a(nxt, rb, T, std::integral_constant<int, k / RS - 8>{});
          fence();
        }
        // upcast part p after MFMA U0 + p (64 - U0) / NU
        static_for(std::make_integer_sequence<int, NU>{}, [&](auto P) {
          constexpr int p = decltype(P)::value;
          if constexpr (U0 + p * (64 - U0) / (NU > 0 ? NU : 1) == k) {
            make_b_part(nxt, std::integral_constant<int, p / 4>{}, std::integral_constant<int, p % 4>{});
            fence();
          }
        });
      });
    };
    auto slot = [&](int s) -> const uint8_t* { return lds + (s % NSTAGE) * STAGE; };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;

    // prologue: NSTAGE stages in flight; stage 0's first-step fragments
#pragma unroll
    for (int st = 0; st < NSTAGE; ++st) issue_all();
    wait_vmcnt<(NSTAGE - 1) * L>();
    asm volatile("s_barrier" ::: "memory");
    Frag X, Y;
    static_for(std::make_integer_sequence<int, 8>{}, [&](auto J) { read_b(X, slot(0), I0{}, J, std::true_type{}); });
    static_for(std::make_integer_sequence<int, 8>{}, [&](auto I) { read_a(X, slot(0), I0{}, I); });
    static_for(std::make_integer_sequence<int, 8>{}, [&](auto J) {
      static_for(std::make_integer_sequence<int, 4>{}, [&](auto JJ) { make_b_part(X, J, JJ); });
    });

    // One stage: step 0 on X (reading step 1 of the same slot into Y); when stage s + 1
    // has landed (this wave's loads, then every wave's) and every wave's reads of slot
    // s are done, a barrier; step 1 on Y, which issues stage s + NSTAGE into slot s
    // and reads step 0 of stage s + 1 into X (its scales when SCL; past the last
    // stage: copies that are never used).
#define QG_BIG_STAGE(s, SCL)                                                    \
  do {                                                                          \
    step(X, Y, slot(s), I1{}, std::false_type{}, std::false_type{});          \
    wait_vm_lgkm0<(NSTAGE - 2) * L>();                                        \
    asm volatile("s_barrier" ::: "memory");                                   \
    step(Y, X, slot((s) + 1), I0{}, std::true_type{}, SCL{});                 \
  } while (0)
    if constexpr (I4) {
      // int4: a superblock is two stages and a part is whole superblocks, so the loop
      // takes two stages per iteration.  Scale groups are whole superblocks (or all of
      // K): the scales change only at even stages of the part, and odd stages keep the
      // registers of the stage before.
      for (int s = 0; s < nst; s += 2) {
        QG_BIG_STAGE(s, std::false_type);
        QG_BIG_STAGE(s + 1, std::true_type);
      }
    } else {
      for (int s = 0; s < nst; ++s) QG_BIG_STAGE(s, std::true_type);
    }
#undef QG_BIG_STAGE
    wait_vmcnt<0>();  // drain the tail copies before the workgroup's LDS is released
  }
  if constexpr (FOLD) {
    // The zero points, applied after the loop: acc += sum over groups g of R[m, g]
    // P[g, n] with P = -(z - r) s - d (the part of the zero point and the rounding of
    // the fma's addend that the loop left, see nc; R: the rows of A summed over each
    // group), on the matrix
    // cores with split bf16 operands, R_hi P_hi + R_hi P_lo + R_lo P_hi (about 16
    // significant bits, and the fp32 range), both read from the planes a pass over A
    // and the scale table wrote before this kernel.  The groups are the K of these
    // products: lane group q of step kk takes groups 32 kk + 8 q .. + 7 in both
    // operands.  Only part 0 adds it.
    if (part == 0) {
      const int gp = a.zr_gp;
      auto mma_bf16 = [&acc](const uint4& x, const uint4& y, auto K) {
        constexpr int k = decltype(K)::value, i = k % 8, j = k / 8;
        // wait states first, in case the compiler copied an operand just before
        asm volatile("s_nop 4\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                     : "+a"(acc[i][j])
                     : "v"(__builtin_bit_cast(int4v, x)), "v"(__builtin_bit_cast(int4v, y)));
      };
      for (int kk = 0; kk < gp / 32; ++kk) {
        const int g0 = kk * 32 + q * 8;
        uint4 rh[8], rl[8], ph[8], pl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int row = min(m0 + wm * 128 + i * 16 + l16, a.M - 1);
          const uint16_t* r = a.zr + (size_t)row * 2 * gp + g0;
          rh[i] = *reinterpret_cast<const uint4*>(r);
          rl[i] = *reinterpret_cast<const uint4*>(r + gp);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int col = n0 + wn * 128 + j * 16 + l16;  // < Npad
          const uint16_t* pz = a.zp + (size_t)col * 2 * gp + g0;
          ph[j] = *reinterpret_cast<const uint4*>(pz);
          pl[j] = *reinterpret_cast<const uint4*>(pz + gp);
        }
        static_for(std::make_integer_sequence<int, 64>{}, [&](auto K) { mma_bf16(rh[K % 8], ph[K / 8], K); });
        static_for(std::make_integer_sequence<int, 64>{}, [&](auto K) { mma_bf16(rh[K % 8], pl[K / 8], K); });
        static_for(std::make_integer_sequence<int, 64>{}, [&](auto K) { mma_bf16(rl[K % 8], ph[K / 8], K); });
      }
    }
  }
  // the last MFMAs' results are read below: more wait states than any MFMA's passes
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");

  // ---- epilogue: lane l holds rows 4 (l / 16) + r, column l % 16 of each sub-tile.
  // One loop per output mode, so that each unrolls completely and the
  // accumulators stay in registers.
  auto each = [&](auto&& f) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int col = n0 + wn * 128 + j * 16 + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = m0 + wm * 128 + i * 16 + q * 4 + r;
          if (row < a.M && col < a.N) f(row, j, (size_t)row * a.N + col, acc[i][j][r]);
        }
      }
  };
  // The per-column values of this lane's 8 columns (epilogue scale, bias, int8 column
  // scale) are read before any store: C is written through pointers of the types of
  // those arrays, so read between the stores each read would wait behind the stores
  // before it.
  float es[8], bf[8], cs[8];
  int bi[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int col = n0 + wn * 128 + j * 16 + l16;
    const bool in = col < a.N;
    es[j] = FP && a.epi_scale && in ? (float)a.epi_scale[col] : 1.f;
    bf[j] = (FP || a.row_scale) && in ? bias_f(a, col) : 0.f;  // fp16 outputs: fp16 bias
    bi[j] = !FP && !a.row_scale && in ? bias_i(a, col) : 0;
    cs[j] = !FP && a.row_scale && in ? a.col_scale[col] : 0.f;
  }
  if (a.out_mode == OUT_STORE) {
    if constexpr (FP)
      each([&](int, int j, size_t o, float v) { static_cast<_Float16*>(a.C)[o] = (_Float16)(v * es[j] + bf[j]); });
    else if (a.row_scale)
      each([&](int row, int j, size_t o, int v) {  // as dq_out, with the column values above
        static_cast<_Float16*>(a.C)[o] = (_Float16)((float)v * a.row_scale[row] * cs[j] + bf[j]);
      });
    else
      each([&](int, int j, size_t o, int v) { static_cast<int*>(a.C)[o] = v + bi[j]; });
  } else if (a.out_mode == OUT_ATOMIC) {
    if constexpr (FP)
      each([&](int, int j, size_t o, float v) { unsafeAtomicAdd(static_cast<float*>(a.ws) + o, v * es[j]); });
    else each([&](int, int, size_t o, int v) { atomicAdd(int_atomic_target(a) + o, v); });
  } else {
    const size_t po = (size_t)part * a.M * a.N;
    if constexpr (FP) each([&](int, int j, size_t o, float v) { static_cast<float*>(a.ws)[po + o] = v * es[j]; });
    else each([&](int, int, size_t o, int v) { static_cast<int*>(a.ws)[po + o] = v; });
  }
}

template <int FMT, bool SCALED, bool FOLD>
hipError_t launch_big_t(const RunArgs& a, hipStream_t st) {
  const int tiles = ((a.M + 255) / 256) * ((a.N + 255) / 256);
  hipLaunchKernelGGL((mfma_big_kernel<FMT, SCALED, FOLD>), dim3(tiles * a.k_parts), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool big_tile_takes(int fmt, const RunArgs& a) {
  // uint4 with zero points only with the group row sums that fold them out of the loop
  return fmt == FMT_F16 || ((fmt == FMT_I4 || fmt == FMT_U4) && !a.zeros) ||
         (fmt == FMT_U4 && a.zeros && a.zr && a.smode == SC_BLOCK);
}

hipError_t launch_mfma_big(int fmt, const RunArgs& a, hipStream_t st) {
  const bool sc = a.smode != SC_NONE;
  switch (fmt) {
    case FMT_F16: return launch_big_t<FMT_F16, false, false>(a, st);
    case FMT_I4:
      if (!sc) return launch_big_t<FMT_I4, false, false>(a, st);
      return a.zr ? launch_big_t<FMT_I4, true, true>(a, st) : launch_big_t<FMT_I4, true, false>(a, st);
    case FMT_U4:
      if (a.zeros) return a.zr && sc ? launch_big_t<FMT_U4, true, true>(a, st) : hipErrorInvalidValue;
      return sc ? launch_big_t<FMT_U4, true, false>(a, st) : launch_big_t<FMT_U4, false, false>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
