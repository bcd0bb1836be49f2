// Direct-load MFMA path (M > 8): BM x BN output tiles (32..256 rows, 64..256
// columns) computed by 4 or 8 waves from a ring of NSTAGE LDS stages that
// global_load_lds_dwordx4 fills straight from memory (lane l's 16 bytes land at
// the instruction's LDS base + 16 l, so no registers or LDS-store instructions
// carry the staging) -- the multi-stage software pipelining of hidet issue #364
// with num_stages = NSTAGE, as deep as the 160 KiB of LDS allows for the tile.
//
// A stage covers SPOS reduction positions: half a superblock for int4 / int2
// (two MFMA steps), one superblock for fp16 / int8 (one step).  Its 1 KiB
// direct loads are dealt round-robin over the waves, and each wave waits for
// its own count.  Each MFMA step consumes 32 (fp16) or 64 (int8) positions;
// lane group q of a step takes piece q of the fp16 / int8 superblock, or packed
// word 2t + (q >> 1) of piece q & 1 of the int4 / int2 half superblock, and the
// activation fragment reads the same positions, so A and B agree on the K
// order by construction.
//
// Activation rows sit unpadded in LDS with their 16-byte chunks XOR-swizzled
// (chunk c of row r at position c ^ swz(r)), which keeps the fragment reads free
// of bank conflicts; the swizzle is applied on the global side of the direct
// loads.  Group scales (and zero points) of the stage ride along as one more
// direct load into LDS.
//
// Register double buffering: the fragments of the next step are read from LDS
// (and int4 / int2 upcast) while the MFMAs of the current step run.
//
// Small int4 / int2 tiles split K inside the workgroup: KS wave groups take
// stages in turn and meet in LDS at the end (the intra-workgroup block
// reduction that the BitBLAS issue #252 discussion names for skinny dequantised
// shapes).  Each wave then covers a wide slice of the tile, so the fixed cost of
// a stage (barrier, waits, addressing) is spread over many MFMAs, and no weight
// is upcast twice.
//
// Workgroups are numbered so each XCD owns a contiguous band of tiles, swept in
// column-major groups of a few tile rows (L2 reuse of the shared A / B blocks, the
// traversal point of the mKernel AG-GEMM PR #41 discussion).
#include "dl_common.hpp"

namespace qg {
namespace {
using namespace dl;

#ifndef QG_DL_GROUP_M
#define QG_DL_GROUP_M 8
#endif
#ifndef QG_DL_GROUP_M_BIG
#define QG_DL_GROUP_M_BIG 2
#endif
#ifndef QG_DL_MAXST
#define QG_DL_MAXST 16
#endif
// ring depth of the 256 x 256 tiles (fp16 / int8, packed formats), before the LDS fit
#ifndef QG_DL_BIG_ST_F
#define QG_DL_BIG_ST_F 4
#endif
#ifndef QG_DL_BIG_ST_P
#define QG_DL_BIG_ST_P 3
#endif

#ifndef QG_DL_IL
#define QG_DL_IL 1
#endif
// int4 / uint4 tiles of four K groups: issue whole rounds from per-round bases (1) or
// stage by stage (0).  Measured at M = 128, N = K = 4096 (32 x 64 tiles): 22.1 -> 17.5 us;
// the two-group tiles and int2 stayed level or lost 1-3 % with it and keep stages.
#ifndef QG_DL_ROUNDS
#define QG_DL_ROUNDS 1
#endif
#ifndef QG_DL_KG_ORDER
#define QG_DL_KG_ORDER 1
#endif
// int4 / int2 stages: 0 keeps the upcasts in a run after each step's MFMAs,
// 1 spreads them word by word, 2 column block by column block (per tile height)
#ifndef QG_DL_IL_P
#define QG_DL_IL_P 2
#endif
#ifndef QG_DL_IL_P_BIG
#define QG_DL_IL_P_BIG 0
#endif
// int2 256 x 256: word by word (W2A8 16384^3 3620 -> 3289 us; int4 stays in runs,
// 8152 against 8228 us)
#ifndef QG_DL_IL_P_BIG_I2
#define QG_DL_IL_P_BIG_I2 1
#endif
// share (percent) of a step's MFMAs that the side ops are spread over, and
// whether the fragment reads go before the direct loads (1) or after (0)
#ifndef QG_DL_IL_SPAN
#define QG_DL_IL_SPAN 100
#endif
#ifndef QG_DL_IL_READS_FIRST
#define QG_DL_IL_READS_FIRST 0
#endif

// Stage geometry of a tile configuration.
template <int FMT, int BM_, int BN_, int WM_, int WN_, int KS_, bool SCALED>
struct Geo {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, NW = WM * WN;  // waves of one K group
  static constexpr int KS = KS_, NWT = NW * KS;                                // K groups, all waves
  static constexpr bool FP = FMT != FMT_I8 && FMT != FMT_I2;  // fp16 activations
  static constexpr bool PACKED = FMT == FMT_I4 || FMT == FMT_U4 || FMT == FMT_I2;
  static constexpr int KB = kb_of(FMT);
  static constexpr int ESZ = FP ? 2 : 1;
  static constexpr int SPOS = PACKED ? KB / 2 : (QG_DL_WIDE ? 2 * KB : KB);
  static constexpr int NSTEP = SPOS / (FP ? 32 : 64);  // MFMA steps per stage
  static constexpr int ROWB = SPOS * ESZ;              // activation bytes per row per stage
  static constexpr int BSB = SPOS * 1024 / KB;         // weight bytes per 16 columns per stage
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BN / 16 * BSB;
  static constexpr int S_BYTES = SCALED ? 1024 : 0;  // one direct-load slot of scales
  static constexpr int STAGE = A_BYTES + B_BYTES + S_BYTES;
  // 1 KiB slots per stage, dealt round-robin over all the waves
  static constexpr int NS_A = A_BYTES / 1024, NS_B = B_BYTES / 1024;
  static constexpr int A_MAX = (NS_A + NWT - 1) / NWT, B_MAX = (NS_B + NWT - 1) / NWT;
  static constexpr int LMIN = NS_A / NWT + NS_B / NWT;              // fewest loads of a wave per stage
  static constexpr int LMAX = A_MAX + B_MAX + (SCALED ? 1 : 0);    // most (wave 0 adds the scale slot)
  static constexpr int WTM = BM / WM / 16, WTN = BN / WN / 16;
  // ring depth: the 256 x 256 tiles keep their measured depth, the others take
  // as many stages as LDS (and the 6-bit load counter) allows, up to 16, in
  // whole rounds of KS stages
  static constexpr int fit(int n) {
    while (n > 2 && (n * STAGE > 160 * 1024 || (n - KS) * LMAX > 63 || n % KS != 0)) --n;
    return n;
  }
  static constexpr int cap(int n) { return n > 3 * KS ? n : 3 * KS; }
  static constexpr int NSTAGE = BM == 256 ? fit((FMT == FMT_F16 || FMT == FMT_I8) ? QG_DL_BIG_ST_F : QG_DL_BIG_ST_P)
                                          : fit(cap(QG_DL_MAXST));
  static constexpr int SB_PER_STAGE = SPOS > KB ? SPOS / KB : 1;  // superblocks per stage (fp16 / int8)
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "whole 1 KiB slots");
  static_assert(NSTEP == 1 || NSTEP == 2, "one or two MFMA steps per stage");
  static_assert(ROWB == 64 || ROWB == 128, "activation row bytes");
  static_assert(NSTAGE >= 3 * KS || (KS == 1 && NSTAGE >= 2), "ring depth");
  static_assert(KS == 1 || ((KS == 2 || KS == 4) && PACKED), "K groups: 2 or 4, for the two-step int4 / int2 stages");
  static constexpr int RED = NW * WTM * WTN * 64;  // accumulator vectors of one K group
  static_assert((KS - 1) * RED * 16 <= NSTAGE * STAGE, "K-group reduction fits in the ring");
};

// s_waitcnt vmcnt(MUL * n) lgkmcnt(0) for a wave-uniform n in [LO, HI]
template <int LO, int HI, int MUL>
__device__ __forceinline__ void wait_loads(int n) {
  if constexpr (LO == HI) {
    wait_vm_lgkm0<MUL * LO>();  // every wave issues the same count
  } else {
    static_for(std::make_integer_sequence<int, HI - LO + 1>{}, [&](auto T) {
      constexpr int v = LO + decltype(T)::value;
      if (n == v) wait_vm_lgkm0<MUL * v>();
    });
  }
}

template <int FMT, class G, bool SCALED, bool ZEROS>
__global__ __launch_bounds__(G::NWT * 64) void mfma_dl_kernel(RunArgs a) {
  constexpr bool FP = G::FP, PACKED = G::PACKED;
  constexpr bool I4 = (FMT == FMT_I4 || FMT == FMT_U4);
  constexpr int BM = G::BM, BN = G::BN, WN = G::WN, NW = G::NW, KS = G::KS, NWT = G::NWT;
  constexpr int WTM = G::WTM, WTN = G::WTN;
  constexpr int SPOS = G::SPOS, ROWB = G::ROWB, BSB = G::BSB, NSTAGE = G::NSTAGE, NSTEP = G::NSTEP;
  constexpr int KB = G::KB, ESZ = G::ESZ;
  constexpr int A_BYTES = G::A_BYTES, B_BYTES = G::B_BYTES, STAGE = G::STAGE;
  constexpr int ILP = BM == 256 ? (FMT == FMT_I2 ? QG_DL_IL_P_BIG_I2 : QG_DL_IL_P_BIG) : QG_DL_IL_P;  // measured
  constexpr int NS_A = G::NS_A, NS_B = G::NS_B, A_MAX = G::A_MAX, B_MAX = G::B_MAX;
  typedef typename std::conditional<FP, float4v, int4v>::type acc_v;

  __shared__ __attribute__((aligned(1024))) uint8_t lds[NSTAGE * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave / NW, wl = wave % NW;  // K group, wave within it
  const int wm = wl / WN, wn = wl % WN;
  const int q = lane >> 4, l16 = lane & 15;

  // ---- tile of this workgroup
  const int tiles_n = (a.N + BN - 1) / BN, tiles_m = (a.M + BM - 1) / BM;
  const int tiles = tiles_m * tiles_n;
  int w = blockIdx.x;
  const int part = w / tiles;
  w -= part * tiles;
  if ((tiles & 7) == 0) w = (w & 7) * (tiles >> 3) + (w >> 3);
  // column-major groups of tile rows: 2 for the 256-row tiles (their A row blocks
  // then stay in the last-level cache between column sweeps), 8 otherwise
  constexpr int GROUP_M = BM == 256 ? QG_DL_GROUP_M_BIG : QG_DL_GROUP_M;
  const int group = w / (GROUP_M * tiles_n);
  const int first_m = group * GROUP_M;
  const int gsz = min(tiles_m - first_m, GROUP_M);
  const int in_group = w - group * GROUP_M * tiles_n;
  const int m0 = (first_m + in_group % gsz) * BM, n0 = (in_group / gsz) * BN;

  // ---- stages of this k-part
  // stages per split unit (a unit is a whole number of stages)
  int u0, u1;
  part_units(a, part, u0, u1);
  const int s0 = u0 * a.unit_kb * KB / SPOS, s1 = u1 * a.unit_kb * KB / SPOS;  // global stage indices
  const int nst = s1 - s0;

  const uint8_t* __restrict__ Ab = static_cast<const uint8_t*>(a.A);
  const uint32_t a_row_bytes = (uint32_t)a.K * ESZ;  // the plan keeps M * K * ESZ below 4 GiB
  const uint8_t* __restrict__ Wb = reinterpret_cast<const uint8_t*>(a.W);
  constexpr int bytes_per_scale = ZEROS ? 4 : 2;

  // This wave's 1 KiB slots of a stage: A slots i * NWT + wave < NS_A, then B
  // slots likewise; wave 0 also loads the scale slot.
  const int la = (NS_A - wave + NWT - 1) / NWT, lb = (NS_B - wave + NWT - 1) / NWT;
  const int my_loads = la + lb + ((SCALED && wave == 0) ? 1 : 0);

  // Per-lane 32-bit offset of each direct load from its stage's source, which is
  // wave-uniform (the loads take the scalar-base form: no per-lane address
  // arithmetic per stage).  A: one slot covers 1024 / ROWB rows.
  constexpr int CPR = ROWB / 16;
  uint32_t a_off[A_MAX];
#pragma unroll
  for (int i = 0; i < A_MAX; ++i) {
    const int sl = min(i * NWT + wave, NS_A - 1);
    const int c16 = sl * 64 + lane;  // 16-byte slot in the stage's A area
    const int r = c16 / CPR, p = c16 % CPR;
    // chunk swz(r, p) of the row belongs at position p
    a_off[i] = (uint32_t)min(m0 + r, a.M - 1) * a_row_bytes + (uint32_t)swz<ROWB, PACKED>(r, p) * 16;
  }
  // B: byte o of the stage's weight area is column block o / BSB, byte o % BSB of
  // it (plus the half-superblock offset of the stage when BSB = 512)
  uint32_t b_off[B_MAX];
#pragma unroll
  for (int i = 0; i < B_MAX; ++i) {
    const int sl = min(i * NWT + wave, NS_B - 1);
    const int o = (sl * 64 + lane) * 16;
    if constexpr (BSB <= 1024) {
      b_off[i] = ((n0 >> 4) + o / BSB) * 1024 + o % BSB;
    } else {
      // superblock o % BSB / 1024 of the stage: the next superblock row of the blob
      const int w = o % BSB;
      b_off[i] = ((n0 >> 4) + o / BSB) * 1024 + (w >> 10) * a.NB * 1024 + (w & 1023);
    }
  }
  // scales: (scale[, zero]) of columns n0 .. n0 + BN - 1, up to 1 KiB (lanes past
  // the end re-read the last 16 bytes into the unused part of the slot)
  const uint32_t s_off = (uint32_t)min(lane * 16, BN * bytes_per_scale - 16);

  // The next stage to issue: its ring slot and its wave-uniform sources.  Stages
  // are issued in order, so each advances the previous one by constant strides;
  // past the part's last stage the sources stay put (clamped copies that are
  // never consumed).
  struct StageSrc {
    uint32_t dst;      // LDS byte address of the ring slot
    const uint8_t* a;  // the stage's activation columns (row 0)
    const uint8_t* w;  // the stage's weights (column block 0)
    const uint8_t* s;  // the stage's scale row (column n0)
  };
  const uint32_t lds0 = lds_off(lds), lds_end = lds0 + NSTAGE * STAGE;
  StageSrc next;
  int next_st = 0;    // part-relative index of `next`
  int grp_left = 0;   // stages from `next` to the end of its scale group
  {
    const int64_t pos0 = (int64_t)s0 * SPOS;
    next.dst = lds0;
    next.a = Ab + pos0 * ESZ;
    next.w = Wb + (pos0 / KB) * a.NB * 1024 + (pos0 % KB) * 1024 / KB;
    next.s = nullptr;
    if constexpr (SCALED) {
      int64_t grp = 0;
      grp_left = 1 << 30;  // one group over K
      if (a.group_size > 0) {
        grp = pos0 / a.group_size;
        grp_left = (int)((a.group_size - pos0 % a.group_size) / SPOS);
      }
      next.s = static_cast<const uint8_t*>(a.S) + ((size_t)grp * a.Npad + n0) * bytes_per_scale;
    }
  }
  auto take_stage = [&]() {
    const StageSrc r = next;
    next.dst = next.dst + STAGE == lds_end ? lds0 : next.dst + STAGE;
    if (next_st < nst - 1) {
      next.a += SPOS * ESZ;
      if constexpr (BSB == 512) next.w += (next_st & 1) ? (size_t)a.NB * 1024 - 512 : (size_t)512;
      else next.w += (size_t)G::SB_PER_STAGE * a.NB * 1024;
      if constexpr (SCALED) {
        if (--grp_left == 0) {
          next.s += (size_t)a.Npad * bytes_per_scale;
          grp_left = a.group_size / SPOS;
        }
      }
    }
    ++next_st;
    return r;
  };
  // this wave's direct load e of a stage: A slots, then B slots, then (wave 0) scales
  constexpr int NDMA = A_MAX + B_MAX + (SCALED ? 1 : 0);
  auto dma_one = [&](const StageSrc& sa, auto E) {
    constexpr int e = decltype(E)::value;
    if constexpr (e < A_MAX) {
      if (NS_A % NWT == 0 || e < la) dma16s(sa.a, a_off[e], sa.dst + (e * NWT + wave) * 1024);
    } else if constexpr (e < A_MAX + B_MAX) {
      constexpr int i = e - A_MAX;
      if (NS_B % NWT == 0 || i < lb) dma16s(sa.w, b_off[i], sa.dst + A_BYTES + (i * NWT + wave) * 1024);
    } else if (wave == 0) {
      dma16s(sa.s, s_off, sa.dst + A_BYTES + B_BYTES);
    }
  };
  auto issue = [&]() {
    const StageSrc sa = take_stage();
    static_for(std::make_integer_sequence<int, NDMA>{}, [&](auto E) { dma_one(sa, E); });
  };

  // Round issue (four K groups, int4 / uint4 weights).  A superblock is two stages and
  // every part starts on one, so the KS stages of round r (part stages r KS ..
  // r KS + KS - 1) are KS / 2 whole superblocks: stage k reads the round's
  // activation columns + 128 k bytes, half k % 2 of weight superblock row k / 2, and
  // the scales of its group, at most one group boundary into the round (groups are
  // whole superblocks, rounds at most two).  Only waves that own direct loads keep
  // these bases, advanced once per round instead of stage by stage.  A round past
  // the part's last stage issues nothing (the waits then drain all loads); one that
  // ends past it takes the per-stage path above with its clamped copies.
  constexpr bool ROUNDS = QG_DL_ROUNDS && KS == 4 && I4 && BSB == 512 && ROWB == 128;
  constexpr int NR = NSTAGE / KS;  // rounds in the ring
  struct RoundSrc {
    const uint8_t* a;   // activations of the round's first stage
    const uint8_t* w;   // weight superblock row of stages 0, 1
    const uint8_t* w2;  // of stages 2, 3 (KS = 4)
    const uint8_t* s;   // scales of the first stage's group
    int pig;            // position of the first stage in its group
    uint32_t dst;       // ring slot of the first stage
  } rs{};
  const int grp_pos = SCALED && a.group_size > 0 ? a.group_size : (1 << 30);  // positions per group
  const size_t srow = (size_t)a.Npad * bytes_per_scale;
  const size_t sbrow = (size_t)a.NB * 1024;  // one superblock row of the blob
  if constexpr (ROUNDS) {
    rs.dst = next.dst;
    rs.a = next.a;
    rs.w = next.w;
    rs.w2 = next.w + sbrow;
    rs.s = next.s;
    rs.pig = SCALED && a.group_size > 0 ? (int)(((int64_t)s0 * SPOS) % a.group_size) : 0;
  }
  auto issue_round = [&](int ri) {
    if (ri * KS >= nst) return;  // past the part: nothing
    if (ri * KS + KS > nst) {
      // the part ends inside this round: stage by stage with clamped sources
      next.dst = rs.dst;
      next.a = rs.a;
      next.w = rs.w;
      next.s = rs.s;
      grp_left = (grp_pos - rs.pig) / SPOS;
      next_st = ri * KS;
#pragma unroll
      for (int k = 0; k < KS; ++k) issue();
      return;
    }
    static_for(std::make_integer_sequence<int, KS>{}, [&](auto K) {
      constexpr int k = decltype(K)::value;
      const uint32_t dst = rs.dst + k * STAGE;
      static_for(std::make_integer_sequence<int, NDMA>{}, [&](auto E) {
        constexpr int e = decltype(E)::value;
        if constexpr (e < A_MAX) {
          if (NS_A % NWT == 0 || e < la) dma16s(rs.a, a_off[e] + k * 128, dst + (e * NWT + wave) * 1024);
        } else if constexpr (e < A_MAX + B_MAX) {
          constexpr int i = e - A_MAX;
          if (NS_B % NWT == 0 || i < lb)
            dma16s(k < 2 ? rs.w : rs.w2, b_off[i] + (k % 2) * 512, dst + A_BYTES + (i * NWT + wave) * 1024);
        } else if (wave == 0) {
          const uint8_t* sp = rs.pig + k * SPOS >= grp_pos ? rs.s + srow : rs.s;
          dma16s(sp, s_off, dst + A_BYTES + B_BYTES);
        }
      });
    });
    // advance the bases by one round
    rs.dst = rs.dst + KS * STAGE == lds_end ? lds0 : rs.dst + KS * STAGE;
    rs.a += KS * 128;
    rs.w += (KS / 2) * sbrow;
    if constexpr (KS == 4) rs.w2 += 2 * sbrow;
    if constexpr (SCALED) {
      rs.pig += KS * SPOS;
      if (rs.pig >= grp_pos) {
        rs.pig -= grp_pos;
        rs.s += srow;
      }
      if (rs.pig >= grp_pos) {
        rs.pig -= grp_pos;
        rs.s += srow;
      }
    }
  };

  acc_v acc[WTM][WTN];
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) acc[i][j] = acc_v{0, 0, 0, 0};

  struct Frag {
    uint4 a[WTM];  // activation fragments (16 rows each)
    uint4 b[WTN];  // MFMA-ready weight fragments (16 columns each)
  };
  // int4 / int2: the packed word a lane feeds to an MFMA step, per column block
  uint32_t rw[WTN];
  uint32_t sc[WTN], zc[WTN];

  auto slot = [&](int s) -> const uint8_t* { return lds + (s % NSTAGE) * STAGE; };

  // Round rn (stages rn * KS .. rn * KS + KS - 1, one per K group) becomes
  // readable: this wave's loads of it are done when at most NSTAGE - 2 KS later
  // stages of loads are outstanding, and lgkmcnt(0) retires this wave's LDS reads
  // of the round held in registers, whose ring slots the loads issued after the
  // barrier overwrite.  A bare s_barrier (a compiler memory barrier through the
  // clobber) instead of __syncthreads, whose fence would drain the loads still in
  // flight.
  auto sync_round = [&](int rn) {
    (void)rn;  // its stages (rn * KS + NSTAGE - KS ..) are the next KS to issue
    wait_loads<G::LMIN, G::LMAX, NSTAGE - 2 * KS>(my_loads);
    asm volatile("s_barrier" ::: "memory");
#pragma unroll
    for (int k = 0; k < KS; ++k) issue();
  };

  // keeps the machine scheduler from moving instructions across it, so that the
  // reads of the next fragments issue before the MFMAs of the current ones and no
  // MFMA of the next step is hoisted above the barrier that guards its data
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };

  // fragment pieces of step t of the stage in the slot at base: activation rows
  // i (16 each), then the weights of column block j (with the stage's scales
  // when t = 0)
  auto read_a = [&](Frag& f, const uint8_t* base, auto T, auto I) {
    constexpr int t = decltype(T)::value, i = decltype(I)::value;
    int chunk;
    if constexpr (PACKED) chunk = (q & 1) * 4 + (2 * t + (q >> 1));  // piece q & 1, word 2t + (q >> 1)
    else chunk = t * 4 + q;  // 8 fp16 / 16 int8 per lane group, four groups per step
    const int r = (wm * WTM + i) * 16 + l16;
    f.a[i] = *reinterpret_cast<const uint4*>(base + r * ROWB + swz<ROWB, PACKED>(r, chunk) * 16);
  };
  auto read_b = [&](Frag& f, const uint8_t* base, auto T, auto J) {
    constexpr int t = decltype(T)::value, j = decltype(J)::value;
    const uint8_t* lb = base + A_BYTES + (wn * WTN + j) * BSB;
    if constexpr (PACKED)
      rw[j] = *reinterpret_cast<const uint32_t*>(lb + ((q & 1) * 16 + l16) * 16 + (2 * t + (q >> 1)) * 4);
    else
      f.b[j] = *reinterpret_cast<const uint4*>(lb + t * 1024 + lane * 16);  // superblock t, piece = lane
    if constexpr (SCALED && t == 0) {
      const int col = (wn * WTN + j) * 16 + l16;
      if constexpr (ZEROS) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(base + A_BYTES + B_BYTES + col * 4);
        sc[j] = __builtin_amdgcn_perm(u, u, 0x01000100u);  // low half in both halves
        zc[j] = __builtin_amdgcn_perm(u, u, 0x03020302u);  // high half in both halves
      } else {
        const uint32_t u = *reinterpret_cast<const uint16_t*>(base + A_BYTES + B_BYTES + col * 2);
        sc[j] = __builtin_amdgcn_perm(u, u, 0x01000100u);
        zc[j] = 0;
      }
    }
  };
  // (the weight words first: the upcasts that wait for them then leave the
  // activation reads in flight)
  auto read_step = [&](Frag& f, int s, auto T) {
    const uint8_t* base = slot(s);
    static_for(std::make_integer_sequence<int, WTN>{}, [&](auto J) { read_b(f, base, T, J); });
    if constexpr (QG_DL_KG_ORDER) fence();
    static_for(std::make_integer_sequence<int, WTM>{}, [&](auto I) { read_a(f, base, T, I); });
  };

  // upcast of word jj of column block j's MFMA operand from its packed word
  // (int4 / int2 only)
  auto make_b_part = [&](Frag& f, auto J, auto JJ) {
    constexpr int j = decltype(J)::value, jj = decltype(JJ)::value;
    if constexpr (PACKED) {
      const uint32_t wd = rw[j];
      uint32_t o;
      if constexpr (I4) {
        constexpr uint32_t bias = (FMT == FMT_I4) ? 0x64086408u : 0x64006400u;
        half2v v = as_h2(and_or(wd >> (4 * jj), 0x000F000Fu, 0x64006400u)) - as_h2(bias);
        if constexpr (ZEROS) v = v - as_h2(zc[j]);
        if constexpr (SCALED) v = v * as_h2(sc[j]);
        o = as_u32(v);
      } else if constexpr (jj < 3) {
        // offset-binary classes: 0,1,2,3 -> -2,-1,0,1
        o = __builtin_amdgcn_perm(0u, 0x0100FFFEu, (wd >> (2 * jj)) & 0x03030303u);
      } else {
        // two's complement class: 0,1,2,3 -> 0,1,-2,-1
        o = __builtin_amdgcn_perm(0u, 0xFFFE0100u, (wd >> 6) & 0x03030303u);
      }
      // pins the upcast here: otherwise the compiler sinks it into the block of
      // its first use, past the barrier, where it runs as one serial stretch
      asm volatile("" : "+v"(o));
      if constexpr (jj == 0) f.b[j].x = o;
      else if constexpr (jj == 1) f.b[j].y = o;
      else if constexpr (jj == 2) f.b[j].z = o;
      else f.b[j].w = o;
    }
  };
  auto make_b = [&](Frag& f, auto J) {
    static_for(std::make_integer_sequence<int, 4>{}, [&](auto JJ) { make_b_part(f, J, JJ); });
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
  // (each column block's MFMAs issue before the upcast that may wait for its reads)
  auto compute = [&](const Frag& cur, Frag& nxt) {
    fence();
    if constexpr (QG_DL_KG_ORDER) {
      static_for(std::make_integer_sequence<int, WTN>{}, [&](auto J) { mma(cur, decltype(J)::value); });
      fence();
      static_for(std::make_integer_sequence<int, WTN>{}, [&](auto J) { make_b(nxt, J); });
    } else {
      static_for(std::make_integer_sequence<int, WTN>{}, [&](auto J) {
        mma(cur, decltype(J)::value);
        fence();
        make_b(nxt, J);
      });
    }
    fence();
  };

  // one MFMA (sub-tile i, j)
  auto mma1 = [&](const Frag& f, auto I, auto J) {
    constexpr int i = decltype(I)::value, j = decltype(J)::value;
    if constexpr (FP)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          __builtin_bit_cast(half8v, f.a[i]), __builtin_bit_cast(half8v, f.b[j]), acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(
          __builtin_bit_cast(int4v, f.a[i]), __builtin_bit_cast(int4v, f.b[j]), acc[i][j], 0, 0, 0);
  };

  // Interleaved step (one K group): the MFMAs of cur with, spread evenly between
  // them in a fixed order, this wave's direct loads of stage st_dma (when DMA),
  // the fragment reads of step T of the stage in the slot at rb into nxt, and
  // the upcasts of nxt.  After a barrier the wave thus goes straight back to
  // MFMAs instead of first issuing its loads and reads in a run, during which
  // the matrix core of its SIMD would idle.
  auto step_il = [&](const Frag& cur, Frag& nxt, const uint8_t* rb, auto T, auto DMA, int st_dma) {
    constexpr bool dma = decltype(DMA)::value;
    (void)st_dma;  // with DMA: stage st_dma, the next one to issue
    StageSrc sa{};
    if constexpr (dma) sa = take_stage();
    constexpr int UPW = ILP == 2 ? 1 : 4;  // upcast side ops per column block
    constexpr int ND = dma ? NDMA : 0, NU = PACKED ? UPW * WTN : 0;
    constexpr int NM = WTM * WTN;
    // With tall wave tiles (16 row fragments) the next activation fragments
    // cannot be held beside the current ones: fragment i is re-read right after
    // its last MFMA (column block WTN - 1), and the other side ops are spread
    // over the MFMAs before that.
    constexpr bool LATE_A = WTM >= 16 && WTN >= 2;
    constexpr int NEARLY = LATE_A ? (WTN - 1) * WTM : NM;  // MFMAs that carry the other side ops
    constexpr int NSIDE = ND + (LATE_A ? 0 : WTM) + WTN + NU;
    constexpr int NCARRY = NEARLY * QG_DL_IL_SPAN / 100 > 0 ? NEARLY * QG_DL_IL_SPAN / 100 : 1;
    fence();
    static_for(std::make_integer_sequence<int, NM>{}, [&](auto K) {
      constexpr int k = decltype(K)::value;
      mma1(cur, std::integral_constant<int, k % WTM>{}, std::integral_constant<int, k / WTM>{});
      fence();
      if constexpr (LATE_A && k >= NEARLY) {
        read_a(nxt, rb, T, std::integral_constant<int, k - NEARLY>{});
        fence();
      } else {
        constexpr int e0 = k < NCARRY ? k * NSIDE / NCARRY : NSIDE;
        constexpr int e1 = k < NCARRY ? (k + 1) * NSIDE / NCARRY : NSIDE;
        static_for(std::make_integer_sequence<int, e1 - e0>{}, [&](auto E) {
          constexpr int e = e0 + decltype(E)::value;
          constexpr int NA = LATE_A ? 0 : WTM;
          // side op e: reads (A then B) and direct loads in the chosen order, then upcasts
          constexpr int RF = QG_DL_IL_READS_FIRST;
          constexpr int er = RF ? e : e - ND;       // index among the reads
          constexpr int ed = RF ? e - NA - WTN : e;  // index among the direct loads
          if constexpr (e < ND + NA + WTN && ((RF && e >= NA + WTN) || (!RF && e < ND)))
            dma_one(sa, std::integral_constant<int, ed>{});
          else if constexpr (e < ND + NA + WTN && er < NA)
            read_a(nxt, rb, T, std::integral_constant<int, er>{});
          else if constexpr (e < ND + NA + WTN)
            read_b(nxt, rb, T, std::integral_constant<int, er - NA>{});
          else if constexpr (UPW == 1) make_b(nxt, std::integral_constant<int, e - ND - NA - WTN>{});
          else make_b_part(nxt, std::integral_constant<int, (e - ND - NA - WTN) / 4>{},
                           std::integral_constant<int, (e - ND - NA - WTN) % 4>{});
          fence();
        });
      }
    });
  };
  // waits until round rn's loads have landed everywhere (see sync_round)
  auto barrier_round = [&] {
    wait_loads<G::LMIN, G::LMAX, NSTAGE - 2 * KS>(my_loads);
    asm volatile("s_barrier" ::: "memory");
  };

  // prologue: NSTAGE stages in flight, then the fragments of step 0
  if constexpr (ROUNDS) {
    if (my_loads > 0) {
#pragma unroll
      for (int r = 0; r < NR; ++r) issue_round(r);
    }
    if ((NR - 1) * KS < nst) wait_loads<G::LMIN, G::LMAX, NSTAGE - KS>(my_loads);
    else wait_vm_lgkm0<0>();  // some rounds of the ring were not issued
  } else {
#pragma unroll
    for (int st = 0; st < NSTAGE; ++st) issue();
    wait_loads<G::LMIN, G::LMAX, NSTAGE - KS>(my_loads);
  }
  asm volatile("s_barrier" ::: "memory");

  Frag X, Y;
  read_step(X, kg, std::integral_constant<int, 0>{});
  static_for(std::make_integer_sequence<int, WTN>{}, [&](auto J) { make_b(X, J); });

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  if constexpr (QG_DL_IL && NSTEP == 1) {
    // one step per stage: each step is preceded by the barrier of the next stage
    int s = 0;
    for (; s + 1 < nst; s += 2) {
      barrier_round();
      step_il(X, Y, slot(s + 1), I0{}, std::true_type{}, s + NSTAGE);
      barrier_round();  // past the last stage this reads clamped copies that are never used
      step_il(Y, X, slot(s + 2), I0{}, std::true_type{}, s + 1 + NSTAGE);
    }
    if (s < nst) compute(X, Y);
  } else if constexpr (QG_DL_IL && (ILP != 0 || !PACKED) && KS == 1) {
    // two steps per stage: step 0 reads step 1 of the same stage, step 1 follows
    // the barrier of the next stage and reads its step 0
    for (int s = 0; s < nst; ++s) {
      step_il(X, Y, slot(s), I1{}, std::false_type{}, 0);
      barrier_round();  // past the last stage this reads clamped copies that are never used
      step_il(Y, X, slot(s + 1), I0{}, std::true_type{}, s + NSTAGE);
    }
  } else if constexpr (NSTEP == 1) {
    // one MFMA step per stage, two stages per iteration
    int s = 0;
    for (; s + 1 < nst; s += 2) {
      sync_round(s + 1);
      fence();
      read_step(Y, s + 1, std::integral_constant<int, 0>{});
      compute(X, Y);
      sync_round(s + 2);  // past the last stage this reads clamped copies that are never used
      fence();
      read_step(X, s + 2, std::integral_constant<int, 0>{});
      compute(Y, X);
    }
    if (s < nst) compute(X, Y);
  } else {
    // two MFMA steps per stage: X holds step 0 of this group's stage of round r,
    // Y step 1.  In a last, partial round the groups past the end only keep the
    // barriers (their reads hit clamped copies and are not used).
    const int nr = (nst + KS - 1) / KS;
    for (int r = 0; r < nr; ++r) {
      const int s = r * KS + kg;
      const bool live = KS == 1 || s < nst;
      fence();
      read_step(Y, s, std::integral_constant<int, 1>{});
      if (live) compute(X, Y);
      if constexpr (ROUNDS) {
        // round r + 1 landed: rounds r + 2 .. r + NR - 1 may still be in flight, when
        // they were issued; then round r + NR into the slots of round r
        if ((r + NR - 1) * KS < nst) wait_loads<G::LMIN, G::LMAX, NSTAGE - 2 * KS>(my_loads);
        else wait_vm_lgkm0<0>();
        asm volatile("s_barrier" ::: "memory");
        if (my_loads > 0) issue_round(r + NR);
      } else {
        sync_round(r + 1);  // past the last round this reads clamped copies that are never used
      }
      fence();
      read_step(X, s + KS, std::integral_constant<int, 0>{});
      if (live) compute(Y, X);
    }
  }
  wait_vmcnt<0>();  // drain the clamped tail loads before the workgroup's LDS is released

  if constexpr (KS > 1) {
    // K groups 1.. hand their partial sums to group 0 through the (now idle)
    // ring, which adds them in group order
    __syncthreads();
    acc_v* red = reinterpret_cast<acc_v*>(lds);
    if (kg > 0) {
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j) red[(kg - 1) * G::RED + ((wl * WTM + i) * WTN + j) * 64 + lane] = acc[i][j];
    }
    __syncthreads();
    if (kg != 0) return;
#pragma unroll
    for (int g = 1; g < KS; ++g)
#pragma unroll
      for (int i = 0; i < WTM; ++i)
#pragma unroll
        for (int j = 0; j < WTN; ++j) acc[i][j] += red[(g - 1) * G::RED + ((wl * WTM + i) * WTN + j) * 64 + lane];
  }

  // epilogue: lane l holds rows 4 (l / 16) + r, column l % 16 of each 16 x 16 sub-tile.
  // The per-column values (bias, epilogue scale, int8 column scale) are read before any
  // store: C is written through pointers of the types of those arrays, so read between
  // the stores each read would wait behind the stores before it.
  float bfv[WTN], esv[WTN], csv[WTN];
  int biv[WTN];
#pragma unroll
  for (int j = 0; j < WTN; ++j) {
    const int col = n0 + (wn * WTN + j) * 16 + l16;
    const bool st = col < a.N && a.out_mode == OUT_STORE;
    bfv[j] = (FP || a.row_scale) && st ? bias_f(a, col) : 0.f;  // fp16 outputs: fp16 bias
    biv[j] = !FP && !a.row_scale && st ? bias_i(a, col) : 0;
    csv[j] = !FP && a.row_scale && st ? a.col_scale[col] : 0.f;
    esv[j] = FP && a.epi_scale && col < a.N ? (float)a.epi_scale[col] : 1.f;
  }
#pragma unroll
  for (int i = 0; i < WTM; ++i)
#pragma unroll
    for (int j = 0; j < WTN; ++j) {
      const int col = n0 + (wn * WTN + j) * 16 + l16;
      if (col >= a.N) continue;
      const float bf = bfv[j], es = esv[j];
      const int bi = biv[j];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = m0 + (wm * WTM + i) * 16 + q * 4 + r;
        if (row >= a.M) continue;
        const size_t o = (size_t)row * a.N + col;
        auto v = acc[i][j][r];
        if constexpr (FP) v *= es;
        if (a.out_mode == OUT_STORE) {
          if constexpr (FP) static_cast<_Float16*>(a.C)[o] = (_Float16)(v + bf);
          else if (a.row_scale)  // as dq_out, with the column values above
            static_cast<_Float16*>(a.C)[o] = (_Float16)((float)v * a.row_scale[row] * csv[j] + bf);
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

// the tile configurations: rows x columns; waves rows x columns x K groups.  Up
// to 128 rows the waves never split the rows, so every weight fragment is
// upcast once per workgroup; int4 / int2 (P) take K groups on the smaller tiles
// and on 128 x 256, fp16 / int8 (F) split the columns (and the rows of 128 x 256).
// Measured against the alternatives at N = K = 16384: fp16 / int8 64 x 128 with 8
// waves instead of 4 (int8 M = 128 73.1 -> 64.3 us, fp16 133 -> 122 us); 128 x 256
// as 2 x 4 waves for fp16 / int8 (M = 512: int8 139 -> 134 us, fp16 267 -> 256 us,
// while int4 went 283 -> 324 us) and 1 x 4 x 2 for int4 / int2 (int4 283 -> 265 us);
// int4 64 x 128 as 1 x 4 x 2 or 1 x 2 x 2 (no register spill) ran M = 128 in
// 121 / 119 against 108 us.
#ifndef QG_DL_WAVES_P_32x64
#define QG_DL_WAVES_P_32x64 1, 2, 4
#endif
#ifndef QG_DL_WAVES_F_32x64
#define QG_DL_WAVES_F_32x64 1, 4, 1
#endif
#ifndef QG_DL_WAVES_P_32x128
#define QG_DL_WAVES_P_32x128 1, 2, 4
#endif
#ifndef QG_DL_WAVES_F_32x128
#define QG_DL_WAVES_F_32x128 1, 4, 1
#endif
#ifndef QG_DL_WAVES_P_32x256
#define QG_DL_WAVES_P_32x256 1, 4, 2
#endif
#ifndef QG_DL_WAVES_F_32x256
#define QG_DL_WAVES_F_32x256 1, 8, 1
#endif
#ifndef QG_DL_WAVES_P_64x128
#define QG_DL_WAVES_P_64x128 1, 2, 4
#endif
#ifndef QG_DL_WAVES_F_64x128
#define QG_DL_WAVES_F_64x128 1, 8, 1
#endif
#ifndef QG_DL_WAVES_P_64x256
#define QG_DL_WAVES_P_64x256 1, 4, 2
#endif
#ifndef QG_DL_WAVES_F_64x256
#define QG_DL_WAVES_F_64x256 1, 8, 1
#endif
#ifndef QG_DL_WAVES_P_128x128
#define QG_DL_WAVES_P_128x128 1, 4, 2
#endif
#ifndef QG_DL_WAVES_F_128x128
#define QG_DL_WAVES_F_128x128 1, 4, 1
#endif
#ifndef QG_DL_WAVES_P_128x256
#define QG_DL_WAVES_P_128x256 1, 4, 2
#endif
#ifndef QG_DL_WAVES_F_128x256
#define QG_DL_WAVES_F_128x256 2, 4, 1
#endif
#ifndef QG_DL_WAVES_P_256x256
#define QG_DL_WAVES_P_256x256 2, 4, 1
#endif
#ifndef QG_DL_WAVES_F_256x256
#define QG_DL_WAVES_F_256x256 2, 4, 1
#endif
template <int FMT, bool SCALED, int T> struct TileGeo;
template <int FMT, int BM, int BN, bool SCALED, int PWM, int PWN, int PKS, int FWM, int FWN, int FKS>
using GeoOf = typename std::conditional<(FMT == FMT_I4 || FMT == FMT_U4 || FMT == FMT_I2),
                                        Geo<FMT, BM, BN, PWM, PWN, PKS, SCALED>,
                                        Geo<FMT, BM, BN, FWM, FWN, FKS, SCALED>>::type;
#define QG_DL_TILE(T, BM, BN, SHAPE)                                                            \
  template <int FMT, bool SCALED> struct TileGeo<FMT, SCALED, T> {                              \
    using type = GeoOf<FMT, BM, BN, SCALED, QG_DL_WAVES_P_##SHAPE, QG_DL_WAVES_F_##SHAPE>;      \
  };
QG_DL_TILE(DL_32x64, 32, 64, 32x64)
QG_DL_TILE(DL_32x128, 32, 128, 32x128)
QG_DL_TILE(DL_32x256, 32, 256, 32x256)
QG_DL_TILE(DL_64x128, 64, 128, 64x128)
QG_DL_TILE(DL_64x256, 64, 256, 64x256)
QG_DL_TILE(DL_128x256, 128, 256, 128x256)
QG_DL_TILE(DL_256x256, 256, 256, 256x256)
QG_DL_TILE(DL_128x128, 128, 128, 128x128)
#undef QG_DL_TILE

template <int FMT, int T, bool SCALED, bool ZEROS>
hipError_t launch_t(const RunArgs& a, hipStream_t st) {
  using G = typename TileGeo<FMT, SCALED, T>::type;
  static_assert((size_t)G::STAGE * G::NSTAGE <= 160 * 1024, "LDS budget");
  const int tiles = ((a.M + G::BM - 1) / G::BM) * ((a.N + G::BN - 1) / G::BN);
  hipLaunchKernelGGL((mfma_dl_kernel<FMT, G, SCALED, ZEROS>), dim3(tiles * a.k_parts), dim3(G::NWT * 64), 0, st,
                     a);
  return hipGetLastError();
}

template <int T>
hipError_t launch_tile(int fmt, const RunArgs& a, hipStream_t st) {
  const bool sc = a.smode != SC_NONE;
  switch (fmt) {
    case FMT_F16: return launch_t<FMT_F16, T, false, false>(a, st);
    case FMT_I8: return launch_t<FMT_I8, T, false, false>(a, st);
    case FMT_I2: return launch_t<FMT_I2, T, false, false>(a, st);
    case FMT_I4: return sc ? launch_t<FMT_I4, T, true, false>(a, st) : launch_t<FMT_I4, T, false, false>(a, st);
    case FMT_U4:
      return !sc ? launch_t<FMT_U4, T, false, false>(a, st)
           : a.zeros ? launch_t<FMT_U4, T, true, true>(a, st) : launch_t<FMT_U4, T, true, false>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

void dl_tile_dims(int tile, int* bm, int* bn) {
  static const int dims[DL_NUM][2] = {{32, 64},  {32, 128},  {32, 256},  {64, 128},
                                      {64, 256}, {128, 256}, {256, 256}, {128, 128}};
  *bm = dims[tile][0];
  *bn = dims[tile][1];
}

int choose_dl_tile(int fmt, int64_t M, int64_t N, int k_parts, int smode) {
  const bool packed = fmt == FMT_I4 || fmt == FMT_U4 || fmt == FMT_I2;
  if (packed && smode == SC_PIECE) return -1;  // one scale slot per stage holds one group per column
  const int cap = M <= 32 ? 32 : M <= 64 ? 64 : M <= 128 ? 128 : 256;
  static const int order[] = {DL_256x256, DL_128x256, DL_128x128, DL_64x256, DL_64x128, DL_32x256, DL_32x128, DL_32x64};
#ifdef QG_FORCE_DL_TILE
  if (QG_FORCE_DL_TILE >= 0) return QG_FORCE_DL_TILE;
#endif
  // The largest tile whose last wave of workgroups still occupies at least 60% of
  // the 256 CUs: larger tiles re-read less of A and B, idle CUs cost in proportion.
  int pick = -1;
  for (int t : order) {
    // 128 x 128 only for int4 / int2 weights, whose upcast it shares over 128 rows
    // (measured at M = 128, N = 32000: 58 -> 50 us for int4)
    if (t == DL_128x128 && !packed) continue;
    int bm, bn;
    dl_tile_dims(t, &bm, &bn);
    if (bm > cap) continue;
    pick = t;
    const int64_t wgs = ((M + bm - 1) / bm) * ((N + bn - 1) / bn) * k_parts;
    const int64_t waves = (wgs + 255) / 256;
    if (wgs * 10 >= waves * 256 * 6) break;
  }
  return pick;
}

hipError_t launch_mfma_dl(int fmt, int tile, const RunArgs& a0, hipStream_t st) {
  // One scale group over K and no zero points: the column scale factors out of the
  // whole sum, so the tiles take the unscaled upcast (exact q rather than q * s rounded
  // to fp16) and the epilogue scales the fp32 sum; W4A16 g = -1 at 16384^3 then runs
  // like g = 0
  RunArgs a = a0;
  if ((fmt == FMT_I4 || fmt == FMT_U4) && a.smode == SC_BLOCK && a.group_size < 0 && !a.zeros) {
    a.epi_scale = static_cast<const _Float16*>(a.S);
    a.smode = SC_NONE;
  }
  switch (tile) {
    case DL_32x64: return launch_tile<DL_32x64>(fmt, a, st);
    case DL_32x128: return launch_tile<DL_32x128>(fmt, a, st);
    case DL_32x256: return launch_tile<DL_32x256>(fmt, a, st);
    case DL_64x128: return launch_tile<DL_64x128>(fmt, a, st);
    case DL_64x256: return launch_tile<DL_64x256>(fmt, a, st);
    case DL_128x256: return launch_tile<DL_128x256>(fmt, a, st);
    case DL_256x256:
      // fp16 and int4 / uint4 without zero points: four waves of 128 x 128 (measured
      // at 16384^3: fp16 6.66 -> 6.41 ms, int4 6.34 -> 5.82 ms); the others keep
      // eight waves of 128 x 64, which measured faster for them
      return QG_BIG4 && big_tile_takes(fmt, a) ? launch_mfma_big(fmt, a, st) : launch_tile<DL_256x256>(fmt, a, st);
    case DL_128x128: return launch_tile<DL_128x128>(fmt, a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace qg
