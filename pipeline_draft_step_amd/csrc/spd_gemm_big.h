// Large-M GEMM for prefill-sized products: C[M][N] = rs[m] * (A[M][K] . B[N][K]^T),
// A and B bf16 with K contiguous (A = activations, B = weights), C fp32.
//
// Block tile 256 x 160, eight waves, two per SIMD: wave v owns rows
// 64 (v % 4) .. +63 and columns 80 (v / 4) .. +79 as 4 x 5 tiles of the
// 16x16x32 bf16 MFMA (80 accumulator registers).  With two waves on each SIMD
// one wave's LDS reads and load issue overlap the other's MFMAs.  K advances in
// 64-wide stages through a ring of three LDS buffers filled with direct
// global->LDS loads (global_load_lds_dwordx4: lane l of an instruction lands at
// LDS offset 16 l) two stages ahead; each wave spreads its share of a stage's
// loads through its MFMAs.  A tile row is 128 bytes held as eight 16-byte
// chunks in the order chunk ^ (row & 7): of the XOR patterns measured for the
// 16-row fragment reads this one streams fastest.
//
// Large tiles halve the bytes each CU pulls through its load path per flop, and
// the K range is split KS ways to still give every CU a block: the KS blocks of
// one tile write fp32 partial tiles, and the last one to arrive adds them in
// the fixed order 0 .. KS-1 and writes C.  Blocks are dealt to the XCDs round
// robin (block b runs on XCD b mod 8); block ids are remapped so that each XCD
// holds all KS parts of its tiles and a compact patch of tiles, which keeps the
// partials and the shared operand rows in that XCD's L2.
//
// LO8 kernels take A as [hi | lo8] rows (bf16 parts, then e4m3 residuals) and B
// twice (bf16 W and its e4m3 copy B8 with per-row E8M0 scales): every 128 columns
// are two bf16 stages and one fp8 stage of the same 52 KB, the fp8 stage on the
// 16x16x128 block-scaled MFMA, with the kinds tied to the three ring slots.
#pragma once

#include "spd_common.h"

namespace spd {

constexpr int BG_BM = 256, BG_BN = 160, BG_BK = 64;
constexpr int BG_THREADS = 512;
constexpr int BG_SLOTS = 3;
constexpr int BG_ROW = BG_BK * 2;                 // bytes per tile row and stage
constexpr int BG_A_BYTES = BG_BM * BG_ROW;        // 32 KB
constexpr int BG_B_BYTES = BG_BN * BG_ROW;        // 20 KB
constexpr int BG_STAGE_BYTES = BG_A_BYTES + BG_B_BYTES;
constexpr int BG_A_GROUPS = BG_A_BYTES / 1024;    // 1 KB load groups of a stage
constexpr int BG_GROUPS = BG_STAGE_BYTES / 1024;  // 52
constexpr int BG_WAVES = BG_THREADS / 64;
constexpr int BG_LOADS = (BG_GROUPS + BG_WAVES - 1) / BG_WAVES;  // per wave and stage: 7
constexpr int BG_MFMAS = 2 * 4 * 5;                              // per wave and stage
constexpr int BG_FRAGS = 20;                      // 16x16 accumulator tiles per wave
constexpr int BG_PART_FLOATS = BG_BM * BG_BN;     // one partial tile
constexpr int BG_MAX_KS = 4;
static_assert(BG_SLOTS * BG_STAGE_BYTES <= 160 * 1024, "LDS ring");

struct BigGemm {
  const bf16* A;       // [M][lda]
  const bf16* B;       // [N][ldb]
  float* C;            // [M][ldc]
  const float* rs;     // [M] row scales, or nullptr
  float* part;         // [tiles][KS][BG_PART_FLOATS] when KS > 1
  unsigned* counters;  // [tiles], zero on entry, left zero
  int M, N, K, lda, ldb, ldc;
  int kb;  // B's K: for K = 2 kb, A's row is [hi | lo] and B's columns repeat
  int mtiles, ntiles, KS;
  int kstages;  // 64-wide K stages per block (K / (64 KS))
  // row statistics of A (RSQ kernels): C rows scaled by 1 / sqrt(sum_k A^2 / rs_k + rs_eps)
  float* sqp;  // [tiles][KS][BG_BM] partial sums of squares when KS > 1
  int rs_k;
  float rs_eps;
  // gate/up with SwiGLU (BG_EPI_SWIGLU): B = [gate; up] with `half` rows each; a tile
  // takes 80 gate rows and the matching 80 up rows and writes silu(gate) * up as
  // [hi | lo] bf16 rows of act (row stride act_ld) instead of C
  bf16* act;
  int act_ld, half;
  // [hi | lo8] activation rows (LO8 kernels): A's row holds kb bf16 hi parts, then at
  // byte 2 kb the kb bytes lo8 = e4m3(256 (x - hi)).  Each 128 columns take two bf16
  // stages (hi parts times B) and one fp8 stage (the same 128 bytes per tile row: lo8
  // times B8 = e4m3(W_n 2^e_n), [N][kb] bytes) on the block-scaled fp8 MFMA, whose
  // scales (2^-8 for A, b8s[n] = 127 - e_n for row n of B, E8M0) undo both factors
  // exactly.
  const unsigned char* B8;
  const unsigned char* b8s;
};

// E8M0 scale of the lo8 operand: 2^(119 - 127) undoes its factor 256
constexpr int BG_LO8_ASCALE = 119;

// lo8 parts: e4m3 (round to nearest even) of 256 r, saturated to +-448; |r| is at
// most 2^-8 |x| for the residual r = x - bf16(x), so only |x| > 448 saturates.
__device__ __forceinline__ float lo8_arg(float r) { return fminf(fmaxf(256.f * r, -448.f), 448.f); }
__device__ __forceinline__ uint32_t lo8_byte(float r) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(lo8_arg(r), 0.f, 0, false) & 0xffu;
}
// four residuals as four bytes, r0 lowest
__device__ __forceinline__ uint32_t lo8_word(float r0, float r1, float r2, float r3) {
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(lo8_arg(r0), lo8_arg(r1), 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(lo8_arg(r2), lo8_arg(r3), v, true);
  return (uint32_t)v;
}

enum { BG_EPI_PLAIN = 0, BG_EPI_RSQ = 1, BG_EPI_SWIGLU = 2 };

typedef f32x4 BgAccT;

typedef void __attribute__((address_space(3))) * lds_ptr_t;

__device__ __forceinline__ int bg_swz(int r) { return r & 7; }

// Wave v issues its share of the loads of K stage `st` into the stage buffer
// `base`: 1 KB groups (8 tile rows) v, v + 8, ...; the 52 groups do not split
// evenly, so waves 4 .. 7 repeat one of their own groups (same bytes to the
// same place) instead of taking a branch.
// B row of tile row r (0 .. 159) of the block whose first column is n0
template <bool GU>
__device__ __forceinline__ int bg_brow(const BigGemm& g, int n0, int r) {
  if constexpr (GU) {
    // rows 0..79: gate rows n0 .., rows 80..159: the matching up rows
    const int rr = r < 80 ? r : r - 80;
    return min(n0 + rr, g.half - 1) + (r < 80 ? 0 : g.half);
  } else {
    return min(n0 + r, g.N - 1);
  }
}

template <bool GU>
__device__ __forceinline__ void bg_issue(const BigGemm& g, unsigned char* base, int st, int m0, int n0,
                                         int v, int lane) {
  const int k0 = st * BG_BK;
  const int kB = k0 < g.kb ? k0 : k0 - g.kb;  // B column of the stage (K <= 2 kb, kb % 64 == 0)
  const int rin = lane >> 3, pc = lane & 7;  // row within the group, physical chunk
#pragma unroll
  for (int i = 0; i < BG_LOADS; ++i) {
    int q = v + BG_WAVES * i;
    if (i == BG_LOADS - 1) q = q < BG_GROUPS ? q : v;
    const bool isA = q < BG_A_GROUPS;
    const int r = 8 * (isA ? q : q - BG_A_GROUPS) + rin;  // tile row
    const int c = pc ^ bg_swz(r);
    const int brow = bg_brow<GU>(g, n0, r);
    const bf16* src = isA ? g.A + (size_t)min(m0 + r, g.M - 1) * g.lda + k0 : g.B + (size_t)brow * g.ldb + kB;
    __builtin_amdgcn_global_load_lds((const void*)(src + 8 * c), (lds_ptr_t)(base + q * 1024), 16, 0, 0);
  }
}

// The same loads for the [hi | lo8] kernels, from 32-bit byte offsets (the host keeps
// every operand below 4 GB).  Per load only its row's offset unit is kept: A row m at
// m (2 lda) bytes, B row n at n kb (fp8) or 2 n kb (bf16) bytes; a stage adds a
// uniform column offset.  The lane's 16-byte chunk (pc ^ (row & 7)) is the same for
// all of its loads (every group starts at a multiple of 8 rows).
struct BgLo8Rows {
  uint32_t unit[BG_LOADS];
  uint32_t c16;
};
template <bool GU>
__device__ __forceinline__ BgLo8Rows bg_lo8_rows(const BigGemm& g, int m0, int n0, int v, int lane) {
  BgLo8Rows R;
  const int rin = lane >> 3, pc = lane & 7;
  R.c16 = 16u * (uint32_t)(pc ^ rin);
#pragma unroll
  for (int i = 0; i < BG_LOADS; ++i) {
    int q = v + BG_WAVES * i;
    if (i == BG_LOADS - 1) q = q < BG_GROUPS ? q : v;
    const bool isA = q < BG_A_GROUPS;
    const int r = 8 * (isA ? q : q - BG_A_GROUPS) + rin;
    R.unit[i] = isA ? (uint32_t)min(m0 + r, g.M - 1) * (uint32_t)(2 * g.lda) : (uint32_t)bg_brow<GU>(g, n0, r) * (uint32_t)g.kb;
  }
  return R;
}
// Stage st of a [hi | lo8] product: round t = st / 3 covers columns 128 t .. 128 t + 127
// as two bf16 stages (st % 3 = 0, 1: the hi parts times B) and one fp8 stage
// (st % 3 = 2: the lo8 bytes times B8), so the kinds follow the three ring slots.
__device__ __forceinline__ void bg_issue_lo8(const BigGemm& g, const BgLo8Rows& R, unsigned char* base, int st,
                                             int v) {
  const int t = st / 3, k = st - 3 * t;
  const bool f8 = k == 2;
  const uint32_t aoff = f8 ? (uint32_t)(2 * g.kb + 128 * t) : (uint32_t)(256 * t + 128 * k);
  const uint32_t boff = f8 ? (uint32_t)(128 * t) : (uint32_t)(256 * t + 128 * k);
  const unsigned char* bbase = f8 ? g.B8 : reinterpret_cast<const unsigned char*>(g.B);
#pragma unroll
  for (int i = 0; i < BG_LOADS; ++i) {
    int q = v + BG_WAVES * i;
    if (i == BG_LOADS - 1) q = q < BG_GROUPS ? q : v;
    const bool isA = q < BG_A_GROUPS;
    const unsigned char* src = isA ? reinterpret_cast<const unsigned char*>(g.A) + (R.unit[i] + aoff + R.c16)
                                   : bbase + ((R.unit[i] << (f8 ? 0 : 1)) + boff + R.c16);
    __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr_t)(base + q * 1024), 16, 0, 0);
  }
}

// s_waitcnt vmcnt(N), other counters left alone (gfx9 encoding)
template <int N>
__device__ __forceinline__ void bg_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// The MFMAs of one stage for wave (wm, wn).  16x16x32 operand layout: lane l
// supplies row l % 16 and k = 8 (l / 16) .. +7 of the 32-wide k step; the B
// tile is stored [n][k], so both operands are read the same way.
template <bool RSQ>
__device__ __forceinline__ void bg_compute(const unsigned char* sa, BgAccT (&acc)[BG_FRAGS], BgAccT (&sq)[2],
                                           int wm, int wn, int lane) {
  const unsigned char* sb = sa + BG_A_BYTES;
  const int lr = lane & 15, lq = lane >> 4;
#pragma unroll
  for (int kk = 0; kk < BG_BK / 32; ++kk) {
    const int c = 4 * kk + lq;  // logical 16-byte chunk
    u32x4 af[4], bfr[5];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + i * 16 + lr;
      af[i] = *reinterpret_cast<const u32x4*>(sa + r * BG_ROW + 16 * (c ^ bg_swz(r)));
    }
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int r = wn * 80 + j * 16 + lr;
      bfr[j] = *reinterpret_cast<const u32x4*>(sb + r * BG_ROW + 16 * (c ^ bg_swz(r)));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 5; ++j)
        acc[i * 5 + j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, af[i]),
                                                                 __builtin_bit_cast(bf16x8_v, bfr[j]),
                                                                 acc[i * 5 + j], 0, 0, 0);
    if constexpr (RSQ) {
      // A A^T of two of the wave's four 16-row tiles (wn picks which): its diagonal
      // holds the rows' sums of squares over this k step
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const u32x4 a = wn ? af[2 + ii] : af[ii];
        sq[ii] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                         __builtin_bit_cast(bf16x8_v, a), sq[ii], 0, 0, 0);
      }
    }
  }
}

// The MFMAs of one fp8 stage (128 columns) for wave (wm, wn): 16x16x128 block-scaled
// e4m3 MFMA, lane l supplying row l % 16 and columns 32 (l / 16) .. +31 (16-byte
// chunks 2 (l / 16) and 2 (l / 16) + 1 of the tile row) of both operands; byte j % 4
// of bs[j / 4] is the E8M0 scale of the B row this lane supplies to fragment j.
typedef int bg_i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ void bg_compute_f8(const unsigned char* sa, BgAccT (&acc)[BG_FRAGS], const int (&bs)[2],
                                              int wm, int wn, int lane) {
  const unsigned char* sb = sa + BG_A_BYTES;
  const int lr = lane & 15, lq = lane >> 4;
  auto frag8 = [&](const unsigned char* t, int r) {
    const u32x4 x0 = *reinterpret_cast<const u32x4*>(t + r * BG_ROW + 16 * ((2 * lq) ^ bg_swz(r)));
    const u32x4 x1 = *reinterpret_cast<const u32x4*>(t + r * BG_ROW + 16 * ((2 * lq + 1) ^ bg_swz(r)));
    return bg_i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3], (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
  };
  // the five B fragments stay in registers; the A fragments are read one at a time
  // (all nine at once would not fit two waves' registers beside the accumulators)
  bg_i32x8 bfr[5];
#pragma unroll
  for (int j = 0; j < 5; ++j) bfr[j] = frag8(sb, wn * 80 + j * 16 + lr);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bg_i32x8 af = frag8(sa, wm * 64 + i * 16 + lr);
    acc[i * 5 + 0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr[0], acc[i * 5 + 0], 0, 0, 0,
                                                                      BG_LO8_ASCALE, 0, bs[0]);
    acc[i * 5 + 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr[1], acc[i * 5 + 1], 0, 0, 0,
                                                                      BG_LO8_ASCALE, 1, bs[0]);
    acc[i * 5 + 2] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr[2], acc[i * 5 + 2], 0, 0, 0,
                                                                      BG_LO8_ASCALE, 2, bs[0]);
    acc[i * 5 + 3] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr[3], acc[i * 5 + 3], 0, 0, 0,
                                                                      BG_LO8_ASCALE, 3, bs[0]);
    acc[i * 5 + 4] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bfr[4], acc[i * 5 + 4], 0, 0, 0,
                                                                      BG_LO8_ASCALE, 0, bs[1]);
  }
}

#define BG_ISSUE(slot, st)                        \
  do {                                            \
    if constexpr (LO8)                            \
      bg_issue_lo8(g, lrows, slot, st, wave);     \
    else                                          \
      bg_issue<GU>(g, slot, st, m0, n0, wave, lane); \
  } while (0)

// One K stage held in ring slot `cur`; `nxt` (the slot of stage s - 1, free
// once every wave has passed the barrier) receives stage s + 2.  The loads are
// unconditional (past the end they re-read the last stage into the free slot),
// so the whole step is one scheduling region and the wait counts never change;
// the group barriers spread the wave's loads through its MFMAs.
#define BG_STEP_BF16(cur, nxt)                                                           \
  do {                                                                                   \
    bg_wait_vm<BG_LOADS>();                                                              \
    __builtin_amdgcn_s_barrier();                                                        \
    BG_ISSUE(nxt, kbeg + min(s + BG_SLOTS - 1, ns - 1));                                 \
    bg_compute<RSQ>(cur, acc, sq, wm, wn, lane);                                         \
    _Pragma("unroll") for (int r_ = 0; r_ < BG_LOADS - 1; ++r_) {                        \
      __builtin_amdgcn_sched_group_barrier(0x008, 6, 0);                                 \
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                                 \
    }                                                                                    \
    __builtin_amdgcn_sched_group_barrier(0x008, MF - 6 * (BG_LOADS - 1), 0);            \
    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                                   \
    ++s;                                                                                 \
  } while (0)
// an fp8 stage: 20 MFMAs of twice the length, a load after every third
#define BG_STEP_F8(cur, nxt)                                                             \
  do {                                                                                   \
    bg_wait_vm<BG_LOADS>();                                                              \
    __builtin_amdgcn_s_barrier();                                                        \
    BG_ISSUE(nxt, kbeg + min(s + BG_SLOTS - 1, ns - 1));                                 \
    bg_compute_f8(cur, acc, bs, wm, wn, lane);                                           \
    _Pragma("unroll") for (int r_ = 0; r_ < BG_LOADS - 1; ++r_) {                        \
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);                                 \
      __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                                 \
    }                                                                                    \
    __builtin_amdgcn_sched_group_barrier(0x008, 20 - 3 * (BG_LOADS - 1), 0);            \
    __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);                                   \
    ++s;                                                                                 \
  } while (0)
// Steps s .. e - 1 of one kind, the ring slot of step s being slot (s mod 3) and the
// current phase P = s mod 3 known: whole rounds of three, then up to two steps.
#define BG_RUN(STEP, e, a, b, c) \
  do {                           \
    while (s + 3 <= (e)) {       \
      STEP(a, c);                \
      STEP(b, a);                \
      STEP(c, b);                \
    }                            \
    if (s < (e)) STEP(a, c);     \
    if (s < (e)) STEP(b, a);     \
  } while (0)

// internal linkage: every translation unit that launches it holds its own copy.
// EPI: BG_EPI_PLAIN writes rs[m] * (A B^T); BG_EPI_RSQ takes the row scale from A
// itself (rs_k, rs_eps) instead of g.rs; BG_EPI_SWIGLU writes silu(gate) * up.
template <int EPI, bool LO8 = false>
static __global__ __launch_bounds__(BG_THREADS) void gemm_big_kernel(BigGemm g) {
  constexpr bool RSQ = EPI == BG_EPI_RSQ, GU = EPI == BG_EPI_SWIGLU;
  static_assert(!(RSQ && LO8), "the row-statistics form takes plain bf16 rows");
  constexpr int MF = BG_MFMAS + (RSQ ? 4 : 0);  // MFMAs per wave and stage
  // one array per ring slot: separate objects let the compiler tell the
  // direct-to-LDS writes of later stages from the reads of the current one
  __shared__ __align__(1024) unsigned char s0[BG_STAGE_BYTES];
  __shared__ __align__(1024) unsigned char s1[BG_STAGE_BYTES];
  __shared__ __align__(1024) unsigned char s2[BG_STAGE_BYTES];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave & 3, wn = wave >> 2;

  const int KS = g.KS;
  const int T = g.mtiles * g.ntiles * KS;
  const int b = blockIdx.x;
  const int tb = (T % 8 == 0) ? (b % 8) * (T / 8) + b / 8 : b;
  const int kh = tb % KS, u = tb / KS;
  constexpr int GM = 4;  // M-tiles per group: a run of consecutive u covers GM x (run / GM) tiles
  const int grp = u / (GM * g.ntiles), first_m = grp * GM;
  const int gsz = min(g.mtiles - first_m, GM);
  const int tin = u - grp * GM * g.ntiles;
  const int mt = first_m + tin % gsz, nt = tin / gsz;
  const int m0 = mt * BG_BM, n0 = nt * (GU ? BG_BN / 2 : BG_BN);
  const int ns = g.kstages, kbeg = kh * ns;  // the host guarantees ns >= BG_SLOTS

  // E8M0 scales of the B rows this lane supplies to its fp8 fragments
  int bs[2] = {0, 0};
  if constexpr (LO8) {
#pragma unroll
    for (int j = 0; j < 5; ++j)
      bs[j / 4] |= (int)g.b8s[bg_brow<GU>(g, n0, wn * 80 + j * 16 + (lane & 15))] << (8 * (j % 4));
  }
  BgLo8Rows lrows{};
  if constexpr (LO8) lrows = bg_lo8_rows<GU>(g, m0, n0, wave, lane);
  BG_ISSUE(s0, kbeg);
  BG_ISSUE(s1, kbeg + 1);

  BgAccT acc[BG_FRAGS];
#pragma unroll
  for (int f = 0; f < BG_FRAGS; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  BgAccT sq[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};

  int s = 0;
  if constexpr (LO8) {
    // whole rounds (the host makes ns a multiple of 3): slots s0, s1 hold the bf16
    // stages of a round, s2 its fp8 stage
    while (s + 3 <= ns) {
      BG_STEP_BF16(s0, s2);
      BG_STEP_BF16(s1, s0);
      BG_STEP_F8(s2, s1);
    }
  } else {
    BG_RUN(BG_STEP_BF16, ns, s0, s1, s2);
  }
  // the surplus loads of the last steps must land before the block's LDS is released
  bg_wait_vm<0>();

  // accumulator register e of tile (i, j): row 64 wm + 16 i + 4 (lane / 16) + e,
  // column 80 wn + 16 j + lane % 16
  const int lr = lane & 15, lq = lane >> 4;
  __shared__ float s_sq[RSQ ? BG_BM : 1];
  if constexpr (RSQ) {
    // the Gram diagonal: register e of lane (lq, lr) is entry (4 lq + e, lr)
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (4 * lq + e == lr) s_sq[wm * 64 + 16 * (2 * wn + ii) + lr] = sq[ii][e];
    __syncthreads();
    if (KS > 1 && threadIdx.x < BG_BM)
      st_coh(g.sqp + ((size_t)u * KS + kh) * BG_BM + threadIdx.x, s_sq[threadIdx.x]);
  }
  if (KS > 1) {
    // partial tile as [wave][f][lane][e]: every store is 1 KB contiguous
    float* mine = g.part + ((size_t)u * KS + kh) * BG_PART_FLOATS + (size_t)wave * (BG_FRAGS * 256);
#pragma unroll
    for (int f = 0; f < BG_FRAGS; ++f)
      st_coh4b(mine, (uint32_t)((f * 256 + lane * 4) * 4), make_float4(acc[f][0], acc[f][1], acc[f][2], acc[f][3]));
    if (!arrive_last(g.counters + u, (unsigned)KS)) return;
    // the sum runs over the parts in the order 0 .. KS-1 whichever block is
    // last; with two parts a + b == b + a, so the own part stays in registers
    const float* base = g.part + (size_t)u * KS * BG_PART_FLOATS + (size_t)wave * (BG_FRAGS * 256);
    if (KS > 2) {
#pragma unroll
      for (int f = 0; f < BG_FRAGS; ++f) acc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int p = 0; p < KS; ++p) {
      if (KS == 2 && p == kh) continue;
      const float* src = base + (size_t)p * BG_PART_FLOATS;
      float4 v[BG_FRAGS];
#pragma unroll
      for (int f = 0; f < BG_FRAGS; ++f) v[f] = ld_coh4(src, (uint32_t)((f * 256 + lane * 4) * 4));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int f = 0; f < BG_FRAGS; ++f) {
        acc[f][0] += v[f].x;
        acc[f][1] += v[f].y;
        acc[f][2] += v[f].z;
        acc[f][3] += v[f].w;
      }
    }
  }
  if constexpr (RSQ) {
    // the parts' sums in the order 0 .. KS-1 whichever block finishes
    if (threadIdx.x < BG_BM) {
      float t = 0.f;
      for (int p = 0; p < KS; ++p)
        t += p == kh ? s_sq[threadIdx.x] : ld_coh(g.sqp + ((size_t)u * KS + p) * BG_BM + threadIdx.x);
      s_sq[threadIdx.x] = 1.0f / sqrtf(t / (float)g.rs_k + g.rs_eps);
    }
    __syncthreads();
  }
  // the 16 row scales of this lane, loaded together before any store
  float rsv[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = m0 + wm * 64 + 16 * i + 4 * lq + e;
      if constexpr (RSQ)
        rsv[i][e] = s_sq[wm * 64 + 16 * i + 4 * lq + e];
      else
        rsv[i][e] = g.rs ? g.rs[min(row, g.M - 1)] : 1.f;
    }
  if constexpr (GU) {
    // the up half (wn = 1) hands its scaled values to the gate half through the
    // stage buffers (every wave is past its last read of them), which writes
    // silu(gate) * up for its 80 columns
    __syncthreads();
    float* xch = reinterpret_cast<float*>(wm < 2 ? s0 : s1) + (size_t)(wm & 1) * (BG_FRAGS * 4 * 64);
    if (wn == 1) {
#pragma unroll
      for (int f = 0; f < BG_FRAGS; ++f)
#pragma unroll
        for (int e = 0; e < 4; ++e) xch[(f * 4 + e) * 64 + lane] = acc[f][e] * rsv[f / 5][e];
    }
    __syncthreads();
    if (wn == 0) {
      // columns 16 j + lr and + 1 sit in neighbouring lanes: the even lane of each
      // pair writes both (4-byte stores); half is even, so a pair never straddles it
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = m0 + wm * 64 + 16 * i + 4 * lq + e;
#pragma unroll
          for (int j = 0; j < 5; ++j) {
            const int col = n0 + 16 * j + lr;
            const float gt = acc[i * 5 + j][e] * rsv[i][e];
            const float up = xch[((i * 5 + j) * 4 + e) * 64 + lane];
            const float a = gt / (1.0f + expf(-gt)) * up;
            const bf16 hi = f2bf(a);
            if constexpr (LO8) {
              // [hi | lo8] rows: hi pairs at act + row act_ld + col, lo8 pairs at byte 2 half + col
              const uint32_t hl = (uint32_t)hi | (lo8_byte(a - bf2f(hi)) << 16);
              const uint32_t nb = (uint32_t)__shfl_xor((int)hl, 1, 64);
              if ((lr & 1) == 0 && row < g.M && col < g.half) {
                bf16* out = g.act + (size_t)row * g.act_ld;
                *reinterpret_cast<uint32_t*>(out + col) = (hl & 0xffffu) | (nb << 16);
                *reinterpret_cast<uint16_t*>(reinterpret_cast<unsigned char*>(out + g.half) + col) =
                    (uint16_t)((hl >> 16) | ((nb >> 8) & 0xff00u));
              }
            } else {
              const bf16 lo = f2bf(a - bf2f(hi));
              const uint32_t hl = (uint32_t)hi | ((uint32_t)lo << 16);
              const uint32_t nb = (uint32_t)__shfl_xor((int)hl, 1, 64);
              if ((lr & 1) == 0 && row < g.M && col < g.half) {
                bf16* out = g.act + (size_t)row * g.act_ld + col;
                *reinterpret_cast<uint32_t*>(out) = (hl & 0xffffu) | (nb << 16);
                *reinterpret_cast<uint32_t*>(out + g.half) = (hl >> 16) | (nb & 0xffff0000u);
              }
            }
          }
        }
    }
    return;
  }
  const bool full = m0 + BG_BM <= g.M && n0 + BG_BN <= g.N;
  if (full) {
    // no bounds checks: one straight run of stores
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float* crow = g.C + (size_t)(m0 + wm * 64 + 16 * i + 4 * lq + e) * g.ldc + n0 + wn * 80 + lr;
#pragma unroll
        for (int j = 0; j < 5; ++j) crow[16 * j] = acc[i * 5 + j][e] * rsv[i][e];
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + wm * 64 + 16 * i + 4 * lq + e;
        if (row < g.M) {
#pragma unroll
          for (int j = 0; j < 5; ++j) {
            const int col = n0 + wn * 80 + 16 * j + lr;
            if (col < g.N) g.C[(size_t)row * g.ldc + col] = acc[i * 5 + j][e] * rsv[i][e];
          }
        }
      }
  }
}

#undef BG_RUN
#undef BG_ISSUE
#undef BG_STEP_BF16
#undef BG_STEP_F8

// ---------------------------------------------------------------------------
// Host-side planning: KS splits K so that the tiles times KS fill the GPU
// (each part keeps at least BG_SLOTS stages of 64).
// ---------------------------------------------------------------------------
constexpr int BG_TARGET_BLOCKS = 256;

struct BigPlan {
  bool use;
  int mtiles, ntiles, KS, kstages;
  size_t part_bytes;  // partial tiles when KS > 1
  size_t sq_bytes;    // partial row sums of squares of the row-statistics form when KS > 1
};

inline BigPlan plan_big_gemm(int M, int N, int K) {
  BigPlan b{};
  if (M < 1 || N < 1 || K % BG_BK) return b;
  b.mtiles = (M + BG_BM - 1) / BG_BM;
  b.ntiles = (N + BG_BN - 1) / BG_BN;
  const int stages = K / BG_BK;
  if (stages < BG_SLOTS) return b;
  b.KS = 1;
  while (b.KS < BG_MAX_KS && b.mtiles * b.ntiles * b.KS * 2 <= BG_TARGET_BLOCKS && stages % (b.KS * 2) == 0 &&
         stages / (b.KS * 2) >= BG_SLOTS)
    b.KS *= 2;
  b.kstages = stages / b.KS;
  b.part_bytes = b.KS > 1 ? (size_t)b.mtiles * b.ntiles * b.KS * BG_PART_FLOATS * 4 : 0;
  b.sq_bytes = b.KS > 1 ? (size_t)b.mtiles * b.ntiles * b.KS * BG_BM * 4 : 0;
  b.use = true;
  return b;
}

// The [hi | lo8] form of a product over kb columns: kb / 64 bf16 stages and kb / 128
// fp8 stages (kb % 128 == 0), planned as one run of equal stages.
// (the kernel addresses its operands with 32-bit byte offsets: A's M rows of 3 kb bytes
// and B's N rows of 2 kb bytes stay below 4 GB)
inline bool lo8_fits(int M, int N, int kb) {
  return kb % 128 == 0 && (uint64_t)M * 3 * kb < (1ull << 32) && (uint64_t)N * 2 * kb < (1ull << 32);
}
// K parts of whole rounds (three stages: 128 columns of hi and of lo8)
inline BigPlan plan_lo8_rounds(int M, int N, int kb) {
  BigPlan b{};
  if (!lo8_fits(M, N, kb) || M < 1 || N < 1) return b;
  b.mtiles = (M + BG_BM - 1) / BG_BM;
  b.ntiles = (N + BG_BN - 1) / BG_BN;
  const int rounds = kb / 128;
  b.KS = 1;
  while (b.KS < BG_MAX_KS && b.mtiles * b.ntiles * b.KS * 2 <= BG_TARGET_BLOCKS && rounds % (b.KS * 2) == 0)
    b.KS *= 2;
  b.kstages = 3 * (rounds / b.KS);
  b.part_bytes = b.KS > 1 ? (size_t)b.mtiles * b.ntiles * b.KS * BG_PART_FLOATS * 4 : 0;
  b.use = true;
  return b;
}
inline BigPlan plan_big_lo8(int M, int N, int kb) { return plan_lo8_rounds(M, N, kb); }
inline BigPlan plan_big_swiglu_lo8(int M, int half, int kb) {
  return plan_lo8_rounds(M, BG_BN * ((half + BG_BN / 2 - 1) / (BG_BN / 2)), kb);
}

// C[M][ldc] = rs[m] * (A[M][lda] . B[N][kb]^T) over K columns of A; K = kb, or
// K = 2 kb with A's rows holding [hi | lo] bf16 parts of an fp32 activation (the
// product then carries the activation to about fp32 accuracy).  counters: at
// least mtiles * ntiles zero words, left zero.  With rs_k > 0 (K = kb) the row
// scale is taken from A itself: rs[m] = 1 / sqrt(sum_k A[m][k]^2 / rs_k + rs_eps),
// the sums formed on the MFMA from the staged A tiles (sqp: p.sq_bytes).
inline void launch_big_gemm(const BigPlan& p, const bf16* A, int lda, const bf16* B, float* C, int ldc,
                            const float* rs, int M, int N, int K, float* part, unsigned* counters,
                            hipStream_t st, int kb = 0, float* sqp = nullptr, int rs_k = 0, float rs_eps = 0.f) {
  BigGemm g{};
  g.A = A;
  g.B = B;
  g.C = C;
  g.rs = rs;
  g.part = part;
  g.counters = counters;
  g.M = M;
  g.N = N;
  g.K = K;
  g.lda = lda;
  g.kb = kb > 0 ? kb : K;
  g.ldb = g.kb;
  g.ldc = ldc;
  g.mtiles = p.mtiles;
  g.ntiles = p.ntiles;
  g.KS = p.KS;
  g.kstages = p.kstages;
  g.sqp = sqp;
  g.rs_k = rs_k;
  g.rs_eps = rs_eps;
  if (rs_k > 0)
    hipLaunchKernelGGL(gemm_big_kernel<BG_EPI_RSQ>, dim3(p.mtiles * p.ntiles * p.KS), dim3(BG_THREADS), 0, st, g);
  else
    hipLaunchKernelGGL(gemm_big_kernel<BG_EPI_PLAIN>, dim3(p.mtiles * p.ntiles * p.KS), dim3(BG_THREADS), 0, st,
                       g);
}

// The same product with A's rows in the [hi | lo8] form (lda in bf16 elements, at
// least 3 kb / 2): the hi parts times B plus the lo8 parts times B8 (e4m3 rows of B
// scaled by 2^e_n, b8s[n] = 127 - e_n).  Plan: plan_big_lo8.
inline void launch_big_gemm_lo8(const BigPlan& p, const bf16* A, int lda, const bf16* B,
                                const unsigned char* B8, const unsigned char* b8s, float* C, int ldc,
                                const float* rs, int M, int N, int kb, float* part, unsigned* counters,
                                hipStream_t st) {
  BigGemm g{};
  g.A = A;
  g.B = B;
  g.B8 = B8;
  g.b8s = b8s;
  g.C = C;
  g.rs = rs;
  g.part = part;
  g.counters = counters;
  g.M = M;
  g.N = N;
  g.K = kb + kb / 2;
  g.lda = lda;
  g.kb = kb;
  g.ldb = kb;
  g.ldc = ldc;
  g.mtiles = p.mtiles;
  g.ntiles = p.ntiles;
  g.KS = p.KS;
  g.kstages = p.kstages;
  hipLaunchKernelGGL((gemm_big_kernel<BG_EPI_PLAIN, true>), dim3(p.mtiles * p.ntiles * p.KS), dim3(BG_THREADS), 0,
                     st, g);
}

// Gate/up product with the SwiGLU epilogue: W = [gate; up] ([2 half][kb] bf16), A as in
// launch_big_gemm; act[m][j] = silu(g_j) * u_j with g, u = rs[m] * (A W^T), written as
// bf16 hi at act + m act_ld + j and lo at + half.  Plan: plan_big_swiglu.
inline BigPlan plan_big_swiglu(int M, int half, int K) {
  return plan_big_gemm(M, BG_BN * ((half + BG_BN / 2 - 1) / (BG_BN / 2)), K);
}
inline void launch_big_swiglu(const BigPlan& p, const bf16* A, int lda, const bf16* W, bf16* act, int act_ld,
                              int half, const float* rs, int M, int K, float* part, unsigned* counters,
                              hipStream_t st, int kb) {
  BigGemm g{};
  g.A = A;
  g.B = W;
  g.rs = rs;
  g.part = part;
  g.counters = counters;
  g.M = M;
  g.N = 2 * half;
  g.K = K;
  g.lda = lda;
  g.kb = kb > 0 ? kb : K;
  g.ldb = g.kb;
  g.mtiles = p.mtiles;
  g.ntiles = p.ntiles;
  g.KS = p.KS;
  g.kstages = p.kstages;
  g.act = act;
  g.act_ld = act_ld;
  g.half = half;
  hipLaunchKernelGGL(gemm_big_kernel<BG_EPI_SWIGLU>, dim3(p.mtiles * p.ntiles * p.KS), dim3(BG_THREADS), 0, st,
                     g);
}

// The gate/up product with A in the [hi | lo8] form (as launch_big_gemm_lo8, B8 and
// b8s over the 2 half rows of W) writing act as [hi | lo8] rows: hi at act + m act_ld + j,
// lo8 at byte 2 half + j of the row (act_ld >= 3 half / 2, half % 4 == 0).
// Plan: plan_big_swiglu_lo8.
inline void launch_big_swiglu_lo8(const BigPlan& p, const bf16* A, int lda, const bf16* W,
                                  const unsigned char* W8, const unsigned char* w8s, bf16* act, int act_ld,
                                  int half, const float* rs, int M, int kb, float* part, unsigned* counters,
                                  hipStream_t st) {
  BigGemm g{};
  g.A = A;
  g.B = W;
  g.B8 = W8;
  g.b8s = w8s;
  g.rs = rs;
  g.part = part;
  g.counters = counters;
  g.M = M;
  g.N = 2 * half;
  g.K = kb + kb / 2;
  g.lda = lda;
  g.kb = kb;
  g.ldb = kb;
  g.mtiles = p.mtiles;
  g.ntiles = p.ntiles;
  g.KS = p.KS;
  g.kstages = p.kstages;
  g.act = act;
  g.act_ld = act_ld;
  g.half = half;
  hipLaunchKernelGGL((gemm_big_kernel<BG_EPI_SWIGLU, true>), dim3(p.mtiles * p.ntiles * p.KS), dim3(BG_THREADS),
                     0, st, g);
}

}  // namespace spd
