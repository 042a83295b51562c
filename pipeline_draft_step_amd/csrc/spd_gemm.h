// Skinny GEMM for decode-shaped products: Y[M][N] = X[M][K] . W[N][K]^T with
// M up to 32 per tile and W streamed from HBM once.
//
// Work split: a workgroup (4 waves) owns an N-block of 64*NT weight rows and one
// of S equal K-slices; each wave owns 16*NT rows.  The X slice (rows of the
// M-tile) is staged in LDS by an input functor `In` that may fuse a gather or a
// normalisation.  bf16 W is read in groups of 8 k-steps as 4-row x 256-byte
// load instructions (the pattern HBM streams fastest) and reordered into MFMA B
// fragments through a small wave-private LDS buffer; fp32 W goes straight from
// global memory to the MFMA operand.  Either way the next group's loads are in
// flight while the current one is multiplied.  With S == 1 the block runs the epilogue functor `Epi` on its own
// tile.  With S > 1 every block writes an fp32 partial tile with coherent (sc1)
// stores and counts itself in; the last of the S blocks of an (N-block, M-tile)
// sums the partials in fixed split order and runs the epilogue (no fences, see
// spd_common.h).  Results are deterministic for a given launch shape.
#pragma once

#include <algorithm>
#include <type_traits>

#include "spd_common.h"

namespace spd {

#ifndef SPD_GEMM_UNROLL
#define SPD_GEMM_UNROLL 8  // fp32 weights: k-steps of loads in flight per wave (double-buffered)
#endif

constexpr int GEMM_THREADS = 256;
constexpr int GEMM_WAVES = 4;
constexpr int GEMM_UNROLL = SPD_GEMM_UNROLL;
// bf16 weight groups: 8 k-steps (512 bytes of each row) per group, fetched as 8
// load instructions that each cover 4 rows x 256 contiguous bytes.  Four of them
// at a time pass through a wave-private LDS buffer (1 KB + 64 B pad each, which
// makes the fragment reads bank-conflict free) to reach the MFMA B layout.
constexpr int WG_STEPS = 8;
constexpr int TB_STRIDE = 1024 + 64;
constexpr int TB_WAVE = 4 * TB_STRIDE;
// transpose buffers per wave: one per column group for 16-row tiles, one for 32-row tiles
constexpr int gemm_tb_buffers(int MT, int NT) { return MT == 1 ? NT : 1; }

struct GemmShape {
  const void* W;
  int N, K, M;
  int S;        // split-K factor
  int nsteps;   // K / KSTEP
  int ldx;      // LDS row pitch of the staged X slice (elements)
  float* part;  // [S][M][N] partials (S > 1)
  int nblocks;
  unsigned* counters;  // [mtiles][nblocks] arrival counters (S > 1), zero between uses
  int x_bytes;         // dynamic LDS: staged X slice (hi + lo), aliased by the
  int ytile_bytes;     // fp32 result tile; the transpose buffers follow both
  // optional per-row scale of the product: 1 / sqrt(sum_p rs_ss[p][row] / rs_K + rs_eps)
  // (the RMSNorm of an input whose gamma the producer has already applied); in the
  // per-row form (RS_SSR) the partials are already divided by the row's own width
  // and a negative sum marks a row that is not normalised (scale 1)
  const float* rs_ss;  // [rs_P][rs_M] partial sums of squares
  int rs_P, rs_M, rs_K;
  float rs_eps;
  const float* rs_inv;  // or the row scales themselves [M]
  // (which one applies is fixed by the input functor, see RowScaleOf)
};

// Row of W that local column c (0 .. 64*NT-1) of N-block nb maps to.
struct RowMapStd {
  template <int NT>
  __device__ __forceinline__ int row(int nb, int c) const { return nb * 64 * NT + c; }
};
// gate/up pairing: columns [0, 32*NT) are gate rows, [32*NT, 64*NT) the matching
// up rows (W = [gate; up], `half` = dff).
struct RowMapGateUp {
  int half;
  template <int NT>
  __device__ __forceinline__ int row(int nb, int c) const {
    const int h = 32 * NT;
    return c < h ? nb * h + c : half + nb * h + (c - h);
  }
};

// Staged X slice.  For bf16 weights every activation is kept as a pair of
// bfloat16 values hi + lo (lo = x - hi, rounded), giving the MFMA about 16
// mantissa bits of the fp32 activation at the cost of a second MFMA per weight
// fragment; the products are HBM-bound, so the matrix cores have room for it.
template <typename WT>
struct XStage {
  WT* hi;
  WT* lo;
  int ldx;
  __device__ __forceinline__ void put(int m, int k, float v) const {
    const WT h = from_f<WT>(v);
    hi[m * ldx + k] = h;
    if constexpr (sizeof(WT) == 2) lo[m * ldx + k] = from_f<WT>(v - to_f<WT>(h));
  }
  // four consecutive k (k % 4 == 0)
  __device__ __forceinline__ void put4(int m, int k, const float (&v)[4]) const {
    if constexpr (sizeof(WT) == 2) {
      const uint32_t h0 = pack2_bf16(v[0], v[1]), h1 = pack2_bf16(v[2], v[3]);
      const uint32_t l0 = pack2_bf16(v[0] - __uint_as_float(h0 << 16), v[1] - __uint_as_float(h0 & 0xffff0000u));
      const uint32_t l1 = pack2_bf16(v[2] - __uint_as_float(h1 << 16), v[3] - __uint_as_float(h1 & 0xffff0000u));
      *reinterpret_cast<uint2*>(hi + m * ldx + k) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(lo + m * ldx + k) = make_uint2(l0, l1);
    } else {
      *reinterpret_cast<float4*>(hi + m * ldx + k) = make_float4(v[0], v[1], v[2], v[3]);
    }
  }
};

// four consecutive elements (16-byte aligned for float, 8-byte for bf16)
__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
__device__ __forceinline__ void load4(const bf16* p, float (&v)[4]) {
  const uint2 a = *reinterpret_cast<const uint2*>(p);
  v[0] = bf2f((bf16)(a.x & 0xffff)); v[1] = bf2f((bf16)(a.x >> 16));
  v[2] = bf2f((bf16)(a.y & 0xffff)); v[3] = bf2f((bf16)(a.y >> 16));
}

// Sum of n values f(i), i < n, by one wave: lane-strided, then a butterfly (fixed order).
template <typename F>
__device__ __forceinline__ float wave_sum_of(int n, const F& f) {
  const int lane = threadIdx.x & 63;
  float t = 0.f;
  for (int i = lane; i < n; i += WAVE) t += f(i);
  return wave_sum(t);
}

// Stagers with kTwoPhase issue their loads (load) before the first weight group
// and write LDS (store) afterwards; the others stage in one call.
template <typename T, typename = void>
struct TwoPhase : std::false_type {};
template <typename T>
struct TwoPhase<T, std::void_t<decltype(T::kTwoPhase)>> : std::bool_constant<T::kTwoPhase> {};

// Row scales of the tile (see GemmShape::rs_ss): wave w owns rows w, w + 4, ...
// (RW = 4 * MT of them); the partial sums are loaded first (load) and reduced
// into s_rs (finish).
// Row-scale mode, a compile-time property of the input functor (kRowScale):
// none, from partial sums of squares (rs_ss), from partial mean squares with a
// per-row width (rs_ss, RS_SSR), or given per row (rs_inv).
enum { RS_NONE = 0, RS_SS = 1, RS_INV = 2, RS_SSR = 3 };
template <typename T, typename = void>
struct RowScaleOf : std::integral_constant<int, RS_NONE> {};
template <typename T>
struct RowScaleOf<T, std::void_t<decltype(T::kRowScale)>> : std::integral_constant<int, T::kRowScale> {};

template <int RW, int RS>
struct RowScale {
  float p[RW][2];
  __device__ __forceinline__ void load(const GemmShape& g, int m0, int Mt) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    if constexpr (RS == RS_INV) {
#pragma unroll
      for (int j = 0; j < RW; ++j) p[j][0] = g.rs_inv[m0 + min(wave + GEMM_WAVES * j, Mt - 1)];
    } else if constexpr (RS == RS_SS || RS == RS_SSR) {
#pragma unroll
      for (int j = 0; j < RW; ++j) {
        const int mm = wave + GEMM_WAVES * j;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int c = lane + WAVE * h;
          const bool ok = mm < Mt && c < g.rs_P;
          p[j][h] = g.rs_ss[ok ? (size_t)c * g.rs_M + m0 + mm : (size_t)m0];  // masked in finish
        }
      }
    }
  }
  __device__ __forceinline__ void finish(const GemmShape& g, int Mt, float* s_rs) const {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < RW; ++j) {
      const int mm = wave + GEMM_WAVES * j;
      float v = 1.f;
      if constexpr (RS == RS_INV) {
        v = p[j][0];
      } else if constexpr (RS == RS_SS) {
        const float a = (mm < Mt && lane < g.rs_P) ? p[j][0] : 0.f;
        const float b = (mm < Mt && lane + WAVE < g.rs_P) ? p[j][1] : 0.f;
        v = 1.0f / sqrtf(wave_sum(a + b) / (float)g.rs_K + g.rs_eps);
      } else if constexpr (RS == RS_SSR) {
        const float a = (mm < Mt && lane < g.rs_P) ? p[j][0] : 0.f;
        const float b = (mm < Mt && lane + WAVE < g.rs_P) ? p[j][1] : 0.f;
        const float t = wave_sum(a + b);
        v = t < 0.f ? 1.f : 1.0f / sqrtf(t + g.rs_eps);
      }
      if (lane == 0) s_rs[mm] = v;
    }
  }
};

template <int TC>
struct TileY {
  const float (*y)[TC + 1];
  __device__ __forceinline__ float operator()(int m, int c) const { return y[m][c]; }
};

template <typename WT, int MT, int NT, typename In, typename Epi, typename RowMap>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_skinny_kernel(GemmShape g, In in, Epi epi,
                                                                   RowMap rmap) {
  typedef Mfma<WT> F;
  typedef typename F::frag frag;
  constexpr int TR = 16 * MT;  // rows per M-tile
  constexpr int TC = 64 * NT;  // columns per N-block
  constexpr bool SPLIT = sizeof(WT) == 2;
  constexpr int TBN = gemm_tb_buffers(MT, NT);  // transpose buffers per wave
  constexpr int U = GEMM_UNROLL;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float s_rs[32];  // row scales of the tile

  // the decode chain is latency-bound and shares the chip with a head streaming on
  // another stream: its waves issue first on a shared SIMD
  __builtin_amdgcn_s_setprio(3);
  const int S = g.S;
  const int nb = blockIdx.x / S;
  const int s = blockIdx.x - nb * S;
  const int mt = blockIdx.y;
  const int m0 = mt * TR;
  const int Mt = min(TR, g.M - m0);
  const int st0 = (int)((long long)s * g.nsteps / S);
  const int st1 = (int)((long long)(s + 1) * g.nsteps / S);
  const int k0 = st0 * F::KSTEP;
  const int kw = (st1 - st0) * F::KSTEP;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int nst = st1 - st0;

  WT* xs = reinterpret_cast<WT*>(smem);
  const int xrows = min(TR, g.M);
  WT* xs_lo = xs + (size_t)xrows * g.ldx;
  f32x4 acc[MT][NT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int u = 0; u < NT; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  const WT* xp[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xp[t] = xs + min(16 * t + lr, Mt - 1) * g.ldx + lg * F::KPL;
  const ptrdiff_t lo_off = xs_lo - xs;

  if constexpr (SPLIT) {
    // rows of load instruction i (q = i % 4): local rows 16u + 4q + lane % 4; this
    // lane's 16 bytes sit at element 8 * (lane / 4) of the instruction's 128-element span
    const WT* wq[NT][4];
#pragma unroll
    for (int u = 0; u < NT; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int row = rmap.template row<NT>(nb, wave * 16 * NT + 16 * u + 4 * q + (lane & 3));
        wq[u][q] = reinterpret_cast<const WT*>(g.W) + (size_t)(row < g.N ? row : 0) * g.K;
      }
    const int ksub = lane >> 4;          // k-step of this lane's chunk inside a half group
    const int loff = k0 + 8 * (lane >> 2);  // this lane's element offset in the row
    // Two register buffers with fixed roles (A: even groups, B: odd groups), so
    // that consuming one never waits for the loads of the other.  Loads are
    // unconditional (a conditional load becomes a branch whose join waits for
    // every outstanding load): chunks past the slice read the first element of
    // the row instead; they only feed k-steps that are never multiplied, and rows
    // past N (clamped to row 0) only feed columns that are never stored.
    frag bufA[NT][WG_STEPS], bufB[NT][WG_STEPS];
    auto issue = [&](frag (&d)[NT][WG_STEPS], int st) {
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int i = 0; i < WG_STEPS; ++i) {
          const int h = i >> 2, q = i & 3;
          d[u][i] = F::load(wq[u][q] + (st + 4 * h + ksub < nst ? loff + st * F::KSTEP + 128 * h : 0));
        }
    };
    // A wave's loads complete in issue order: the row-scale and X-slice loads go
    // out before the first weight group, so waiting for them never waits for it.
    RowScale<4 * MT, RowScaleOf<In>::value> rsc;
    rsc.load(g, m0, Mt);
    const XStage<WT> xst{xs, xs_lo, g.ldx};
    if constexpr (TwoPhase<In>::value) {
      constexpr int SB = In::SB, CH = In::CH;
      // round 0; program order is pinned: X loads, first weight group, LDS writes
      // (native vectors: HIP's uint4 struct is copied with memcpy, which keeps the
      // array out of registers)
      {
        u32x4 rh[SB], rl[SB];
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          int m, c;
          bool ok;
          In::chunk(0, i, Mt, kw, m, c, ok);
          const size_t off = (size_t)(m0 + m) * in.K + k0 + c * CH;
          rh[i] = *reinterpret_cast<const u32x4*>(in.hi + off);
          rl[i] = *reinterpret_cast<const u32x4*>(in.lo + off);
        }
        __builtin_amdgcn_sched_barrier(0);
        issue(bufA, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < SB; ++i) {
          int m, c;
          bool ok;
          In::chunk(0, i, Mt, kw, m, c, ok);
          if (ok) {
            *reinterpret_cast<u32x4*>(xst.hi + m * xst.ldx + c * CH) = rh[i];
            *reinterpret_cast<u32x4*>(xst.lo + m * xst.ldx + c * CH) = rl[i];
          }
        }
      }
      // further rounds (slices larger than one round), one chunk at a time
      const int nch = kw / CH, n = Mt * nch;
      for (int e = SB * GEMM_THREADS + threadIdx.x; e < n; e += GEMM_THREADS) {
        const int m = e / nch, c = e - m * nch;
        const size_t off = (size_t)(m0 + m) * in.K + k0 + c * CH;
        *reinterpret_cast<uint4*>(xst.hi + m * xst.ldx + c * CH) = *reinterpret_cast<const uint4*>(in.hi + off);
        *reinterpret_cast<uint4*>(xst.lo + m * xst.ldx + c * CH) = *reinterpret_cast<const uint4*>(in.lo + off);
      }
    } else {
      in.stage(xst, m0, Mt, k0, kw, nb, s, S);
      issue(bufA, 0);
    }
    rsc.finish(g, Mt, s_rs);
    __syncthreads();
    unsigned char* tb = reinterpret_cast<unsigned char*>(xs_lo + (size_t)xrows * g.ldx) +
                        (size_t)(max(g.ytile_bytes - g.x_bytes, 0)) + wave * TBN * TB_WAVE;
    const int rdb = (lr >> 2) * TB_STRIDE + 16 * ((lr & 3) + 4 * lg);
    // multiply one group; FULL: all WG_STEPS k-steps are inside the slice.  With
    // 16-row tiles the NT column groups of a half group pass through TBN = NT
    // transpose buffers, so each X fragment is read from LDS once per k-step for
    // all of them (measured: headline PDM step 178.6 -> 171.0 us); 32-row tiles
    // keep one buffer and read X per column group (their LDS budget goes to the X
    // slice: sharing cost the 9B-shaped step 685 -> 718 us)
    auto consume = [&](const frag (&c)[NT][WG_STEPS], int st, auto full) {
      constexpr bool FULL = decltype(full)::value;
      if constexpr (TBN == 1) {
#pragma unroll
        for (int u = 0; u < NT; ++u)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            if (!FULL && st + 4 * h >= nst) continue;
#pragma unroll
            for (int j = 0; j < 4; ++j)
              *reinterpret_cast<frag*>(tb + j * TB_STRIDE + 16 * lane) = c[u][4 * h + j];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int ks = st + 4 * h + j;
              if (FULL || ks < nst) {
                const frag b = *reinterpret_cast<const frag*>(tb + rdb + 256 * j);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                  const frag af = F::load(xp[t] + ks * F::KSTEP);
                  const frag al = F::load(xp[t] + lo_off + ks * F::KSTEP);
                  acc[t][u] = F::mma(af, b, acc[t][u]);
                  acc[t][u] = F::mma(al, b, acc[t][u]);
                }
              }
            }
          }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (!FULL && st + 4 * h >= nst) continue;
#pragma unroll
          for (int u = 0; u < NT; ++u)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              *reinterpret_cast<frag*>(tb + u * TB_WAVE + j * TB_STRIDE + 16 * lane) = c[u][4 * h + j];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int ks = st + 4 * h + j;
            if (FULL || ks < nst) {
              frag af[MT], al[MT];
#pragma unroll
              for (int t = 0; t < MT; ++t) {
                af[t] = F::load(xp[t] + ks * F::KSTEP);
                al[t] = F::load(xp[t] + lo_off + ks * F::KSTEP);
              }
#pragma unroll
              for (int u = 0; u < NT; ++u) {
                const frag b = *reinterpret_cast<const frag*>(tb + u * TB_WAVE + rdb + 256 * j);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                  acc[t][u] = F::mma(af[t], b, acc[t][u]);
                  acc[t][u] = F::mma(al[t], b, acc[t][u]);
                }
              }
            }
          }
        }
      }
    };
    // Main loop over pairs of full groups with unconditional issues, so that every
    // path into a wait has the same loads outstanding (the wait counts are taken
    // over all paths); the last one or two groups follow outside the loop.
    const int ng = (nst + WG_STEPS - 1) / WG_STEPS;
    int gi = 0;
    for (; gi + 2 < ng; gi += 2) {
      issue(bufB, (gi + 1) * WG_STEPS);
      __builtin_amdgcn_sched_barrier(0);
      consume(bufA, gi * WG_STEPS, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      issue(bufA, (gi + 2) * WG_STEPS);
      __builtin_amdgcn_sched_barrier(0);
      consume(bufB, (gi + 1) * WG_STEPS, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
    }
    if (gi + 1 < ng) {
      issue(bufB, (gi + 1) * WG_STEPS);
      __builtin_amdgcn_sched_barrier(0);
      consume(bufA, gi * WG_STEPS, std::true_type{});
      __builtin_amdgcn_sched_barrier(0);
      consume(bufB, (gi + 1) * WG_STEPS, std::false_type{});
    } else if (gi < ng) {
      consume(bufA, gi * WG_STEPS, std::false_type{});
    }
  } else {
    // fp32 weights: fragments straight from global memory in the MFMA layout
    const WT* wp[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int row = rmap.template row<NT>(nb, wave * 16 * NT + 16 * u + lr);
      wp[u] = reinterpret_cast<const WT*>(g.W) + (size_t)(row < g.N ? row : 0) * g.K + k0 + lg * F::KPL;
    }
    frag cur[U][NT], nxt[U][NT];
#pragma unroll
    for (int i = 0; i < U; ++i)
#pragma unroll
      for (int u = 0; u < NT; ++u) cur[i][u] = F::load(wp[u] + (i < nst ? i * F::KSTEP : 0));
    RowScale<4 * MT, RowScaleOf<In>::value> rsc;
    rsc.load(g, m0, Mt);
    const XStage<WT> xst{xs, xs_lo, g.ldx};
    if constexpr (TwoPhase<In>::value) {
      constexpr int CH = In::CH;
      const int nch = kw / CH, n = Mt * nch;
      for (int e = threadIdx.x; e < n; e += GEMM_THREADS) {
        const int m = e / nch, c = e - m * nch;
        *reinterpret_cast<uint4*>(xst.hi + m * xst.ldx + c * CH) =
            *reinterpret_cast<const uint4*>(in.hi + (size_t)(m0 + m) * in.K + k0 + c * CH);
      }
    } else {
      in.stage(xst, m0, Mt, k0, kw, nb, s, S);
    }
    rsc.finish(g, Mt, s_rs);
    __syncthreads();
    for (int st = 0; st < nst; st += U) {
      const int nxt0 = st + U;
      if (nxt0 < nst) {
#pragma unroll
        for (int i = 0; i < U; ++i)
#pragma unroll
          for (int u = 0; u < NT; ++u)
            nxt[i][u] = F::load(wp[u] + (nxt0 + i < nst ? (nxt0 + i) * F::KSTEP : 0));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < U; ++i) {
        if (st + i < nst) {
#pragma unroll
          for (int t = 0; t < MT; ++t) {
            const frag af = F::load(xp[t] + (st + i) * F::KSTEP);
#pragma unroll
            for (int u = 0; u < NT; ++u) acc[t][u] = F::mma(af, cur[i][u], acc[t][u]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < U; ++i)
#pragma unroll
        for (int u = 0; u < NT; ++u) cur[i][u] = nxt[i][u];
    }
  }

  // lane holds D[16t + 4*lg + i][16u + lr] of this wave
  float (*ytile)[TC + 1] = reinterpret_cast<float (*)[TC + 1]>(smem);  // aliases the X slice
  if (S == 1) {
    __syncthreads();  // every wave is done reading X
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          ytile[16 * t + 4 * lg + i][wave * 16 * NT + 16 * u + lr] = acc[t][u][i] * s_rs[16 * t + 4 * lg + i];
    __syncthreads();
    epi.template run<MT, NT>(TileY<TC>{ytile}, nb, m0, Mt, rmap);
    return;
  }
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int row = rmap.template row<NT>(nb, wave * 16 * NT + 16 * u + lr);
      if (row >= g.N) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * t + 4 * lg + i;
        if (m < Mt) st_coh(g.part + ((size_t)s * g.M + m0 + m) * g.N + row, acc[t][u][i]);
      }
    }
  if (!arrive_last(g.counters + mt * g.nblocks + nb, (unsigned)S)) {
    return;
  }
  // last block of this tile: sum the S partials (fixed order) into LDS.  Each
  // thread owns 4 consecutive columns of PER4 rows; 16 partial loads of every
  // element are in flight at once.
  constexpr int C4 = TC / 4;
  constexpr int PER4 = TR * C4 / GEMM_THREADS;
  uint32_t off[PER4];
  bool ok[PER4];
  float4 sum[PER4];
#pragma unroll
  for (int j = 0; j < PER4; ++j) {
    const int e = threadIdx.x + GEMM_THREADS * j;
    const int m = e / C4, c = (e - m * C4) * 4;
    const int row = rmap.template row<NT>(nb, c);
    ok[j] = m < Mt && row < g.N;
    off[j] = (uint32_t)(((size_t)(m0 + (ok[j] ? m : 0)) * g.N + (ok[j] ? row : 0)) * 4);
    sum[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
  const uint32_t stride = (uint32_t)((size_t)g.M * g.N * 4);
  constexpr int QB = 16 / PER4 > 0 ? 16 / PER4 : 1;
  for (int q0 = 0; q0 < S; q0 += QB) {
    float4 v[QB][PER4];
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int j = 0; j < PER4; ++j)
        v[q][j] = (q0 + q < S && ok[j]) ? ld_coh4(g.part, off[j] + (uint32_t)(q0 + q) * stride)
                                        : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int q = 0; q < QB; ++q)
#pragma unroll
      for (int j = 0; j < PER4; ++j) {
        sum[j].x += v[q][j].x;
        sum[j].y += v[q][j].y;
        sum[j].z += v[q][j].z;
        sum[j].w += v[q][j].w;
      }
  }
#pragma unroll
  for (int j = 0; j < PER4; ++j) {
    const int e = threadIdx.x + GEMM_THREADS * j;
    const int m = e / C4, c = (e - m * C4) * 4;
    const float sc = s_rs[m];
    ytile[m][c] = sum[j].x * sc;
    ytile[m][c + 1] = sum[j].y * sc;
    ytile[m][c + 2] = sum[j].z * sc;
    ytile[m][c + 3] = sum[j].w * sc;
  }
  __syncthreads();
  epi.template run<MT, NT>(TileY<TC>{ytile}, nb, m0, Mt, rmap);
}

// ---------------------------------------------------------------------------
// Input functors: stage X[m0 .. m0+Mt)[k0 .. k0+kw) into LDS.
// ---------------------------------------------------------------------------

// Staging layout shared by the input functors: wave w stages rows w, w + 4, ...
// of the M-tile (at most STAGE_ROWS), lane l the 4-column groups l, l + 64, ... of
// each of them.  A lane's items are handled in batches of STAGE_BATCH whose loads
// are all issued before any result is used: with HBM saturated by the weight
// stream every dependent round trip costs microseconds.
constexpr int STAGE_BATCH = 12;
constexpr int STAGE_ROWS = 8;

struct StageIdx {
  int wave, lane, per_row, n;
  __device__ __forceinline__ StageIdx(int Mt, int kv) {
    wave = threadIdx.x >> 6;
    lane = threadIdx.x & 63;
    per_row = (kv + WAVE - 1) / WAVE;
    const int nr = (Mt - wave + GEMM_WAVES - 1) / GEMM_WAVES;
    n = nr > 0 ? nr * per_row : 0;
  }
  // item -> (row slot j of this wave, tile row mm, column group u)
  __device__ __forceinline__ void at(int it, int& j, int& mm, int& u) const {
    j = it / per_row;
    mm = wave + GEMM_WAVES * j;
    u = lane + WAVE * (it - j * per_row);
  }
};

__device__ __forceinline__ float4 ldg4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ldg4(const bf16* p) {
  const uint2 a = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf2f((bf16)(a.x & 0xffff)), bf2f((bf16)(a.x >> 16)), bf2f((bf16)(a.y & 0xffff)),
                     bf2f((bf16)(a.y >> 16)));
}

// Activations handed from one GEMM to the next are stored ready to stage: for
// bf16 weights as two bf16 arrays, hi = bf16(x) and lo = bf16(x - hi), which give
// the MFMA about 16 mantissa bits of x; for fp32 weights as one fp32 array.
template <typename WT>
struct XSplit {
  WT* hi;
  WT* lo;
  int ld;  // row stride (elements)
  __device__ __forceinline__ void put1(int m, int k, float v) const {
    if constexpr (sizeof(WT) == 2) {
      const uint32_t h = pack2_bf16(v, 0.f);
      hi[(size_t)m * ld + k] = (WT)(h & 0xffffu);
      lo[(size_t)m * ld + k] = (WT)(pack2_bf16(v - __uint_as_float(h << 16), 0.f) & 0xffffu);
    } else {
      hi[(size_t)m * ld + k] = v;
    }
  }
  // the rounded value only (for consumers that take bf16 operands as they are)
  __device__ __forceinline__ void put4_hi(int m, int k, float4 v) const {
    if constexpr (sizeof(WT) == 2) {
      *reinterpret_cast<uint2*>(hi + (size_t)m * ld + k) = make_uint2(pack2_bf16(v.x, v.y), pack2_bf16(v.z, v.w));
    } else {
      *reinterpret_cast<float4*>(hi + (size_t)m * ld + k) = v;
    }
  }
  __device__ __forceinline__ void put4(int m, int k, float4 v) const {
    if constexpr (sizeof(WT) == 2) {
      const uint32_t h0 = pack2_bf16(v.x, v.y), h1 = pack2_bf16(v.z, v.w);
      const uint32_t l0 = pack2_bf16(v.x - __uint_as_float(h0 << 16), v.y - __uint_as_float(h0 & 0xffff0000u));
      const uint32_t l1 = pack2_bf16(v.z - __uint_as_float(h1 << 16), v.w - __uint_as_float(h1 & 0xffff0000u));
      *reinterpret_cast<uint2*>(hi + (size_t)m * ld + k) = make_uint2(h0, h1);
      *reinterpret_cast<uint2*>(lo + (size_t)m * ld + k) = make_uint2(l0, l1);
    } else {
      *reinterpret_cast<float4*>(hi + (size_t)m * ld + k) = v;
    }
  }
};

// X given as an XSplit pair: staging is a copy of 16-byte chunks.  The kernel
// issues the first round of chunk loads before the first weight group and writes
// them to LDS afterwards (chunk() gives the addresses); further rounds follow.
template <typename WT, int RS = RS_NONE>
struct InSplit {
  const WT* hi;
  const WT* lo;
  int K;  // row stride (elements)
  static constexpr bool kTwoPhase = true;
  static constexpr int kRowScale = RS;
  static constexpr int CH = 16 / (int)sizeof(WT);  // elements per chunk
  static constexpr int SB = 4;                     // chunks per thread in the first round
  // chunk i of round r of this thread: tile row m, chunk column c (clamped to a
  // valid chunk when !ok, so that the load can be unconditional)
  static __device__ __forceinline__ void chunk(int r, int i, int Mt, int kw, int& m, int& c, bool& ok) {
    const int nch = kw / CH, n = Mt * nch;
    const int e = (r * SB + i) * GEMM_THREADS + threadIdx.x;
    ok = e < n;
    const int ec = ok ? e : 0;
    m = ec / nch;
    c = ec - m * nch;
  }
};

// X given (float activations)
template <typename WT, typename XT>
struct InAct {
  const XT* X;
  int K;
  __device__ void stage(const XStage<WT>& xs, int m0, int Mt, int k0, int kw, int, int, int) const {
    const int kv = kw >> 2;
    const StageIdx ix(Mt, kv);
    for (int b0 = 0; b0 < ix.n; b0 += STAGE_BATCH) {
      float4 v[STAGE_BATCH];
#pragma unroll
      for (int i = 0; i < STAGE_BATCH; ++i) {
        int j, mm, u;
        ix.at(b0 + i, j, mm, u);
        const bool ok = b0 + i < ix.n && u < kv;
        v[i] = ldg4(X + (ok ? (size_t)(m0 + mm) * K + k0 + 4 * u : (size_t)m0 * K + k0));
      }
#pragma unroll
      for (int i = 0; i < STAGE_BATCH; ++i) {
        int j, mm, u;
        ix.at(b0 + i, j, mm, u);
        if (b0 + i < ix.n && u < kv) {
          const float t[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
          xs.put4(mm, 4 * u, t);
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Epilogues
// ---------------------------------------------------------------------------

// h[row][col] += y; ss_out[nb][row] = sum over the block's columns of h^2; and,
// when xo.hi is set, the next GEMM's input h * gnext as an XSplit (its RMSNorm
// row scale is applied to that GEMM's product from ss_out).
// With `final_`, the epilogue blocks of the M-tile holding row M-1 count in and
// the last one writes h_last = RMSNorm(h[M-1]) * final_norm (h and the sums are
// stored coherently so that block can read them).
template <typename WT>
struct EpiResid {
  float* h;
  float* ss_out;
  int N;  // = d
  int M;
  int final_;
  const WT* final_norm;
  float* h_last;
  unsigned* ctr_final;
  int nblocks;
  float eps;
  XSplit<WT> xo;
  const WT* gnext;
  int n_out;  // final_: rows M - n_out .. M - 1 are final-normed into h_last [n_out][N]
  template <int MT, int NT, typename Y, typename RM>
  __device__ void run(const Y& y, int nb, int m0, int Mt, const RM&) const {
    constexpr int R = 4 * MT;  // rows per wave at most
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float hv[R][NT];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int m = wave + GEMM_WAVES * r;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int col = nb * 64 * NT + lane + 64 * u;
        hv[r][u] = h[(m < Mt && col < N) ? (size_t)(m0 + m) * N + col : (size_t)m0 * N];
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int m = wave + GEMM_WAVES * r;
      if (m >= Mt) break;
      float sq = 0.f;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int c = lane + 64 * u;
        const int col = nb * 64 * NT + c;
        if (col < N) {
          const float v = hv[r][u] + y(m, c);
          st_coh(h + (size_t)(m0 + m) * N + col, v);
          sq += v * v;
          if (xo.hi) xo.put1(m0 + m, col, v * to_f<WT>(gnext[col]));
        }
      }
      sq = wave_sum(sq);
      if (lane == 0) st_coh(ss_out + (size_t)nb * M + m0 + m, sq);
    }
    if (!final_) return;
    // every tile of every row block arrives; the last one normalises the output rows
    const int mtiles = (M + 16 * MT - 1) / (16 * MT);
    if (!arrive_last(ctr_final, (unsigned)(nblocks * mtiles))) return;
    __shared__ float s_inv;
    for (int o = 0; o < n_out; ++o) {
      const int row = M - n_out + o;
      if (threadIdx.x < 64) {
        float t = 0.f;
        for (int p = threadIdx.x; p < nblocks; p += 64) t += ld_coh(ss_out + (size_t)p * M + row);
        t = wave_sum(t);
        if (threadIdx.x == 0) s_inv = 1.0f / sqrtf(t / (float)N + eps);
      }
      __syncthreads();
#pragma unroll 4
      for (int c = threadIdx.x; c < N; c += GEMM_THREADS)
        h_last[(size_t)o * N + c] = ld_coh(h + (size_t)row * N + c) * s_inv * to_f<WT>(final_norm[c]);
      __syncthreads();
    }
  }
};

// act[row][j] = silu(gate_j) * up_j, written as the down projection's XSplit input
template <typename WT>
struct EpiSilu {
  XSplit<WT> out;
  int dff;
  template <int MT, int NT, typename Y, typename RM>
  __device__ void run(const Y& y, int nb, int m0, int Mt, const RM&) const {
    constexpr int H = 32 * NT;
    for (int e = threadIdx.x; e < Mt * H; e += GEMM_THREADS) {
      const int m = e / H, c = e - m * H;
      const int j = nb * H + c;
      if (j >= dff) continue;
      const float gt = y(m, c), up = y(m, c + H);
      out.put1(m0 + m, j, gt / (1.0f + expf(-gt)) * up);
    }
  }
};

// ---------------------------------------------------------------------------
// Host-side launch planning
// ---------------------------------------------------------------------------
struct GemmPlan {
  int MT, NT, S, nblocks, mtiles, nsteps, ldx, x_bytes, ytile_bytes;
  size_t lds_bytes;
};

// Choose split-K so that the grid has at most `target` blocks (or one split), each
// with at least `min_steps` k-steps, and the block's dynamic LDS fits `lds_cap`
// (0: 62 KB for tiles of 16 rows, 78 KB for 32-row tiles, whose staged X slice is
// twice as tall: two blocks per CU either way.  Measured for 32-row tiles against
// 62, 72, 76, 100 and 140 KB: the 9B-shaped 17-row cycle 1105 us (140 KB: 1137),
// a 29-node draft tree's PDM step 363-367 us (379-383) and features 46 us (52);
// 16-row tiles at 70 or 78 KB slow the headline PDM step from 180 to 189 us).
inline GemmPlan plan_gemm(int N, int K, int M, int kstep, int esize, int NT, int target = 512,
                          int min_steps = 8, size_t lds_cap = 0) {
  GemmPlan p;
  if (lds_cap == 0) lds_cap = M > 16 ? 78 * 1024 : 62 * 1024;
  p.MT = M > 16 ? 2 : 1;
  p.NT = NT;
  p.nblocks = (N + 64 * NT - 1) / (64 * NT);
  p.mtiles = (M + 16 * p.MT - 1) / (16 * p.MT);
  p.nsteps = K / kstep;
  int S = target / (p.nblocks * p.mtiles);  // the grid stays within `target` blocks
  int smax = p.nsteps / min_steps;
  if (smax < 1) smax = 1;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  const int rows = M < 16 * p.MT ? M : 16 * p.MT;  // rows actually staged
  p.ytile_bytes = 16 * p.MT * (64 * NT + 1) * 4;
  const int tbn = gemm_tb_buffers(p.MT, NT);
  const size_t tb = esize == 2 ? (size_t)GEMM_WAVES * tbn * TB_WAVE : 0;
  if (esize == 2) lds_cap += (size_t)(tbn - 1) * GEMM_WAVES * TB_WAVE;  // the X budget stays
  for (;;) {
    const int steps = (p.nsteps + S - 1) / S;
    const int ldx = steps * kstep + 16 / esize * 2;  // +32 bytes of padding
    const size_t xb = (size_t)rows * ldx * esize * (esize == 2 ? 2 : 1);  // bf16: hi + lo
    const size_t lds = std::max(xb, (size_t)p.ytile_bytes) + tb;
    if (lds <= lds_cap || S >= p.nsteps) {
      p.S = S;
      p.ldx = ldx;
      p.x_bytes = (int)xb;
      p.lds_bytes = lds;
      break;
    }
    ++S;
  }
  return p;
}

}  // namespace spd
