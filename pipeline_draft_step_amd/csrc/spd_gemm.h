// Skinny GEMM for decode-shaped products: Y[M][N] = X[M][K] . W[N][K]^T with
// M up to 32 per tile and W streamed from HBM once.
//
// Work split: a workgroup (4 waves) owns an N-block of 64*NT weight rows and one
// of S equal K-slices; each wave owns 16*NT rows.  The X slice (rows of the
// M-tile) is staged in LDS by an input functor `In` that may fuse a gather or a
// normalisation; W fragments go straight from global memory to the MFMA B
// operand, double-buffered so that a full unrolled group of loads is always in
// flight.  With S == 1 the block runs the epilogue functor `Epi` on its own
// tile.  With S > 1 it writes an fp32 partial tile and a second, small kernel
// sums the S partials in fixed order and runs the epilogue: cross-block
// reductions happen at kernel boundaries only (a device-scope fence per block
// costs far more than a launch on this multi-die part).  Results are
// deterministic for a given launch shape.
#pragma once

#include "spd_common.h"

namespace spd {

#ifndef SPD_GEMM_UNROLL
#define SPD_GEMM_UNROLL 8     // k-steps of weight loads in flight per wave (double-buffered)
#endif
#ifndef SPD_GEMM_TARGET
#define SPD_GEMM_TARGET 1024  // blocks a split-K launch aims for
#endif
#ifndef SPD_GEMM_MIN_STEPS
#define SPD_GEMM_MIN_STEPS 8  // minimum k-steps per split
#endif

constexpr int GEMM_THREADS = 256;
constexpr int GEMM_WAVES = 4;
constexpr int GEMM_UNROLL = SPD_GEMM_UNROLL;

struct GemmShape {
  const void* W;
  int N, K, M;
  int S;        // split-K factor
  int nsteps;   // K / KSTEP
  int ldx;      // LDS row pitch of the staged X slice (elements)
  float* part;  // [S][M][N] partials (S > 1)
  int nblocks;
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
      bf16 h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = f2bf(v[e]);
        l[e] = f2bf(v[e] - bf2f(h[e]));
      }
      *reinterpret_cast<uint2*>(hi + m * ldx + k) =
          make_uint2(h[0] | ((uint32_t)h[1] << 16), h[2] | ((uint32_t)h[3] << 16));
      *reinterpret_cast<uint2*>(lo + m * ldx + k) =
          make_uint2(l[0] | ((uint32_t)l[1] << 16), l[2] | ((uint32_t)l[3] << 16));
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
  constexpr int U = GEMM_UNROLL;
  extern __shared__ __align__(16) unsigned char smem[];

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

  // this wave's weight rows: local columns wave*16*NT + 16*u + lr
  const WT* wp[NT];
  bool wv[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int row = rmap.template row<NT>(nb, wave * 16 * NT + 16 * u + lr);
    wv[u] = row < g.N;
    wp[u] = reinterpret_cast<const WT*>(g.W) + (size_t)(wv[u] ? row : 0) * g.K + k0 + lg * F::KPL;
  }
  // the first group of weight loads goes out before the X slice is staged
  frag cur[U][NT], nxt[U][NT];
#pragma unroll
  for (int i = 0; i < U; ++i)
#pragma unroll
    for (int u = 0; u < NT; ++u) cur[i][u] = i < nst ? F::load(wp[u] + i * F::KSTEP) : F::zero();

  WT* xs = reinterpret_cast<WT*>(smem);
  WT* xs_lo = xs + (size_t)min(TR, g.M) * g.ldx;
  in.stage(XStage<WT>{xs, xs_lo, g.ldx}, m0, Mt, k0, kw, nb, s, S);
  __syncthreads();

  f32x4 acc[MT][NT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int u = 0; u < NT; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};
  const WT* xp[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xp[t] = xs + min(16 * t + lr, Mt - 1) * g.ldx + lg * F::KPL;
  const ptrdiff_t lo_off = xs_lo - xs;

  for (int st = 0; st < nst; st += U) {
    const int nxt0 = st + U;
    if (nxt0 < nst) {
#pragma unroll
      for (int i = 0; i < U; ++i)
#pragma unroll
        for (int u = 0; u < NT; ++u)
          nxt[i][u] = nxt0 + i < nst ? F::load(wp[u] + (nxt0 + i) * F::KSTEP) : F::zero();
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
          if constexpr (SPLIT) {
            const frag al = F::load(xp[t] + lo_off + (st + i) * F::KSTEP);
#pragma unroll
            for (int u = 0; u < NT; ++u) acc[t][u] = F::mma(al, cur[i][u], acc[t][u]);
          }
        }
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < U; ++i)
#pragma unroll
      for (int u = 0; u < NT; ++u) cur[i][u] = nxt[i][u];
  }

  // lane holds D[16t + 4*lg + i][16u + lr] of this wave
  if (S == 1) {
    __shared__ float ytile[TR][TC + 1];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) ytile[16 * t + 4 * lg + i][wave * 16 * NT + 16 * u + lr] = acc[t][u][i];
    __syncthreads();
    epi.template run<MT, NT>(TileY<TC>{ytile}, nb, m0, Mt, rmap);
    return;
  }
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      if (!wv[u]) continue;
      const int row = rmap.template row<NT>(nb, wave * 16 * NT + 16 * u + lr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * t + 4 * lg + i;
        if (m < Mt) g.part[((size_t)s * g.M + m0 + m) * g.N + row] = acc[t][u][i];
      }
    }
}

// Sum of the S partial tiles of one (N-block, M-tile) into LDS (fixed order over
// the splits, all loads of a split in flight together), then the epilogue.
template <int MT, int NT, typename Epi, typename RowMap>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_finish_kernel(GemmShape g, Epi epi, RowMap rmap) {
  constexpr int TR = 16 * MT, TC = 64 * NT;
  constexpr int PER = TR * TC / GEMM_THREADS;  // tile entries per thread
  __shared__ float ytile[TR][TC + 1];
  const int nb = blockIdx.x, mt = blockIdx.y;
  const int m0 = mt * TR;
  const int Mt = min(TR, g.M - m0);
  const float* ptr[PER];
  bool ok[PER];
  float acc[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = threadIdx.x + GEMM_THREADS * j;
    const int m = e / TC, c = e - m * TC;
    const int row = rmap.template row<NT>(nb, c);
    ok[j] = m < Mt && row < g.N;
    ptr[j] = g.part + (size_t)(m0 + (ok[j] ? m : 0)) * g.N + (ok[j] ? row : 0);
    acc[j] = 0.f;
  }
  const size_t stride = (size_t)g.M * g.N;
#pragma unroll 2
  for (int q = 0; q < g.S; ++q) {
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = ok[j] ? ptr[j][q * stride] : 0.f;
#pragma unroll
    for (int j = 0; j < PER; ++j) acc[j] += v[j];
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = threadIdx.x + GEMM_THREADS * j;
    ytile[e / TC][e % TC] = acc[j];
  }
  __syncthreads();
  epi.template run<MT, NT>(TileY<TC>{ytile}, nb, m0, Mt, rmap);
}

// ---------------------------------------------------------------------------
// Input functors: stage X[m0 .. m0+Mt)[k0 .. k0+kw) into LDS.
// ---------------------------------------------------------------------------

// X given (float or bf16 activations)
template <typename WT, typename XT>
struct InAct {
  const XT* X;
  int K;
  __device__ void stage(const XStage<WT>& xs, int m0, int Mt, int k0, int kw, int, int, int) const {
    const int kv = kw >> 2;
#pragma unroll 4
    for (int e = threadIdx.x; e < Mt * kv; e += GEMM_THREADS) {
      const int m = e / kv, k = (e - m * kv) << 2;
      float v[4];
      load4(X + (size_t)(m0 + m) * K + k0 + k, v);
      xs.put4(m, k, v);
    }
  }
};

// X = RMSNorm(H) * gamma, with the row statistics summed from per-block
// partial sums of squares ss[p][row] written by the producer of H.
template <typename WT>
struct InNorm {
  const float* H;
  const WT* gamma;
  const float* ss;
  int P;  // partial count
  int M;  // rows of H (ss row stride)
  int K;
  float eps;
  __device__ void stage(const XStage<WT>& xs, int m0, int Mt, int k0, int kw, int, int, int) const {
    __shared__ float inv[32];
    const int wave = threadIdx.x >> 6;
    for (int m = wave; m < Mt; m += GEMM_WAVES) {
      const float* sp = ss + m0 + m;
      const float t = wave_sum_of(P, [&](int p) { return sp[(size_t)p * M]; });
      if ((threadIdx.x & 63) == 0) inv[m] = 1.0f / sqrtf(t / (float)K + eps);
    }
    __syncthreads();
    const int kv = kw >> 2;
#pragma unroll 4
    for (int e = threadIdx.x; e < Mt * kv; e += GEMM_THREADS) {
      const int m = e / kv, k = (e - m * kv) << 2;
      float v[4], gm[4];
      load4(H + (size_t)(m0 + m) * K + k0 + k, v);
      load4(gamma + k0 + k, gm);
      const float iv = inv[m];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = v[i] * iv * gm[i];
      xs.put4(m, k, v);
    }
  }
};

// ---------------------------------------------------------------------------
// Epilogues
// ---------------------------------------------------------------------------

// h[row][col] += y; ss_out[nb][row] = sum over the block's columns of h^2.
struct EpiResid {
  float* h;
  float* ss_out;
  int N;  // = d
  int M;
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
        hv[r][u] = (m < Mt && col < N) ? h[(size_t)(m0 + m) * N + col] : 0.f;
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
          h[(size_t)(m0 + m) * N + col] = v;
          sq += v * v;
        }
      }
      sq = wave_sum(sq);
      if (lane == 0) ss_out[(size_t)nb * M + m0 + m] = sq;
    }
  }
};

// act[row][j] = silu(gate_j) * up_j
struct EpiSilu {
  float* act;
  int dff;
  template <int MT, int NT, typename Y, typename RM>
  __device__ void run(const Y& y, int nb, int m0, int Mt, const RM&) const {
    constexpr int H = 32 * NT;
    for (int e = threadIdx.x; e < Mt * H; e += GEMM_THREADS) {
      const int m = e / H, c = e - m * H;
      const int j = nb * H + c;
      if (j >= dff) continue;
      const float gt = y(m, c), up = y(m, c + H);
      act[(size_t)(m0 + m) * dff + j] = gt / (1.0f + expf(-gt)) * up;
    }
  }
};

// ---------------------------------------------------------------------------
// Host-side launch planning
// ---------------------------------------------------------------------------
struct GemmPlan {
  int MT, NT, S, nblocks, mtiles, nsteps, ldx;
  size_t lds_bytes;
};

// Choose split-K so that the grid has about `target` blocks, each with at least
// `min_steps` k-steps, and the staged slice fits `lds_cap` bytes.
inline GemmPlan plan_gemm(int N, int K, int M, int kstep, int esize, int NT, int target = 1024,
                          int min_steps = 8, size_t lds_cap = 40 * 1024) {
  GemmPlan p;
  p.MT = M > 16 ? 2 : 1;
  p.NT = NT;
  p.nblocks = (N + 64 * NT - 1) / (64 * NT);
  p.mtiles = (M + 16 * p.MT - 1) / (16 * p.MT);
  p.nsteps = K / kstep;
  int S = (target + p.nblocks * p.mtiles - 1) / (p.nblocks * p.mtiles);
  int smax = p.nsteps / min_steps;
  if (smax < 1) smax = 1;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  const int rows = M < 16 * p.MT ? M : 16 * p.MT;  // rows actually staged
  for (;;) {
    const int steps = (p.nsteps + S - 1) / S;
    const int ldx = steps * kstep + 16 / esize * 2;  // +32 bytes of padding
    const size_t lds = (size_t)rows * ldx * esize * (esize == 2 ? 2 : 1);  // bf16: hi + lo
    if (lds <= lds_cap || S >= p.nsteps) {
      p.S = S;
      p.ldx = ldx;
      p.lds_bytes = lds;
      break;
    }
    ++S;
  }
  return p;
}

}  // namespace spd
