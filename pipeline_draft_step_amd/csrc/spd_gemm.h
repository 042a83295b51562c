// Skinny GEMM for decode-shaped products: Y[M][N] = X[M][K] . W[N][K]^T with
// M up to 32 per tile and W streamed from HBM once.
//
// Work split: a workgroup (4 waves) owns an N-block of 64*NT weight rows and one
// K-slice of S equal slices; each wave owns 16*NT rows.  The X slice (rows of
// the M-tile) is staged in LDS by an input functor `In` that may fuse a gather
// or a normalisation; W fragments go straight from global memory to the MFMA
// B operand.  With S > 1 each block writes an fp32 partial tile, and the last
// block to arrive for an (N-block, M-tile) sums the S partials in fixed order
// and runs the epilogue functor `Epi`; with S == 1 the tile stays in LDS.
// Results are therefore deterministic for a given launch shape.
#pragma once

#include "spd_common.h"

namespace spd {

constexpr int GEMM_THREADS = 256;
constexpr int GEMM_WAVES = 4;
constexpr int GEMM_UNROLL = 8;

struct GemmShape {
  const void* W;
  int N, K, M;
  int S;             // split-K factor
  int nsteps;        // K / KSTEP
  int ldx;           // LDS row pitch of the staged X slice (elements)
  float* part;       // [S][M][N] partials (S > 1)
  unsigned* counters;  // [mtiles][nblocks]
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
};

template <typename WT, int MT, int NT, typename In, typename Epi, typename RowMap>
__global__ __launch_bounds__(GEMM_THREADS) void gemm_skinny_kernel(GemmShape g, In in, Epi epi,
                                                                   RowMap rmap) {
  typedef Mfma<WT> F;
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int TR = 16 * MT;        // rows per M-tile
  constexpr int TC = 64 * NT;        // columns per N-block
  __shared__ float ytile[TR][TC + 1];  // S == 1 result tile

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

  constexpr bool SPLIT = sizeof(WT) == 2;
  WT* xs = reinterpret_cast<WT*>(smem);
  WT* xs_lo = xs + (size_t)min(TR, g.M) * g.ldx;
  in.stage(XStage<WT>{xs, xs_lo, g.ldx}, m0, Mt, k0, kw, nb, s, S);
  __syncthreads();

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;

  f32x4 acc[MT][NT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int u = 0; u < NT; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // this wave's weight rows: local columns wave*16*NT + 16*u + lr
  const WT* wp[NT];
  bool wv[NT];
#pragma unroll
  for (int u = 0; u < NT; ++u) {
    const int row = rmap.template row<NT>(nb, wave * 16 * NT + 16 * u + lr);
    wv[u] = row < g.N;
    wp[u] = reinterpret_cast<const WT*>(g.W) + (size_t)(wv[u] ? row : 0) * g.K + k0 + lg * F::KPL;
  }
  const WT* xp[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) xp[t] = xs + min(16 * t + lr, Mt - 1) * g.ldx + lg * F::KPL;
  const ptrdiff_t lo_off = xs_lo - xs;

  const int nst = st1 - st0;
  int st = 0;
  for (; st + GEMM_UNROLL <= nst; st += GEMM_UNROLL) {
    typename F::frag wf[GEMM_UNROLL][NT];
#pragma unroll
    for (int i = 0; i < GEMM_UNROLL; ++i)
#pragma unroll
      for (int u = 0; u < NT; ++u) wf[i][u] = F::load(wp[u] + (st + i) * F::KSTEP);
#pragma unroll
    for (int i = 0; i < GEMM_UNROLL; ++i) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        typename F::frag af = F::load(xp[t] + (st + i) * F::KSTEP);
#pragma unroll
        for (int u = 0; u < NT; ++u) acc[t][u] = F::mma(af, wf[i][u], acc[t][u]);
        if constexpr (SPLIT) {
          typename F::frag al = F::load(xp[t] + lo_off + (st + i) * F::KSTEP);
#pragma unroll
          for (int u = 0; u < NT; ++u) acc[t][u] = F::mma(al, wf[i][u], acc[t][u]);
        }
      }
    }
  }
  for (; st < nst; ++st) {
    typename F::frag wf[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) wf[u] = F::load(wp[u] + st * F::KSTEP);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      typename F::frag af = F::load(xp[t] + st * F::KSTEP);
#pragma unroll
      for (int u = 0; u < NT; ++u) acc[t][u] = F::mma(af, wf[u], acc[t][u]);
      if constexpr (SPLIT) {
        typename F::frag al = F::load(xp[t] + lo_off + st * F::KSTEP);
#pragma unroll
        for (int u = 0; u < NT; ++u) acc[t][u] = F::mma(al, wf[u], acc[t][u]);
      }
    }
  }

  // write the tile: lane holds D[16t + 4*lg + i][16u + lr] of this wave
  if (S == 1) {
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int u = 0; u < NT; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) ytile[16 * t + 4 * lg + i][wave * 16 * NT + 16 * u + lr] = acc[t][u][i];
    __syncthreads();
    struct { const float (*y)[TC + 1]; __device__ float operator()(int m, int c) const { return y[m][c]; } } fy{ytile};
    epi.template run<NT>(fy, nb, m0, Mt, rmap);
    return;
  }
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int u = 0; u < NT; ++u) {
      const int row = rmap.template row<NT>(nb, wave * 16 * NT + 16 * u + lr);
      if (!wv[u]) continue;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 16 * t + 4 * lg + i;
        if (m < Mt) g.part[((size_t)s * g.M + m0 + m) * g.N + row] = acc[t][u][i];
      }
    }
  unsigned* ctr = g.counters + mt * g.nblocks + nb;
  if (!arrive_last(ctr, (unsigned)S)) return;
  struct {
    const float* part; int M, N, S, m0, nb; RowMap rm;
    __device__ float operator()(int m, int c) const {
      const int row = rm.template row<NT>(nb, c);
      float v = 0.f;
      for (int q = 0; q < S; ++q) v += part[((size_t)q * M + m0 + m) * N + row];
      return v;
    }
  } fp{g.part, g.M, g.N, S, m0, nb, rmap};
  epi.template run<NT>(fp, nb, m0, Mt, rmap);
  arrival_reset(ctr);
}

// ---------------------------------------------------------------------------
// Input functors: stage X[m0 .. m0+Mt)[k0 .. k0+kw) into LDS as WT.
// ---------------------------------------------------------------------------

// X given (float or bf16 activations) -> WT
template <typename WT, typename XT>
struct InAct {
  const XT* X;
  int K;
  __device__ void stage(const XStage<WT>& xs, int m0, int Mt, int k0, int kw, int, int, int) const {
    const int tot = Mt * kw;
    for (int e = threadIdx.x; e < tot; e += GEMM_THREADS) {
      const int m = e / kw, k = e - m * kw;
      xs.put(m, k, to_f<XT>(X[(size_t)(m0 + m) * K + k0 + k]));
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
  int P;     // partial count
  int M;     // rows of H (ss row stride)
  int K;
  float eps;
  __device__ void stage(const XStage<WT>& xs, int m0, int Mt, int k0, int kw, int, int, int) const {
    __shared__ float inv[32];
    if (threadIdx.x < Mt) {
      float t = 0.f;
      for (int p = 0; p < P; ++p) t += ss[(size_t)p * M + m0 + threadIdx.x];
      inv[threadIdx.x] = 1.0f / sqrtf(t / (float)K + eps);
    }
    __syncthreads();
    const int tot = Mt * kw;
    for (int e = threadIdx.x; e < tot; e += GEMM_THREADS) {
      const int m = e / kw, k = e - m * kw;
      const float v = H[(size_t)(m0 + m) * K + k0 + k] * inv[m] * to_f<WT>(gamma[k0 + k]);
      xs.put(m, k, v);
    }
  }
};

// ---------------------------------------------------------------------------
// Epilogue helpers
// ---------------------------------------------------------------------------

// h[row][col] += y; ss_out[nb][row] = sum over the block's columns of h^2.
// With `final`, the last block of the M-tile holding row M-1 writes
// h_last = RMSNorm(h[M-1]) * final_norm.
template <typename WT>
struct EpiResid {
  float* h;
  float* ss_out;
  int N;   // = d
  int M;
  int final_;
  const WT* final_norm;
  float* h_last;
  unsigned* ctr2;
  int nblocks;
  float eps;
  template <int NT, typename Y, typename RM>
  __device__ void run(const Y& y, int nb, int m0, int Mt, const RM&) const {
    constexpr int TC = 64 * NT;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int m = wave; m < Mt; m += GEMM_WAVES) {
      float sq = 0.f;
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int c = lane + 64 * u;
        const int col = nb * TC + c;
        if (col < N) {
          float* hp = h + (size_t)(m0 + m) * N + col;
          const float v = *hp + y(m, c);
          *hp = v;
          sq += v * v;
        }
      }
      sq = wave_sum(sq);
      if (lane == 0) ss_out[(size_t)nb * M + m0 + m] = sq;
    }
    if (!final_ || m0 + Mt != M) return;
    if (!arrive_last(ctr2, (unsigned)nblocks)) return;
    __shared__ float s_inv;
    if (threadIdx.x == 0) {
      float t = 0.f;
      for (int p = 0; p < nblocks; ++p) t += ss_out[(size_t)p * M + M - 1];
      s_inv = 1.0f / sqrtf(t / (float)N + eps);
    }
    __syncthreads();
    for (int c = threadIdx.x; c < N; c += GEMM_THREADS)
      h_last[c] = h[(size_t)(M - 1) * N + c] * s_inv * to_f<WT>(final_norm[c]);
    arrival_reset(ctr2);
  }
};

// act[row][j] = silu(gate_j) * up_j
template <typename AT>
struct EpiSilu {
  AT* act;
  int dff;
  template <int NT, typename Y, typename RM>
  __device__ void run(const Y& y, int nb, int m0, int Mt, const RM&) const {
    constexpr int H = 32 * NT;
    for (int e = threadIdx.x; e < Mt * H; e += GEMM_THREADS) {
      const int m = e / H, c = e - m * H;
      const int j = nb * H + c;
      if (j >= dff) continue;
      const float gt = y(m, c), up = y(m, c + H);
      const float v = gt / (1.0f + expf(-gt)) * up;
      act[(size_t)(m0 + m) * dff + j] = from_f<AT>(v);
    }
  }
};

// plain store of y (float)
struct EpiStore {
  float* Y;
  int N;
  template <int NT, typename Yf, typename RM>
  __device__ void run(const Yf& y, int nb, int m0, int Mt, const RM&) const {
    constexpr int TC = 64 * NT;
    for (int e = threadIdx.x; e < Mt * TC; e += GEMM_THREADS) {
      const int m = e / TC, c = e - m * TC;
      const int col = nb * TC + c;
      if (col < N) Y[(size_t)(m0 + m) * N + col] = y(m, c);
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
                          int min_steps = 4, size_t lds_cap = 40 * 1024) {
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
