// spd_lm_head: logits = W_lm h over the vocabulary, then the next-token choice.
// ("Speculative Pipeline Decoding", arXiv 2605.30852: section 3.1 Eq. (1), the PDM's
// own head drafts x_{t+1}; section 3.4, the target head forms P of the token under
// verification.)
//
// Launch 1, the vocabulary GEMV (HBM-bound, W_lm read once):
//   rows == 1, bf16, d % 512 == 0: a VALU kernel; each wave owns 8 vocabulary
//     rows, reads every row as 1 KB contiguous loads (lane l: bytes 16l..16l+15
//     of each 1 KB piece) and accumulates v_dot2_f32_bf16 products against h held
//     in registers as a bf16 hi + lo pair; a butterfly reduction finishes a row.
//   otherwise: the MFMA skinny GEMM.
//   Both write the logits and, per block, (max, first argmax, sum exp((l-max)/T)).
// T == 0, launch 2: one block per row merges the block statistics -> greedy token.
// T > 0, launch 2: per 2048-entry chunk, each block merges the statistics (fixed
//   order, so every block gets the same (max, sum)), writes p = exp((l-max)/T)/sum
//   and sums the exact integer weights floor(p*2^52) of its chunk;
//   launch 3: one block per row scans the chunk sums, finds the chunk holding
//   tau = floor(u*S/2^32) and the first index inside it whose prefix exceeds tau.
#include <algorithm>

#include "spd_common.h"
#include "spd_gemm.h"
#include "spd_host.h"

namespace spd {

constexpr int SMX_CHUNK = 2048;  // vocabulary entries per softmax block
constexpr int SMX_THREADS = 256;
constexpr int DOT_ROWS = 8;      // vocabulary rows per wave in the VALU GEMV

struct BlockStat {
  float mx;
  int arg;
  float se;
};

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_v;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a),
                                         __builtin_bit_cast(bf16x2_v, b), c, false);
}

// per-wave statistics of `cnt` logits held one per lane (lanes >= cnt hold -inf)
__device__ __forceinline__ BlockStat lane_stats(float v, int idx, float inv_t) {
  ArgMax am = wave_argmax(ArgMax{v, idx});
  float se = 0.f;
  if (inv_t > 0.f && am.v > -INFINITY) se = wave_sum(v > -INFINITY ? expf((v - am.v) * inv_t) : 0.f);
  return BlockStat{am.v, am.i, se};
}

__device__ __forceinline__ BlockStat stat_merge(BlockStat a, BlockStat b, float inv_t) {
  const ArgMax mm = argmax_merge(ArgMax{a.mx, a.arg}, ArgMax{b.mx, b.arg});
  BlockStat r;
  r.arg = mm.i;
  if (inv_t > 0.f) {
    const float nm = fmaxf(a.mx, b.mx);
    float acc = 0.f;
    if (a.mx > -INFINITY) acc += a.se * expf((a.mx - nm) * inv_t);
    if (b.mx > -INFINITY) acc += b.se * expf((b.mx - nm) * inv_t);
    r.mx = nm;
    r.se = acc;
  } else {
    r.mx = mm.v;
    r.se = 0.f;
  }
  return r;
}

// Merge n block statistics in a fixed order: thread-strided, then a tree.
__device__ BlockStat block_merge_stats(const BlockStat* st, int stride, int n, float inv_t) {
  __shared__ BlockStat sh[SMX_THREADS];
  BlockStat a{-INFINITY, ARG_NONE, 0.f};
#pragma unroll 8
  for (int b = threadIdx.x; b < n; b += SMX_THREADS) a = stat_merge(a, st[(size_t)b * stride], inv_t);
  sh[threadIdx.x] = a;
  __syncthreads();
  for (int w = SMX_THREADS / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) sh[threadIdx.x] = stat_merge(sh[threadIdx.x], sh[threadIdx.x + w], inv_t);
    __syncthreads();
  }
  const BlockStat r = sh[0];
  __syncthreads();
  return r;
}

// VALU GEMV for one hidden row: J = d / 512 loads of 1 KB per vocabulary row.
template <int J>
__global__ __launch_bounds__(256) void lmh_dot_kernel(const bf16* __restrict__ W, const float* __restrict__ h,
                                                      int V, float inv_t, float* __restrict__ logits,
                                                      BlockStat* __restrict__ stat) {
  constexpr int K = 512 * J;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int row0 = (blockIdx.x * 4 + wave) * DOT_ROWS;
  // lane's slice of h: k = 512 j + 8 lane + e, as bf16 hi and lo pairs
  uint32_t hh[J][4], hl[J][4];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const float4 a = *reinterpret_cast<const float4*>(h + 512 * j + 8 * lane);
    const float4 b = *reinterpret_cast<const float4*>(h + 512 * j + 8 * lane + 4);
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16 h0 = f2bf(x[2 * e]), h1 = f2bf(x[2 * e + 1]);
      hh[j][e] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      hl[j][e] = (uint32_t)f2bf(x[2 * e] - bf2f(h0)) | ((uint32_t)f2bf(x[2 * e + 1] - bf2f(h1)) << 16);
    }
  }
  uint4 w[DOT_ROWS][J];
#pragma unroll
  for (int r = 0; r < DOT_ROWS; ++r) {
    const int row = min(row0 + r, V - 1);
#pragma unroll
    for (int j = 0; j < J; ++j) w[r][j] = *reinterpret_cast<const uint4*>(W + (size_t)row * K + 512 * j + 8 * lane);
  }
  float mine = -INFINITY;  // lane r < DOT_ROWS ends with row r's logit
#pragma unroll
  for (int r = 0; r < DOT_ROWS; ++r) {
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const uint32_t* a = reinterpret_cast<const uint32_t*>(&w[r][j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = dot2(a[e], hh[j][e], s);
        s = dot2(a[e], hl[j][e], s);
      }
    }
    s = wave_sum(s);
    if (lane == r) mine = s;
  }
  const int row = row0 + lane;
  const bool valid = lane < DOT_ROWS && row < V;
  if (valid) logits[row] = mine;
  // block statistics over the block's 4 * DOT_ROWS logits
  __shared__ BlockStat ws[4];
  const BlockStat bs = lane_stats(valid ? mine : -INFINITY, valid ? row : ARG_NONE, inv_t);
  if (lane == 0) ws[wave] = bs;
  __syncthreads();
  if (threadIdx.x == 0) {
    BlockStat a = ws[0];
    for (int q = 1; q < 4; ++q) a = stat_merge(a, ws[q], inv_t);
    stat[blockIdx.x] = a;
  }
}

// MFMA-path epilogue: logits and per-block statistics of each row.
struct EpiLogits {
  float* logits;    // [rows][V]
  BlockStat* stat;  // [nblocks][rows]
  int V, rows;
  float inv_t;
  template <int MT, int NT, typename Y, typename RM>
  __device__ void run(const Y& y, int nb, int m0, int Mt, const RM&) const {
    constexpr int TC = 64 * NT;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int m = wave; m < Mt; m += GEMM_WAVES) {
      float v[NT];
      ArgMax am{-INFINITY, ARG_NONE};
#pragma unroll
      for (int u = 0; u < NT; ++u) {
        const int col = nb * TC + lane + 64 * u;
        v[u] = -INFINITY;
        if (col < V) {
          v[u] = y(m, lane + 64 * u);
          logits[(size_t)(m0 + m) * V + col] = v[u];
          am = argmax_merge(am, ArgMax{v[u], col});
        }
      }
      am = wave_argmax(am);
      float se = 0.f;
      if (inv_t > 0.f && am.v > -INFINITY) {
#pragma unroll
        for (int u = 0; u < NT; ++u)
          if (v[u] > -INFINITY) se += expf((v[u] - am.v) * inv_t);
        se = wave_sum(se);
      }
      if (lane == 0) stat[(size_t)nb * rows + m0 + m] = BlockStat{am.v, am.i, se};
    }
  }
};

__global__ __launch_bounds__(SMX_THREADS) void lm_argmax_kernel(const BlockStat* stat, int nstat,
                                                                int rows, int32_t* token) {
  const int r = blockIdx.x;
  const BlockStat s = block_merge_stats(stat + r, rows, nstat, 0.f);
  if (threadIdx.x == 0) token[r] = s.arg == ARG_NONE ? 0 : s.arg;
}

__global__ __launch_bounds__(SMX_THREADS) void softmax_chunk_kernel(const BlockStat* stat, int nstat,
                                                                    int rows, const float* logits,
                                                                    float* probs, uint64_t* csum,
                                                                    int V, int nchunks, float inv_t) {
  const int c = blockIdx.x, r = blockIdx.y;
  const BlockStat s = block_merge_stats(stat + r, rows, nstat, inv_t);
  const float inv_sum = 1.0f / s.se;
  const float* lr = logits + (size_t)r * V;
  float* pr = probs + (size_t)r * V;
  const int base = c * SMX_CHUNK;
  uint64_t part = 0;
  constexpr int PER = SMX_CHUNK / SMX_THREADS;
  float lv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = base + threadIdx.x + SMX_THREADS * e;
    lv[e] = j < V ? lr[j] : -INFINITY;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = base + threadIdx.x + SMX_THREADS * e;
    if (j < V) {
      const float p = expf((lv[e] - s.mx) * inv_t) * inv_sum;
      pr[j] = p;
      part += prob_weight(p);
    }
  }
  part = wave_sum_u64(part);
  __shared__ uint64_t sh[SMX_THREADS / 64];
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = part;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
    for (int w = 0; w < SMX_THREADS / 64; ++w) t += sh[w];
    csum[(size_t)r * nchunks + c] = t;
  }
}

// Inclusive scan of one uint64 per thread across the block (fixed order).
__device__ uint64_t block_scan_u64(uint64_t v, uint64_t* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int o = 1; o < SMX_THREADS; o <<= 1) {
    const uint64_t add = (int)threadIdx.x >= o ? sh[threadIdx.x - o] : 0ull;
    __syncthreads();
    sh[threadIdx.x] += add;
    __syncthreads();
  }
  const uint64_t r = sh[threadIdx.x];
  __syncthreads();
  return r;
}

// Smallest index j of [0, n) whose inclusive prefix of wfun(j), started at
// `offset`, exceeds tau; -1 if none.  Indices are split into contiguous runs of
// `per` per thread, so the scan over thread totals keeps index order.
template <typename WF>
__device__ int block_locate(const WF& wfun, int n, uint64_t offset, uint64_t tau, uint64_t* sh) {
  __shared__ int s_found;
  const int per = (n + SMX_THREADS - 1) / SMX_THREADS;
  if (threadIdx.x == 0) s_found = -1;
  uint64_t tot = 0;
  for (int e = 0; e < per; ++e) {
    const int j = threadIdx.x * per + e;
    if (j < n) tot += wfun(j);
  }
  const uint64_t incl = block_scan_u64(tot, sh);
  uint64_t run = offset + incl - tot;
  if (run <= tau && offset + incl > tau) {  // exactly one thread owns tau
    for (int e = 0; e < per; ++e) {
      const int j = threadIdx.x * per + e;
      if (j >= n) break;
      run += wfun(j);
      if (run > tau) {
        s_found = j;
        break;
      }
    }
  }
  __syncthreads();
  return s_found;
}

struct ChunkSum {
  const uint64_t* c;
  __device__ uint64_t operator()(int j) const { return c[j]; }
};
struct ProbWeight {
  const float* p;
  __device__ uint64_t operator()(int j) const { return prob_weight(p[j]); }
};

__global__ __launch_bounds__(SMX_THREADS) void sample_locate_kernel(const float* probs,
                                                                    const uint64_t* csum,
                                                                    const uint64_t* words, int V,
                                                                    int nchunks, int32_t* token) {
  __shared__ uint64_t sh[SMX_THREADS];
  __shared__ uint64_t s_tau;
  const int r = blockIdx.x;
  const uint64_t* cs = csum + (size_t)r * nchunks;
  uint64_t mine = 0;
  for (int k = threadIdx.x; k < nchunks; k += SMX_THREADS) mine += cs[k];
  mine = wave_sum_u64(mine);
  __shared__ uint64_t s_w[SMX_THREADS / 64];
  if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = mine;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t S = 0;
    for (int w = 0; w < SMX_THREADS / 64; ++w) S += s_w[w];
    s_tau = scale_u32((uint32_t)(words[r] >> 32), S);
  }
  __syncthreads();
  const uint64_t tau = s_tau;
  const int c = block_locate(ChunkSum{cs}, nchunks, 0, tau, sh);
  int tok = 0;
  if (c >= 0) {
    uint64_t off = 0;  // weight before chunk c (same fixed-order sum as the scan)
    __shared__ uint64_t s_off;
    uint64_t part = 0;
    for (int k = threadIdx.x; k < c; k += SMX_THREADS) part += cs[k];
    part = wave_sum_u64(part);
    if ((threadIdx.x & 63) == 0) s_w[threadIdx.x >> 6] = part;
    __syncthreads();
    if (threadIdx.x == 0) {
      for (int w = 0; w < SMX_THREADS / 64; ++w) off += s_w[w];
      s_off = off;
    }
    __syncthreads();
    const int b0 = c * SMX_CHUNK;
    const int j = block_locate(ProbWeight{probs + (size_t)r * V + b0}, min(SMX_CHUNK, V - b0), s_off,
                               tau, sh);
    tok = j < 0 ? 0 : b0 + j;
  }
  if (threadIdx.x == 0) token[r] = tok;
}

struct LmPlan {
  bool dot;
  int J;
  GemmPlan gp;
  int nstat, nchunks;
  size_t off_part, off_stat, off_csum, total;
};

static LmPlan plan_lm(const spd_config* c, int rows) {
  LmPlan p;
  const bool bf = c->dtype == SPD_BF16;
  p.dot = bf && rows == 1 && c->d % 512 == 0 && c->d / 512 <= 8;
  p.J = c->d / 512;
  p.gp = plan_gemm(c->V, c->d, rows, bf ? Mfma<bf16>::KSTEP : Mfma<float>::KSTEP, bf ? 2 : 4, 2,
                   /*target=*/1, /*min_steps=*/1 << 30);
  p.nstat = p.dot ? (c->V + 4 * DOT_ROWS - 1) / (4 * DOT_ROWS) : p.gp.nblocks;
  p.nchunks = (c->V + SMX_CHUNK - 1) / SMX_CHUNK;
  size_t off = SPD_WS_COUNTER_BYTES;
  auto take = [&](size_t b) { size_t r = off; off = align256(off + b); return r; };
  p.off_part = take(!p.dot && p.gp.S > 1 ? (size_t)p.gp.S * rows * c->V * 4 : 0);
  p.off_stat = take((size_t)p.nstat * rows * sizeof(BlockStat));
  p.off_csum = take((size_t)rows * p.nchunks * 8);
  p.total = off;
  return p;
}

size_t lm_head_workspace(const spd_config* cfg, int rows) { return plan_lm(cfg, rows).total; }

template <int J>
static void launch_dot(int nblk, hipStream_t st, const void* w, const float* h, int V, float inv_t,
                       float* logits, BlockStat* stat) {
  hipLaunchKernelGGL((lmh_dot_kernel<J>), dim3(nblk), dim3(256), 0, st, static_cast<const bf16*>(w), h,
                     V, inv_t, logits, stat);
}

template <typename WT>
static int lm_impl(const spd_config* c, const void* w_lm, const float* h, int rows, float T,
                   const uint64_t* words, float* logits, float* probs, int32_t* token, void* ws,
                   hipStream_t st) {
  const LmPlan p = plan_lm(c, rows);
  char* w = static_cast<char*>(ws);
  BlockStat* stat = reinterpret_cast<BlockStat*>(w + p.off_stat);
  const float inv_t = T > 0.f ? 1.0f / T : 0.f;
  int rc;
  if (p.dot) {
    switch (p.J) {
      case 1: launch_dot<1>(p.nstat, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 2: launch_dot<2>(p.nstat, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 3: launch_dot<3>(p.nstat, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 4: launch_dot<4>(p.nstat, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 5: launch_dot<5>(p.nstat, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 6: launch_dot<6>(p.nstat, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 7: launch_dot<7>(p.nstat, st, w_lm, h, c->V, inv_t, logits, stat); break;
      default: launch_dot<8>(p.nstat, st, w_lm, h, c->V, inv_t, logits, stat); break;
    }
    rc = check_launch();
  } else {
    GemmShape g{};
    g.W = w_lm;
    g.N = c->V;
    g.K = c->d;
    g.M = rows;
    g.S = p.gp.S;
    g.nsteps = p.gp.nsteps;
    g.ldx = p.gp.ldx;
    g.part = reinterpret_cast<float*>(w + p.off_part);
    g.nblocks = p.gp.nblocks;
    EpiLogits epi{logits, stat, c->V, rows, inv_t};
    rc = launch_gemm<WT, 2>(p.gp, g, InAct<WT, float>{h, c->d}, epi, RowMapStd{}, st);
  }
  if (rc) return rc;
  if (T <= 0.f) {
    hipLaunchKernelGGL(lm_argmax_kernel, dim3(rows), dim3(SMX_THREADS), 0, st, stat, p.nstat, rows,
                       token);
    return check_launch();
  }
  uint64_t* csum = reinterpret_cast<uint64_t*>(w + p.off_csum);
  hipLaunchKernelGGL(softmax_chunk_kernel, dim3(p.nchunks, rows), dim3(SMX_THREADS), 0, st, stat,
                     p.nstat, rows, logits, probs, csum, c->V, p.nchunks, inv_t);
  rc = check_launch();
  if (rc) return rc;
  hipLaunchKernelGGL(sample_locate_kernel, dim3(rows), dim3(SMX_THREADS), 0, st, probs, csum, words,
                     c->V, p.nchunks, token);
  return check_launch();
}

}  // namespace spd

using namespace spd;

extern "C" int spd_lm_head(const spd_config* cfg, const void* w_lm, const float* h, int32_t rows,
                           float temperature, const uint64_t* words, float* logits, float* probs,
                           int32_t* token, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!w_lm || !h || !logits || !token || !ws) return SPD_E_INVALID;
  if (rows < 1 || rows > 16) return SPD_E_INVALID;
  if (!(temperature >= 0.f) || temperature == INFINITY) return SPD_E_INVALID;
  if (temperature > 0.f && (!probs || !words)) return SPD_E_INVALID;
  if (cfg->d % 64) return SPD_E_UNSUPPORTED;
  if ((int64_t)cfg->V * cfg->d > ((int64_t)1 << 40)) return SPD_E_UNSUPPORTED;
  if (!aligned16(w_lm) || !aligned16(h) || !aligned16(ws)) return SPD_E_INVALID;
  if (ws_bytes < lm_head_workspace(cfg, rows)) return SPD_E_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cfg->dtype == SPD_BF16)
    return lm_impl<bf16>(cfg, w_lm, h, rows, temperature, words, logits, probs, token, ws, st);
  return lm_impl<float>(cfg, w_lm, h, rows, temperature, words, logits, probs, token, ws, st);
}
