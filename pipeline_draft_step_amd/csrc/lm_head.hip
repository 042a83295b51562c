// spd_lm_head: logits = W_lm h over the vocabulary, then the next-token choice.
// ("Speculative Pipeline Decoding", arXiv 2605.30852: section 3.1 Eq. (1), the PDM's
// own head drafts x_{t+1}; section 3.4, the target head forms P of the token under
// verification.)
//
// Launch 1, the vocabulary GEMV (HBM-bound, W_lm read once):
//   rows == 1, bf16, d % 512 == 0: a VALU kernel; each wave owns 8 vocabulary
//     rows, reads every row as 1 KB contiguous loads (lane l: bytes 16l..16l+15
//     of each 1 KB piece) and accumulates v_dot2_f32_bf16 products against h held
//     in registers as a bf16 hi + lo pair; a reduction finishes a row.  A wave
//     issues the loads of all 8 rows at once, or of one row at a time when the
//     grid is capped (a head streaming beside other work).
//   otherwise: the MFMA skinny GEMM.
//   Both write the logits and, per block, (max, first argmax, sum exp((l-max)/T)).
//   The last block to finish merges the block statistics in a fixed order into
//   the row's (max, argmax, sum); at T == 0 it writes the greedy token.
// T > 0, launch 2: per 2048-entry chunk, p = exp((l-max)/T)/sum and the sum of
//   the exact integer weights floor(p*2^52) of the chunk; the last chunk block
//   of a row scans the chunk sums, finds the chunk holding tau = floor(u*S/2^32)
//   and the first index inside it whose prefix exceeds tau.
#include <algorithm>
#include <mutex>

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

// per-wave statistics of logits held one per lane (lanes without one hold -inf)
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

__device__ __forceinline__ void st_stat(BlockStat* p, BlockStat s) {
  float* q = reinterpret_cast<float*>(p);
  st_coh(q, s.mx);
  st_coh_i32(reinterpret_cast<int*>(q + 1), s.arg);
  st_coh(q + 2, s.se);
}
__device__ __forceinline__ BlockStat ld_stat(const BlockStat* p) {
  const float* q = reinterpret_cast<const float*>(p);
  return BlockStat{ld_coh(q), ld_coh_i32(reinterpret_cast<const int*>(q + 1)), ld_coh(q + 2)};
}

// Block-wide merge of the n statistics st[b * stride], b < n, in a fixed order:
// thread-strided runs (every load of a round issued first), then a butterfly
// within each wave, then the four waves in order.  Every thread gets the result.
template <bool COH>
__device__ BlockStat merge_stats(const BlockStat* st, int stride, int n, float inv_t) {
  __shared__ BlockStat s_ws[SMX_THREADS / 64];
  constexpr int PB = 20;  // one round of loads for up to 5120 statistics
  BlockStat a{-INFINITY, ARG_NONE, 0.f};
  for (int b0 = 0; b0 < n; b0 += PB * SMX_THREADS) {
    BlockStat v[PB];
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int b = b0 + threadIdx.x + SMX_THREADS * i;
      const BlockStat* q = st + (size_t)(b < n ? b : 0) * stride;
      v[i] = COH ? ld_stat(q) : *q;
    }
#pragma unroll
    for (int i = 0; i < PB; ++i)
      if (b0 + (int)threadIdx.x + SMX_THREADS * i < n) a = stat_merge(a, v[i], inv_t);
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const BlockStat b{__shfl_xor(a.mx, o, WAVE), __shfl_xor(a.arg, o, WAVE), __shfl_xor(a.se, o, WAVE)};
    // lower lane index first, so that both partners compute the same value
    a = (threadIdx.x & o) ? stat_merge(b, a, inv_t) : stat_merge(a, b, inv_t);
  }
  if ((threadIdx.x & 63) == 0) s_ws[threadIdx.x >> 6] = a;
  __syncthreads();
  BlockStat r = s_ws[0];
#pragma unroll
  for (int w = 1; w < SMX_THREADS / 64; ++w) r = stat_merge(r, s_ws[w], inv_t);
  __syncthreads();
  return r;
}

// Where the merged statistics of each row go.
struct HeadFinish {
  unsigned* counters;  // arrival counters (two-level, 17 x 16 words)
  BlockStat* gstat;    // [rows] merged statistics
  int32_t* token;      // [rows], written when greedy (T == 0)
  int greedy;
};

__device__ void finish_row(const BlockStat* st, int stride, int n, int r, float inv_t,
                           const HeadFinish& f) {
  const BlockStat g = merge_stats<true>(st, stride, n, inv_t);
  if (threadIdx.x == 0) {
    f.gstat[r] = g;
    if (f.greedy) f.token[r] = g.arg == ARG_NONE ? 0 : g.arg;
  }
}

// T == 0 after the VALU GEMV: one block per row merges the block statistics.
__global__ __launch_bounds__(SMX_THREADS) void greedy_kernel(const BlockStat* stat, int nstat,
                                                             int rows, int32_t* token) {
  const int r = blockIdx.x;
  const BlockStat g = merge_stats<false>(stat + r, rows, nstat, 0.f);
  if (threadIdx.x == 0) token[r] = g.arg == ARG_NONE ? 0 : g.arg;
}

// VALU GEMV for one hidden row: J = d / 512 loads of 1 KB per vocabulary row.
// A row group is 4 waves x DOT_ROWS rows; block b takes groups b, b + grid, ...
// and writes one statistics record per group.  A wave loads its rows R at a time
// (R == DOT_ROWS: all at once); the arithmetic of every row is the same for any R.
template <int J, int R>
__global__ __launch_bounds__(256) void lmh_dot_kernel(const bf16* __restrict__ W, const float* __restrict__ h,
                                                      int V, float inv_t, float* __restrict__ logits,
                                                      BlockStat* __restrict__ stat) {
  static_assert(DOT_ROWS % R == 0, "row batches");
  constexpr int K = 512 * J;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ngroups = (V + 4 * DOT_ROWS - 1) / (4 * DOT_ROWS);
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
  __shared__ BlockStat ws[4];
  for (int grp = blockIdx.x; grp < ngroups; grp += gridDim.x) {
    const int row0 = (grp * 4 + wave) * DOT_ROWS;
    float mine = -INFINITY;  // lane r < DOT_ROWS ends with row r's logit
#pragma unroll
    for (int rb = 0; rb < DOT_ROWS; rb += R) {
      uint4 w[R][J];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const int row = min(row0 + rb + r, V - 1);
#pragma unroll
        for (int j = 0; j < J; ++j) {
          // the head is read once per call: nontemporal loads stream it past the caches
          w[r][j] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                                 reinterpret_cast<const u32x4*>(W + (size_t)row * K + 512 * j + 8 * lane)));
        }
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
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
        if (lane == rb + r) mine = s;
      }
      // the next batch's loads go out only after this batch is consumed
      if (R < DOT_ROWS) __builtin_amdgcn_sched_barrier(0);
    }
    const int row = row0 + lane;
    const bool valid = lane < DOT_ROWS && row < V;
    if (valid) logits[row] = mine;
    // statistics over the group's 4 * DOT_ROWS logits
    const BlockStat bs = lane_stats(valid ? mine : -INFINITY, valid ? row : ARG_NONE, inv_t);
    if (lane == 0) ws[wave] = bs;
    __syncthreads();
    if (threadIdx.x == 0) {
      BlockStat a = ws[0];
      for (int q = 1; q < 4; ++q) a = stat_merge(a, ws[q], inv_t);
      stat[grp] = a;
    }
    __syncthreads();  // ws is rewritten by the next group
  }
}

// MFMA-path epilogue: logits and per-block statistics of each row.
struct EpiLogits {
  float* logits;    // [rows][V]
  BlockStat* stat;  // [nblocks][rows]
  int V, rows;
  float inv_t;
  int nblocks;
  HeadFinish f;
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
      if (lane == 0) st_stat(stat + (size_t)nb * rows + m0 + m, BlockStat{am.v, am.i, se});
    }
    // every N-block runs this epilogue once (the tile covers all rows)
    if (!arrive_last2(f.counters, nb, nblocks, 16)) return;
    for (int r = 0; r < rows; ++r) finish_row(stat + r, rows, nblocks, r, inv_t, f);
  }
};

// inclusive prefix sum over the lanes of a wave (lane order)
__device__ __forceinline__ uint64_t wave_scan_u64(uint64_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < WAVE; o <<= 1) {
    const uint32_t lo = __shfl_up((uint32_t)v, o, WAVE), hi = __shfl_up((uint32_t)(v >> 32), o, WAVE);
    if (lane >= o) v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

// Row statistics at T > 0 from the GEMV's block statistics: M = max mx_b, then
// S = sum_b se_b exp((mx_b - M)/T), each in a fixed order (thread runs, DPP
// within waves, waves in order); every thread gets the result.  Up to
// 20 * 256 statistics stay in registers between the two passes.
__device__ void stats_max_sum(const BlockStat* st, int stride, int n, float inv_t, float& M, float& S) {
  __shared__ float s_r[SMX_THREADS / 64];
  constexpr int PB = 20;
  const int wave = threadIdx.x >> 6;
  const bool one_round = n <= PB * SMX_THREADS;
  float m[PB], e[PB];
  float mx = -INFINITY;
  for (int b0 = 0; b0 < n; b0 += PB * SMX_THREADS) {
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int b = b0 + threadIdx.x + SMX_THREADS * i;
      const BlockStat q = st[(size_t)(b < n ? b : 0) * stride];
      const bool ok = b < n;
      m[i] = ok ? q.mx : -INFINITY;
      e[i] = ok ? q.se : 0.f;
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) mx = fmaxf(mx, m[i]);
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) s_r[wave] = mx;
  __syncthreads();
  M = fmaxf(fmaxf(s_r[0], s_r[1]), fmaxf(s_r[2], s_r[3]));
  __syncthreads();
  float sum = 0.f;
  if (one_round) {
#pragma unroll
    for (int i = 0; i < PB; ++i)
      if (m[i] > -INFINITY) sum += e[i] * expf((m[i] - M) * inv_t);
  } else {
    for (int b0 = 0; b0 < n; b0 += PB * SMX_THREADS) {
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        const int b = b0 + threadIdx.x + SMX_THREADS * i;
        const BlockStat q = st[(size_t)(b < n ? b : 0) * stride];
        const bool ok = b < n;
        m[i] = ok ? q.mx : -INFINITY;
        e[i] = ok ? q.se : 0.f;
      }
#pragma unroll
      for (int i = 0; i < PB; ++i)
        if (m[i] > -INFINITY) sum += e[i] * expf((m[i] - M) * inv_t);
    }
  }
  sum = wave_sum(sum);
  if ((threadIdx.x & 63) == 0) s_r[wave] = sum;
  __syncthreads();
  S = (s_r[0] + s_r[1]) + (s_r[2] + s_r[3]);
  __syncthreads();
}

constexpr int SMX_MAXCH = 4 * WAVE;  // chunks one wave scans (vocabulary <= 524288)

// T > 0: one block per (2048-entry chunk, row).  Probabilities and chunk weight
// sums are stored coherently; the last chunk block of the row samples: wave 0
// scans the chunk sums and finds the chunk holding tau, then the block scans the
// weights of that chunk (8 consecutive entries per thread).
// The row statistics are either derived here from the GEMV's nstat block
// statistics (every block in the same fixed order, so all agree) or, when
// nstat == 0, read from gstat.
__global__ __launch_bounds__(SMX_THREADS) void softmax_sample_kernel(
    const BlockStat* stat, int nstat, int rows, const BlockStat* gstat, const float* logits,
    float* probs, uint64_t* csum, unsigned* counters, const uint64_t* words, int V, int nchunks,
    float inv_t, int32_t* token) {
  __shared__ uint64_t s_w[SMX_THREADS / 64];
  __shared__ uint64_t s_tau, s_off;
  __shared__ int s_cc, s_tok;
  const int c = blockIdx.x, r = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  float M, S;
  if (nstat > 0) {
    stats_max_sum(stat + r, rows, nstat, inv_t, M, S);
  } else {
    M = gstat[r].mx;
    S = gstat[r].se;
  }
  const float inv_sum = 1.0f / S;
  const float* lr = logits + (size_t)r * V;
  float* pr = probs + (size_t)r * V;
  const int base = c * SMX_CHUNK;
  constexpr int PER = SMX_CHUNK / SMX_THREADS;
  float lv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = base + threadIdx.x + SMX_THREADS * e;
    lv[e] = lr[j < V ? j : 0];
  }
  uint64_t part = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = base + threadIdx.x + SMX_THREADS * e;
    if (j < V) {
      const float p = expf((lv[e] - M) * inv_t) * inv_sum;
      st_coh(pr + j, p);
      part += prob_weight(p);
    }
  }
  part = wave_sum_u64(part);
  if (lane == 0) s_w[wave] = part;
  __syncthreads();
  if (threadIdx.x == 0)
    st_coh_u64(csum + (size_t)r * nchunks + c, (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]));
  if (!arrive_last(counters + r, (unsigned)nchunks)) {
    return;
  }
  const uint64_t* cs = csum + (size_t)r * nchunks;
  if (wave == 0) {
    // lane l holds chunks 4l .. 4l+3
    uint64_t cw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = 4 * lane + i;
      const uint64_t t = ld_coh_u64(cs + (k < nchunks ? k : 0));
      cw[i] = k < nchunks ? t : 0ull;
    }
    const uint64_t tot = (cw[0] + cw[1]) + (cw[2] + cw[3]);
    const uint64_t incl = wave_scan_u64(tot);
    const uint64_t Sw = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(incl >> 32), 63) << 32) |
                        (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)incl, 63);
    const uint64_t tau = scale_u32((uint32_t)(words[r] >> 32), Sw);
    uint64_t run = incl - tot;
    if (lane == 0) {
      s_tau = tau;
      s_cc = -1;
    }
    if (run <= tau && tau < incl) {  // exactly one lane (none when the total is 0)
      int cc = -1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (cc < 0 && tau < run + cw[i]) {
          cc = 4 * lane + i;
        } else if (cc < 0) {
          run += cw[i];
        }
      }
      s_cc = cc;
      s_off = run;
    }
  }
  __syncthreads();
  const int cc = s_cc;
  if (cc < 0) {
    if (threadIdx.x == 0) token[r] = 0;
    return;
  }
  // weights of chunk cc: thread t owns entries 8t .. 8t+7
  const int b0 = cc * SMX_CHUNK;
  const int n = min(SMX_CHUNK, V - b0);
  uint64_t w[PER];
  {
    float pv[PER];  // clamped indices: the last chunk may be partial
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int j = (int)threadIdx.x * PER + e;
      pv[e] = ld_coh(pr + b0 + (j < n ? j : 0));
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) w[e] = (int)threadIdx.x * PER + e < n ? prob_weight(pv[e]) : 0ull;
  }
  uint64_t tot = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) tot += w[e];
  const uint64_t winc = wave_scan_u64(tot);
  if (lane == 63) s_w[wave] = winc;
  if (threadIdx.x == 0) s_tok = -1;
  __syncthreads();
  uint64_t before = s_off;
  for (int q = 0; q < wave; ++q) before += s_w[q];
  uint64_t run = before + winc - tot;
  const uint64_t tau = s_tau;
  if (run <= tau && tau < run + tot) {
    int found = -1;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (found < 0) {
        run += w[e];
        if (run > tau) found = (int)threadIdx.x * PER + e;
      }
    }
    s_tok = b0 + found;
  }
  __syncthreads();
  if (threadIdx.x == 0) token[r] = s_tok < 0 ? 0 : s_tok;
}

// ---------------------------------------------------------------- top-k / top-p sampling
//
// Sampling filters of the evaluation setting of "Speculative Pipeline Decoding"
// (section 4: T = 1 with top-k = 50 and top-p = 1.0).  One kernel, grid
// (chunks, rows): every block selects its chunk's k largest logits with a radix
// selection in LDS, hands them over as candidates and zeroes the rest of its
// probability range; the last block to arrive selects the k largest of all
// candidates, applies the nucleus cut, writes their probabilities and draws the
// token with the same exact integer inverse CDF as the unfiltered path.  Every
// probability entry is written by exactly one block.

constexpr int TOPK_BINS = 2048;        // 11-bit digits
constexpr int TOPK_KMAX = SPD_TOP_K_MAX;
constexpr int TOPK_BATCH = 16;         // candidate keys per thread and load batch
static_assert(TOPK_KMAX <= SMX_THREADS, "one set member per thread in the last block");

// 64-bit selection key: the logit's order-preserving bit pattern above the
// complemented index, so keys are distinct and a larger key means a larger value,
// equal values ranking by ascending index.  NaN maps below every number and -0 onto
// +0.  A real key has bit 31 set (indices are below 2^31); 0 means "no item".
__device__ __forceinline__ uint64_t topk_key(float x, int j) {
  const uint32_t b = x == 0.f ? 0u : __float_as_uint(x);
  const uint32_t o = x != x ? 0u : ((b & 0x80000000u) ? ~b : (b | 0x80000000u));
  return ((uint64_t)o << 32) | (uint32_t)~(uint32_t)j;
}
__device__ __forceinline__ float topk_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int topk_index(uint64_t key) { return (int)~(uint32_t)key; }

struct SelShared {
  unsigned hist[TOPK_BINS];
  unsigned wtot[SMX_THREADS / 64];
  unsigned digit, need, exact;
};

// The k-th largest of the non-zero keys the block visits (exactly k of them are
// >= the result).  Needs more than k non-zero keys.  Most significant digit first,
// 11 bits at a time; a pass histograms the keys that share the digits fixed so far
// and fixes the digit whose bucket holds the k-th key.  It stops once that bucket
// holds exactly the keys still needed: all of them are selected, so the bucket's
// lowest key value (digits below zero) is a valid threshold.  With distinct keys
// this happens at the latest on the last digit.  visit(f) calls f(key) for every
// key of every thread; all threads call this function.
template <class Visit>
__device__ uint64_t select_kth(const Visit& visit, unsigned k, SelShared& s) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  constexpr int BPT = TOPK_BINS / SMX_THREADS;  // bins owned by a thread in the search
  uint64_t prefix = 0;
  unsigned need = k;
  int hi = 64;  // bits >= hi are fixed
  while (hi > 0) {
    const int bits = hi > 11 ? 11 : hi;
    const int shift = hi - bits;
    for (int b = t; b < TOPK_BINS; b += SMX_THREADS) s.hist[b] = 0u;
    __syncthreads();
    const uint64_t hmask = hi == 64 ? 0ull : ~0ull << hi;
    const unsigned dmask = (1u << bits) - 1u;
    visit([&](uint64_t key) {
      if (key != 0ull && (key & hmask) == prefix)
        atomicAdd(&s.hist[(unsigned)(key >> shift) & dmask], 1u);
    });
    __syncthreads();
    unsigned c[BPT], sum = 0;
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
      c[i] = s.hist[BPT * t + i];
      sum += c[i];
    }
    int incl = (int)sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    if (lane == 63) s.wtot[wave] = (unsigned)incl;
    __syncthreads();
    // keys in higher bins: the later lanes of this wave, then the later waves
    unsigned above = (unsigned)(__shfl(incl, 63, 64) - incl);
    for (int w = wave + 1; w < SMX_THREADS / 64; ++w) above += s.wtot[w];
    if (above < need && need <= above + sum) {  // exactly one thread
      for (int i = BPT - 1; i >= 0; --i) {
        if (above + c[i] >= need) {
          s.digit = (unsigned)(BPT * t + i);
          s.need = need - above;
          s.exact = c[i] == need - above;
          break;
        }
        above += c[i];
      }
    }
    __syncthreads();
    prefix |= (uint64_t)s.digit << shift;
    need = s.need;
    hi = shift;
    const bool done = s.exact != 0u;
    __syncthreads();  // s is reused by the next pass or the caller
    if (done) break;
  }
  return prefix;
}

__device__ __forceinline__ float block_sum_f32(float v, float* red) {
  v = wave_sum(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  v = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return v;
}

// exclusive prefix sum over the threads of the block, in thread order; *total gets the sum
__device__ __forceinline__ double block_excl_scan_f64(double v, double* red, double* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const double u = __shfl_up(incl, o, 64);
    if (lane >= o) incl += u;
  }
  if (lane == 63) red[wave] = incl;
  __syncthreads();
  double before = 0.0;
  for (int w = 0; w < wave; ++w) before += red[w];
  *total = (red[0] + red[1]) + (red[2] + red[3]);
  __syncthreads();
  return before + incl - v;
}

__global__ __launch_bounds__(SMX_THREADS) void topk_sample_kernel(
    const float* logits, float* probs, uint64_t* cand, unsigned* counters, const uint64_t* words,
    int V, int nchunks, int k, float T, float top_p, int32_t* token) {
  __shared__ SelShared s;
  __shared__ unsigned s_cnt;
  __shared__ uint64_t s_sel[TOPK_KMAX];   // the selected keys, in arrival order
  __shared__ uint64_t s_ord[TOPK_KMAX];   // ... in descending key order
  __shared__ int s_irank[TOPK_KMAX];      // index rank of s_ord[i]
  __shared__ uint64_t s_w[TOPK_KMAX];     // integer weights in ascending index order
  __shared__ int s_idx[TOPK_KMAX];        // vocabulary index in ascending index order
  __shared__ float s_rf[SMX_THREADS / 64];
  __shared__ double s_rd[SMX_THREADS / 64];
  __shared__ uint64_t s_ru[SMX_THREADS / 64];
  const int c = blockIdx.x, r = blockIdx.y, t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const int cs = k < SMX_CHUNK ? k : SMX_CHUNK;  // candidate slots per chunk
  const float* lr = logits + (size_t)r * V;
  float* pr = probs + (size_t)r * V;
  uint64_t* cr = cand + (size_t)r * nchunks * cs;
  const int base = c * SMX_CHUNK;
  const int n = min(SMX_CHUNK, V - base);
  constexpr int PER = SMX_CHUNK / SMX_THREADS;
  uint64_t key[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = base + t + SMX_THREADS * e;
    const float x = lr[j < V ? j : 0];
    key[e] = j < V ? topk_key(x, j) : 0ull;
  }
  uint64_t th = 1ull;  // every real key is >= 1
  if (n > k)
    th = select_kth(
        [&](auto f) {
#pragma unroll
          for (int e = 0; e < PER; ++e) f(key[e]);
        },
        (unsigned)k, s);
  if (t == 0) s_cnt = 0u;
  __syncthreads();
  const bool list_only = probs == nullptr;  // T = 0: the ordered top-k list, no probabilities
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    if (key[e] == 0ull) continue;
    if (key[e] >= th) {
      const unsigned slot = atomicAdd(&s_cnt, 1u);  // < min(k, n) <= cs
      if (slot < (unsigned)cs) st_coh_u64(cr + (size_t)c * cs + slot, key[e]);
    } else if (!list_only) {
      pr[base + t + SMX_THREADS * e] = 0.f;
    }
  }
  if (!arrive_last(counters + r, (unsigned)nchunks)) return;

  // ---- last block: the k largest of all candidates
  const int ncand = (nchunks - 1) * cs + min(k, V - (nchunks - 1) * SMX_CHUNK);
  int kk = min(k, V);
  auto visit_cand = [&](auto f) {
    for (int b0 = 0; b0 < ncand; b0 += SMX_THREADS * TOPK_BATCH) {
      uint64_t kv[TOPK_BATCH];
#pragma unroll
      for (int e = 0; e < TOPK_BATCH; ++e) {
        const int i = b0 + t + SMX_THREADS * e;
        const uint64_t v = ld_coh_u64(cr + (i < ncand ? i : 0));
        kv[e] = i < ncand ? v : 0ull;
      }
#pragma unroll
      for (int e = 0; e < TOPK_BATCH; ++e) f(kv[e]);
    }
  };
  uint64_t th2 = 1ull;
  if (ncand > kk) th2 = select_kth(visit_cand, (unsigned)kk, s);
  if (t == 0) s_cnt = 0u;
  __syncthreads();
  visit_cand([&](uint64_t key2) {
    if (key2 == 0ull) return;
    if (key2 >= th2) {
      const unsigned slot = atomicAdd(&s_cnt, 1u);  // exactly kk keys pass
      if (slot < (unsigned)TOPK_KMAX) s_sel[slot] = key2;
    } else if (!list_only && (unsigned)topk_index(key2) < (unsigned)V) {
      pr[topk_index(key2)] = 0.f;
    }
  });
  __syncthreads();
  kk = min(kk, (int)s_cnt);  // equal unless the candidates were inconsistent
  // ranks of each member by key (descending) and by index (ascending)
  if (t < kk) {
    const uint64_t mine = s_sel[t];
    const int mi = topk_index(mine);
    int rk = 0, ri = 0;
    for (int q = 0; q < kk; ++q) {
      const uint64_t o = s_sel[q];
      rk += o > mine;
      ri += topk_index(o) < mi;
    }
    s_ord[rk] = mine;
    s_irank[rk] = ri;
  }
  __syncthreads();
  if (list_only) {  // token[r][i] = i-th largest logit's index, -1 past the vocabulary
    if (t < k) token[(size_t)r * k + t] = t < kk ? topk_index(s_ord[t]) : -1;
    return;
  }
  // thread t < kk now owns the member of key rank t
  const bool member = t < kk;
  const uint64_t my = member ? s_ord[t] : 0ull;
  const float v = member ? topk_value(my) : 0.f;
  const float vmax = topk_value(s_ord[0]);
  bool keep = member;
  if (top_p > 0.f && top_p < 1.f) {
    // nucleus: keep the members whose preceding top-k mass (descending order) is below
    // top_p; the mass is taken in float64
    const double z0 = (double)vmax / (double)T;
    const double e64 = member ? exp((double)v / (double)T - z0) : 0.0;
    double S64, S2;
    block_excl_scan_f64(e64, s_rd, &S64);
    const double p64 = member ? e64 / S64 : 0.0;
    const double before = block_excl_scan_f64(p64, s_rd, &S2);
    keep = member && before < (double)top_p;
  }
  const float inv_t = 1.0f / T;
  const float e32 = keep ? expf((v - vmax) * inv_t) : 0.f;
  const float Z = block_sum_f32(e32, s_rf);
  const float p = keep ? e32 * (1.0f / Z) : 0.f;
  if (member) {
    const int ix = topk_index(my);
    if ((unsigned)ix < (unsigned)V) st_coh(pr + ix, p);
    s_w[s_irank[t]] = prob_weight(p);
    s_idx[s_irank[t]] = ix;
  }
  __syncthreads();
  // inverse CDF in ascending index order
  const uint64_t w = member ? s_w[t] : 0ull;
  const uint64_t winc = wave_scan_u64(w);
  if (lane == 63) s_ru[wave] = winc;
  __syncthreads();
  uint64_t before = 0;
  for (int q = 0; q < wave; ++q) before += s_ru[q];
  const uint64_t Sw = (s_ru[0] + s_ru[1]) + (s_ru[2] + s_ru[3]);
  const uint64_t tau = scale_u32((uint32_t)(words[r] >> 32), Sw);
  const uint64_t lo = before + winc - w;
  if (Sw == 0ull) {
    if (t == 0) token[r] = 0;
  } else if (member && lo <= tau && tau < lo + w) {
    token[r] = s_idx[t];
  }
}

struct LmPlan {
  bool dot;
  int J;
  GemmPlan gp;
  int nstat, nchunks;
  size_t off_part, off_stat, off_gstat, off_csum, off_cand, total;
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
  p.off_gstat = take((size_t)rows * sizeof(BlockStat));
  p.off_csum = take((size_t)rows * p.nchunks * 8);
  p.off_cand = take(c->top_k > 0 ? (size_t)rows * p.nchunks * std::min(c->top_k, SMX_CHUNK) * 8 : 0);
  p.total = off;
  return p;
}

size_t lm_head_workspace(const spd_config* cfg, int rows) { return plan_lm(cfg, rows).total; }

// A capped GEMV streams beside latency-bound work on another stream: each wave
// keeps one row's loads in flight instead of eight, so the memory queues that the
// other work's dependent loads wait in stay short (measured on the headline cycle:
// 1.1% more cycles/s than eight rows in flight, at any cap from 192 to 320).
constexpr int DOT_ROWS_CAPPED = 1;

template <int J>
static void launch_dot(int nblk, bool capped, hipStream_t st, const void* w, const float* h, int V,
                       float inv_t, float* logits, BlockStat* stat) {
  if (capped)
    hipLaunchKernelGGL((lmh_dot_kernel<J, DOT_ROWS_CAPPED>), dim3(nblk), dim3(256), 0, st,
                       static_cast<const bf16*>(w), h, V, inv_t, logits, stat);
  else
    hipLaunchKernelGGL((lmh_dot_kernel<J, DOT_ROWS>), dim3(nblk), dim3(256), 0, st,
                       static_cast<const bf16*>(w), h, V, inv_t, logits, stat);
}

template <typename WT>
static int lm_impl(const spd_config* c, const void* w_lm, const float* h, int rows, float T,
                   const uint64_t* words, float* logits, float* probs, int32_t* token, void* ws,
                   hipStream_t st) {
  const LmPlan p = plan_lm(c, rows);
  char* w = static_cast<char*>(ws);
  BlockStat* stat = reinterpret_cast<BlockStat*>(w + p.off_stat);
  unsigned* ctr = reinterpret_cast<unsigned*>(w);
  const float inv_t = T > 0.f ? 1.0f / T : 0.f;
  const bool topk_list = T <= 0.f && c->top_k >= 2;  // greedy draft-tree children
  const HeadFinish f{ctr + CTR_HEAD, reinterpret_cast<BlockStat*>(w + p.off_gstat), token,
                     (T > 0.f || topk_list) ? 0 : 1};
  int rc;
  if (p.dot) {
    const int nblk = c->head_workgroups > 0 ? std::min(p.nstat, c->head_workgroups) : p.nstat;
    switch (p.J) {
      case 1: launch_dot<1>(nblk, c->head_workgroups > 0, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 2: launch_dot<2>(nblk, c->head_workgroups > 0, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 3: launch_dot<3>(nblk, c->head_workgroups > 0, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 4: launch_dot<4>(nblk, c->head_workgroups > 0, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 5: launch_dot<5>(nblk, c->head_workgroups > 0, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 6: launch_dot<6>(nblk, c->head_workgroups > 0, st, w_lm, h, c->V, inv_t, logits, stat); break;
      case 7: launch_dot<7>(nblk, c->head_workgroups > 0, st, w_lm, h, c->V, inv_t, logits, stat); break;
      default: launch_dot<8>(nblk, c->head_workgroups > 0, st, w_lm, h, c->V, inv_t, logits, stat); break;
    }
    rc = check_launch();
    if (rc) return rc;
    if (T <= 0.f && !topk_list) {
      hipLaunchKernelGGL(greedy_kernel, dim3(rows), dim3(SMX_THREADS), 0, st, stat, p.nstat, rows, token);
      return check_launch();
    }
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
    g.counters = ctr;
    EpiLogits epi{logits, stat, c->V, rows, inv_t, p.gp.nblocks, f};
    rc = launch_gemm<WT, 2>(p.gp, g, InAct<WT, float>{h, c->d}, epi, RowMapStd{}, st);
    if (rc || (T <= 0.f && !topk_list)) return rc;
  }
  if (c->top_k > 0) {
    hipLaunchKernelGGL(topk_sample_kernel, dim3(p.nchunks, rows), dim3(SMX_THREADS), 0, st, logits,
                       topk_list ? nullptr : probs, reinterpret_cast<uint64_t*>(w + p.off_cand),
                       ctr + CTR_HEAD + 512, words, c->V, p.nchunks, c->top_k, T, c->top_p, token);
    return check_launch();
  }
  hipLaunchKernelGGL(softmax_sample_kernel, dim3(p.nchunks, rows), dim3(SMX_THREADS), 0, st, stat,
                     p.dot ? p.nstat : 0, rows, f.gstat, logits, probs,
                     reinterpret_cast<uint64_t*>(w + p.off_csum), ctr + CTR_HEAD + 512, words, c->V,
                     p.nchunks, inv_t, token);
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
  // the nucleus is cut among the top-k candidates; over the whole vocabulary it
  // would need a vocabulary-wide ordering, which this library does not offer
  if (temperature > 0.f && cfg->top_k == 0 && cfg->top_p > 0.f && cfg->top_p < 1.f)
    return SPD_E_UNSUPPORTED;
  if (cfg->d % 64) return SPD_E_UNSUPPORTED;
  if ((int64_t)cfg->V * cfg->d > ((int64_t)1 << 40)) return SPD_E_UNSUPPORTED;
  if (temperature > 0.f && cfg->V > SMX_MAXCH * SMX_CHUNK) return SPD_E_UNSUPPORTED;
  if (!aligned16(w_lm) || !aligned16(h) || !aligned16(ws)) return SPD_E_INVALID;
  if (ws_bytes < lm_head_workspace(cfg, rows)) return SPD_E_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cfg->dtype == SPD_BF16)
    return lm_impl<bf16>(cfg, w_lm, h, rows, temperature, words, logits, probs, token, ws, st);
  return lm_impl<float>(cfg, w_lm, h, rows, temperature, words, logits, probs, token, ws, st);
}

// ---------------------------------------------------------------------------
// spd_lm_head_noalloc: spd_lm_head with its workspace in a file-scope device array
// instead of a caller buffer.  Each GPU the library runs on holds its own copy of
// the array (allocated with the code object, held until the process ends); host
// code never passes the array's name to a kernel (in host code it is only a
// stand-in), but the device address hipGetSymbolAddress returns for the GPU.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)SPD_NOALLOC_SCRATCH_BYTES;
constexpr int NOALLOC_MAX_DEVICES = 64;

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

__global__ void zero_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

std::mutex g_scratch_mu;
void* g_scratch_ptr[NOALLOC_MAX_DEVICES];

// Device address of `scratch` on the stream's GPU.  The first call on a GPU looks
// it up with that GPU current and clears the arrival counters (a fill kernel on
// the caller's stream, not a memset); later calls reuse the address.
int scratch_of(hipStream_t st, void** out) {
  int dev = -1;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) {
    last_hip_error_ref() = (int)e;
    return SPD_E_HIP;
  }
  if (dev < 0 || dev >= NOALLOC_MAX_DEVICES) return SPD_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e == hipSuccess && !ptr) e = hipErrorInvalidSymbol;
    if (e == hipSuccess) {
      hipLaunchKernelGGL(zero_words_kernel, dim3(16), dim3(256), 0, st, static_cast<uint32_t*>(ptr),
                         (int)(SPD_WS_COUNTER_BYTES / 4));
      e = hipGetLastError();
    }
    if (cur >= 0 && cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) {
      last_hip_error_ref() = (int)e;
      return SPD_E_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SPD_OK;
}

}  // namespace

extern "C" int spd_lm_head_noalloc(const spd_config* cfg, const void* w_lm, const float* h,
                                   int32_t rows, float temperature, const uint64_t* words,
                                   float* logits, float* probs, int32_t* token, void* stream) {
  // the same argument checks as spd_lm_head, then the scratch size
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!w_lm || !h || !logits || !token) return SPD_E_INVALID;
  if (rows < 1 || rows > 16) return SPD_E_INVALID;
  if (lm_head_workspace(cfg, rows) > NOALLOC_SCRATCH_BYTES) return SPD_E_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  rc = scratch_of(st, &ws);
  if (rc) return rc;
  return spd_lm_head(cfg, w_lm, h, rows, temperature, words, logits, probs, token, ws,
                     NOALLOC_SCRATCH_BYTES, stream);
}
