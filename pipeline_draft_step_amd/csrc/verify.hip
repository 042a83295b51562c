// spd_verify: speculative-sampling verification of drafted tokens.
// ("Speculative Pipeline Decoding", arXiv 2605.30852, section 3.4: streaming
// verification, greedy argmax match at T = 0, standard rejection sampling at T > 0;
// the speculative-decoding explainer's four-phase loop and acceptance criterion:
// accept if r <= min(1, p/q), else resample from norm(max(0, p - q)); bonus token
// from p_{gamma+1} when every draft is accepted.)
//
// T > 0, launch 1, grid (vocabulary chunks, sequences): every block decides the
//   sequence's outcome from the 2*gamma scalars p_j(x_j), q_j(x_j) (cheap, exact;
//   one lane per draft), so a fully accepted sequence without bonus reads no rows;
//   otherwise it sums the exact integer weights of its chunk of the row to sample
//   from (residual and target weights both, for the empty-residual fallback).
//   Launch 2, one block per sequence: the same decision, the chunk scan and the
//   search inside the chosen chunk.
// T == 0, launch 1: per chunk (max, first argmax) of every row; launch 2: merge
//   per row and compare with the drafts.
#include <algorithm>

#include "spd_common.h"
#include "spd_host.h"

namespace spd {

constexpr int VER_CHUNK = 2048;
constexpr int VER_THREADS = 256;
constexpr int VER_MAX_ROWS = 64;  // gamma + bonus limit

struct VerArgs {
  const float* p;
  const float* q;
  const int32_t* draft;
  const uint64_t* words;
  int32_t* n_accept;
  int32_t* next_token;
  void* part;
  int32_t* jrej;  // [B] first rejected position (T > 0: the sums pass leaves it for the draw)
  int B, gamma, V, bonus, nchunks;
  int W;  // sibling candidates per sequence (greedy sibling verification)
};

__device__ uint64_t vblock_scan(uint64_t v, uint64_t* sh) {
  sh[threadIdx.x] = v;
  __syncthreads();
  for (int o = 1; o < VER_THREADS; o <<= 1) {
    const uint64_t add = (int)threadIdx.x >= o ? sh[threadIdx.x - o] : 0ull;
    __syncthreads();
    sh[threadIdx.x] += add;
    __syncthreads();
  }
  const uint64_t r = sh[threadIdx.x];
  __syncthreads();
  return r;
}

__device__ __forceinline__ uint64_t res_weight(float p, float q) {
  const uint64_t P = prob_weight(p), Q = prob_weight(q);
  return P > Q ? P - Q : 0ull;
}

// First rejected position of sequence b (gamma if all accepted).  Lane j of wave 0
// tests draft j (gamma <= 63), all loads issued at once; the lowest rejecting lane
// wins, which is the position a sequential scan would stop at.  Called by every
// thread of the block; every thread gets the result.
__device__ int first_reject(const VerArgs& a, int b) {
  __shared__ int s_first;
  if (threadIdx.x < WAVE) {
    const int j = threadIdx.x;
    bool acc = true;  // lanes past gamma never reject
    if (j < a.gamma) {
      const int rowsP = a.gamma + a.bonus;
      const int x = a.draft[b * a.gamma + j];
      const uint64_t R = a.words[((size_t)b * (a.gamma + 1) + j) * 2] >> 40;
      acc = false;
      if (x >= 0 && x < a.V) {
        const double px = (double)a.p[((size_t)b * rowsP + j) * a.V + x];
        const double qx = (double)a.q[((size_t)b * a.gamma + j) * a.V + x];
        acc = (double)(R + 1) * qx <= px * 16777216.0;
      }
    }
    const uint64_t rej = __ballot(!acc);
    if (threadIdx.x == 0) s_first = rej ? (int)__builtin_ctzll(rej) : a.gamma;
  }
  __syncthreads();
  const int j = s_first;
  __syncthreads();  // s_first is rewritten by the next call
  return j;
}

// Sums of the exact integer weights (residual, target) of chunk c of the rows that
// sequence b samples from, once its decision j is known; thread 0 of the block gets
// them.  pv / qv hold the chunk's probabilities (8 per thread).
template <int PER>
__device__ void chunk_weight_sums(const float (&pv)[PER], const float (&qv)[PER], bool rejected,
                                  uint64_t& tres, uint64_t& tp) {
  __shared__ uint64_t s_w[2][VER_THREADS / 64];
  uint64_t sres = 0, sp = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    sp += prob_weight(pv[e]);
    if (rejected) sres += res_weight(pv[e], qv[e]);
  }
  sres = wave_sum_u64(sres);
  sp = wave_sum_u64(sp);
  if ((threadIdx.x & 63) == 0) {
    s_w[0][threadIdx.x >> 6] = sres;
    s_w[1][threadIdx.x >> 6] = sp;
  }
  __syncthreads();
  tres = 0;
  tp = 0;
  for (int w = 0; w < VER_THREADS / 64; ++w) {
    tres += s_w[0][w];
    tp += s_w[1][w];
  }
  __syncthreads();  // s_w is rewritten by the next call
}

// The draw of sequence b once every chunk's weight sums (residual, target) are in
// pb[2 c], pb[2 c + 1]: the residual if it has mass, else the target row; the
// chunk scan, then the search inside the chosen chunk.  Writes n_accept / next_token.
__device__ void locate_and_write(const VerArgs& a, int b, int j, const uint64_t* pb) {
  __shared__ uint64_t sh[VER_THREADS];
  __shared__ uint64_t s_tau, s_off;
  __shared__ int s_chunk, s_found;
  __shared__ uint64_t s_t[VER_THREADS / 64];
  auto ld = [&](int i) { return pb[i]; };
  const bool rejected = j < a.gamma;
  const int rowsP = a.gamma + a.bonus;
  const float* prow = a.p + ((size_t)b * rowsP + j) * a.V;
  const float* qrow = rejected ? a.q + ((size_t)b * a.gamma + j) * a.V : nullptr;
  // residual if it has mass, else the target row itself
  uint64_t tr = 0;
  for (int k = threadIdx.x; k < a.nchunks; k += VER_THREADS) tr += ld(2 * k);
  tr = wave_sum_u64(tr);
  if ((threadIdx.x & 63) == 0) s_t[threadIdx.x >> 6] = tr;
  __syncthreads();
  uint64_t total_res = 0;
  for (int w = 0; w < VER_THREADS / 64; ++w) total_res += s_t[w];
  const int which = (rejected && total_res > 0) ? 0 : 1;
  const uint64_t U = a.words[((size_t)b * (a.gamma + 1) + j) * 2 + 1] >> 32;

  const int per = (a.nchunks + VER_THREADS - 1) / VER_THREADS;
  uint64_t mine = 0;
  for (int e = 0; e < per; ++e) {
    const int k = threadIdx.x * per + e;
    if (k < a.nchunks) mine += ld(2 * k + which);
  }
  const uint64_t incl = vblock_scan(mine, sh);
  if (threadIdx.x == VER_THREADS - 1) {
    s_tau = scale_u32((uint32_t)U, incl);
    s_chunk = -1;
    s_found = -1;
  }
  __syncthreads();
  const uint64_t tau = s_tau;
  uint64_t run = incl - mine;
  if (run <= tau && incl > tau) {
    for (int e = 0; e < per; ++e) {
      const int k = threadIdx.x * per + e;
      if (k >= a.nchunks) break;
      const uint64_t w = ld(2 * k + which);
      if (run + w > tau) {
        s_chunk = k;
        s_off = run;
        break;
      }
      run += w;
    }
  }
  __syncthreads();
  if (s_chunk >= 0) {
    constexpr int PER = VER_CHUNK / VER_THREADS;
    const int b0 = s_chunk * VER_CHUNK;
    uint64_t w[PER];
    uint64_t tot = 0;
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int i = b0 + threadIdx.x * PER + e;
      uint64_t v = 0;
      if (i < a.V) v = which == 0 ? res_weight(prow[i], qrow[i]) : prob_weight(prow[i]);
      w[e] = v;
      tot += v;
    }
    const uint64_t in2 = vblock_scan(tot, sh);
    uint64_t r2 = s_off + in2 - tot;
    if (r2 <= tau && s_off + in2 > tau) {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        r2 += w[e];
        if (r2 > tau) {
          s_found = b0 + threadIdx.x * PER + e;
          break;
        }
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    a.n_accept[b] = j;
    a.next_token[b] = s_found < 0 ? 0 : s_found;
  }
}

// T > 0, launch 1: the chunk sums of every (chunk, sequence); launch 2: one block
// per sequence draws.  (One launch, with the last chunk block of each sequence
// drawing, was measured slower: 30.5 against 25 us for 64 x 7 sequences.)
__global__ __launch_bounds__(VER_THREADS) void verify_sums_kernel(VerArgs a) {
  const int c = blockIdx.x, b = blockIdx.y;
  const int j = first_reject(a, b);
  if (c == 0 && threadIdx.x == 0) a.jrej[b] = j;
  const bool rejected = j < a.gamma;
  if (!rejected && !a.bonus) return;
  const int rowsP = a.gamma + a.bonus;
  const float* prow = a.p + ((size_t)b * rowsP + j) * a.V;
  const float* qrow = rejected ? a.q + ((size_t)b * a.gamma + j) * a.V : nullptr;
  constexpr int PER = VER_CHUNK / VER_THREADS;
  float pv[PER], qv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int i = c * VER_CHUNK + threadIdx.x + VER_THREADS * e;
    pv[e] = i < a.V ? prow[i] : 0.f;
    qv[e] = (rejected && i < a.V) ? qrow[i] : 0.f;
  }
  uint64_t tres, tp;
  chunk_weight_sums(pv, qv, rejected, tres, tp);
  if (threadIdx.x == 0) {
    uint64_t* part = static_cast<uint64_t*>(a.part) + ((size_t)b * a.nchunks + c) * 2;
    part[0] = tres;
    part[1] = tp;
  }
}

// (the decision of sequence b comes from the sums pass: one load instead of the
// draft and probability loads one after the other)
__global__ __launch_bounds__(VER_THREADS) void verify_locate_kernel(VerArgs a) {
  const int b = blockIdx.x;
  const int j = a.jrej[b];
  if (j == a.gamma && !a.bonus) {
    if (threadIdx.x == 0) {
      a.n_accept[b] = a.gamma;
      a.next_token[b] = -1;
    }
    return;
  }
  locate_and_write(a, b, j, static_cast<const uint64_t*>(a.part) + (size_t)b * a.nchunks * 2);
}

__global__ __launch_bounds__(VER_THREADS) void verify_greedy_chunks_kernel(VerArgs a) {
  const int c = blockIdx.x, b = blockIdx.y;
  const int rows = a.gamma + a.bonus;
  const int end = min((c + 1) * VER_CHUNK, a.V);
  ArgMax* part = static_cast<ArgMax*>(a.part);
  __shared__ ArgMax s_am[VER_THREADS / 64];
  for (int j = 0; j < rows; ++j) {
    const float* prow = a.p + ((size_t)b * rows + j) * a.V;
    ArgMax am{-INFINITY, ARG_NONE};
#pragma unroll 8
    for (int i = c * VER_CHUNK + threadIdx.x; i < end; i += VER_THREADS) am = argmax_merge(am, ArgMax{prow[i], i});
    am = wave_argmax(am);
    if ((threadIdx.x & 63) == 0) s_am[threadIdx.x >> 6] = am;
    __syncthreads();
    if (threadIdx.x == 0) {
      ArgMax t = s_am[0];
      for (int w = 1; w < VER_THREADS / 64; ++w) t = argmax_merge(t, s_am[w]);
      part[((size_t)b * rows + j) * a.nchunks + c] = t;
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(VER_THREADS) void verify_greedy_final_kernel(VerArgs a) {
  const int b = blockIdx.x;
  const int rows = a.gamma + a.bonus;
  const ArgMax* part = static_cast<const ArgMax*>(a.part);
  __shared__ ArgMax s_am[VER_THREADS / 64];
  __shared__ int s_best[VER_MAX_ROWS];
  for (int j = 0; j < rows; ++j) {
    const ArgMax* pj = part + ((size_t)b * rows + j) * a.nchunks;
    ArgMax am{-INFINITY, ARG_NONE};
    for (int k = threadIdx.x; k < a.nchunks; k += VER_THREADS) am = argmax_merge(am, pj[k]);
    am = wave_argmax(am);
    if ((threadIdx.x & 63) == 0) s_am[threadIdx.x >> 6] = am;
    __syncthreads();
    if (threadIdx.x == 0) {
      ArgMax t = s_am[0];
      for (int w = 1; w < VER_THREADS / 64; ++w) t = argmax_merge(t, s_am[w]);
      s_best[j] = t.i == ARG_NONE ? 0 : t.i;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    int j = 0;
    while (j < a.gamma && a.draft[b * a.gamma + j] == s_best[j]) ++j;
    a.n_accept[b] = j;
    a.next_token[b] = j < a.gamma ? s_best[j] : (a.bonus ? s_best[a.gamma] : -1);
  }
}

// Greedy verification of W sibling candidates of one position per sequence (a draft
// tree's oldest level): draft[b][i], i < W, is accepted when it equals the target
// argmax of row b; the first such i is reported.  Row argmax from the chunk pass.
__global__ __launch_bounds__(VER_THREADS) void verify_siblings_final_kernel(VerArgs a) {
  const int b = blockIdx.x;
  const ArgMax* pj = static_cast<const ArgMax*>(a.part) + (size_t)b * a.nchunks;
  __shared__ ArgMax s_am[VER_THREADS / 64];
  ArgMax am{-INFINITY, ARG_NONE};
  for (int k = threadIdx.x; k < a.nchunks; k += VER_THREADS) am = argmax_merge(am, pj[k]);
  am = wave_argmax(am);
  if ((threadIdx.x & 63) == 0) s_am[threadIdx.x >> 6] = am;
  __syncthreads();
  if (threadIdx.x == 0) {
    ArgMax t = s_am[0];
    for (int w = 1; w < VER_THREADS / 64; ++w) t = argmax_merge(t, s_am[w]);
    const int best = t.i == ARG_NONE ? 0 : t.i;
    int acc = -1;
    for (int i = 0; i < a.W && acc < 0; ++i)
      if (a.draft[(size_t)b * a.W + i] == best) acc = i;
    a.n_accept[b] = acc;
    a.next_token[b] = acc < 0 ? best : -1;
  }
}

// Stochastic verification of W sibling candidates drawn independently from q
// (multi-round rejection: each rejection makes the normalised residual max(0, p_i - q)
// the next round's target; after W rejections the token is drawn from the last
// residual).  Exact integer form: A = floor(p 2^51), B = floor(q 2^51); round i
// accepts x_i iff (R_i + 1) B(x_i) sum(A) <= 2^24 A(x_i) sum(B); on rejection
// A <- max(0, A sum(B) - B sum(A)) >> s with s = max(0, bitlength(sum) - 52), which keeps
// sum(A) < 2^52 and every product below 2^128.  A row's round-i weight is recomputed
// from (p_j, q_j) and the per-round scalars, so nothing but scalars is stored.
// One block per sequence.
constexpr int SIB_THREADS = 1024;
constexpr int SIB_WAVES = SIB_THREADS / 64;
typedef unsigned __int128 u128;

__device__ __forceinline__ uint64_t sib_weight(float p) {  // floor(p * 2^51), 0 unless p > 0
  return (p > 0.f) ? (uint64_t)((double)p * 2251799813685248.0) : 0ull;
}
__device__ __forceinline__ u128 sib_resid(uint64_t a, uint64_t b, uint64_t SA, uint64_t SB) {
  const u128 x = (u128)a * SB, y = (u128)b * SA;
  return x > y ? x - y : (u128)0;
}
// round-`rounds` weight of an entry with first-round weights (a, b)
__device__ __forceinline__ uint64_t sib_chain(uint64_t a, uint64_t b, int rounds, const uint64_t* hSA,
                                              const int* hS, uint64_t SB) {
  for (int k = 0; k < rounds; ++k) a = (uint64_t)(sib_resid(a, b, hSA[k], SB) >> hS[k]);
  return a;
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m, 64), hi = __shfl_xor((uint32_t)(v >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
// block sum of a 128-bit value (exact, any order); every thread gets the result
__device__ u128 sib_block_sum(u128 v, u128* red) {
  uint64_t lo = (uint64_t)v, hi = (uint64_t)(v >> 64);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint64_t olo = shfl_xor_u64(lo, m), ohi = shfl_xor_u64(hi, m);
    const uint64_t nlo = lo + olo;
    hi = hi + ohi + (nlo < lo ? 1ull : 0ull);
    lo = nlo;
  }
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = ((u128)hi << 64) | lo;
  __syncthreads();
  u128 t = 0;
  for (int w = 0; w < SIB_WAVES; ++w) t += red[w];
  __syncthreads();
  return t;
}

__global__ __launch_bounds__(SIB_THREADS) void verify_siblings_sampled_kernel(VerArgs a) {
  __shared__ u128 s_red[SIB_WAVES];
  __shared__ uint64_t s_hSA[SPD_TREE_MAX_NODES];
  __shared__ int s_hS[SPD_TREE_MAX_NODES];
  __shared__ int s_acc;
  __shared__ uint64_t s_wt[SIB_WAVES];
  __shared__ int s_tok;
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const float* prow = a.p + (size_t)b * a.V;
  const float* qrow = a.q + (size_t)b * a.V;
  const uint64_t* wd = a.words + (size_t)b * (a.W + 1) * 2;
  u128 sa = 0, sb = 0;
  for (int j = t; j < a.V; j += SIB_THREADS) {
    sa += sib_weight(prow[j]);
    sb += sib_weight(qrow[j]);
  }
  const uint64_t SA0 = (uint64_t)sib_block_sum(sa, s_red);
  const uint64_t SB = (uint64_t)sib_block_sum(sb, s_red);
  uint64_t SA = SA0;
  for (int i = 0; i < a.W; ++i) {
    if (t == 0) {
      const int x = a.draft[(size_t)b * a.W + i];
      int acc = 0;
      if (x >= 0 && x < a.V) {
        const uint64_t bx = sib_weight(qrow[x]);
        const uint64_t ax = sib_chain(sib_weight(prow[x]), bx, i, s_hSA, s_hS, SB);
        const uint64_t R1 = (wd[2 * i] >> 40) + 1;
        acc = (u128)R1 * bx * SA <= ((u128)ax * SB) << 24;
      }
      s_acc = acc;
      s_hSA[i] = SA;
    }
    __syncthreads();
    if (s_acc) {
      if (t == 0) {
        a.n_accept[b] = i;
        a.next_token[b] = -1;
      }
      return;
    }
    // residual of round i: its 128-bit total fixes the shift, then the new total
    u128 dsum = 0;
    for (int j = t; j < a.V; j += SIB_THREADS) {
      const uint64_t bj = sib_weight(qrow[j]);
      const uint64_t aj = sib_chain(sib_weight(prow[j]), bj, i, s_hSA, s_hS, SB);
      dsum += sib_resid(aj, bj, SA, SB);
    }
    const u128 D = sib_block_sum(dsum, s_red);
    const uint64_t dhi = (uint64_t)(D >> 64), dlo = (uint64_t)D;
    const int bits = dhi ? 128 - __builtin_clzll(dhi) : (dlo ? 64 - __builtin_clzll(dlo) : 0);
    if (t == 0) s_hS[i] = bits > 52 ? bits - 52 : 0;
    __syncthreads();
    u128 asum = 0;
    for (int j = t; j < a.V; j += SIB_THREADS)
      asum += sib_chain(sib_weight(prow[j]), sib_weight(qrow[j]), i + 1, s_hSA, s_hS, SB);
    SA = (uint64_t)sib_block_sum(asum, s_red);
  }
  // every candidate rejected: inverse-CDF draw from the last residual (from p if empty)
  const int rounds = SA > 0 ? a.W : 0;
  const uint64_t S = SA > 0 ? SA : SA0;
  const uint64_t tau = scale_u32((uint32_t)(wd[2 * a.W + 1] >> 32), S);
  if (t == 0) s_tok = -1;
  uint64_t before = 0;
  for (int base = 0; base < a.V; base += SIB_THREADS) {
    const int j = base + t;
    const uint64_t w = j < a.V ? sib_chain(sib_weight(prow[j]), sib_weight(qrow[j]), rounds, s_hSA, s_hS, SB)
                               : 0ull;
    uint64_t incl = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t lo = __shfl_up((uint32_t)incl, o, 64), hi = __shfl_up((uint32_t)(incl >> 32), o, 64);
      if (lane >= o) incl += ((uint64_t)hi << 32) | lo;
    }
    if (lane == 63) s_wt[wave] = incl;
    __syncthreads();
    uint64_t off = before, tile = 0;
    for (int w2 = 0; w2 < SIB_WAVES; ++w2) {
      if (w2 < wave) off += s_wt[w2];
      tile += s_wt[w2];
    }
    if (w > 0 && off + incl - w <= tau && tau < off + incl) s_tok = j;
    __syncthreads();
    if (s_tok >= 0) break;
    before += tile;
  }
  if (t == 0) {
    a.n_accept[b] = -1;
    a.next_token[b] = s_tok >= 0 ? s_tok : 0;
  }
}

// ---------------------------------------------------------------------------
// The same verification spread over many blocks per sequence, for small batches
// (one block per sequence would leave the GPU idle).  Each pass over the
// vocabulary is one launch over (chunk of SIB_CHUNK entries, sequence); the last
// block of a sequence to arrive adds the chunk partials in chunk order (exact
// integer sums, so the order does not change them) and does the pass's scalar
// work: the totals and the first accept test, a round's shift, or the round's new
// total with the next accept test -- after the last round, the final draw, whose
// chunk totals are the partials it has just added.  A sequence that has finished
// makes the later launches return at once.  The decisions are the single-block
// kernel's, bit for bit.
constexpr int SIB_CHUNK = 1024;
constexpr int SIB_MB_THREADS = 256;
constexpr int SIB_PER = SIB_CHUNK / SIB_MB_THREADS;  // entries per thread (contiguous)
constexpr int SIB_MULTI_MAX_B = 64;  // batches below this use the multi-block form

struct SibState {
  uint64_t SA0, SB;
  uint64_t hSA[SPD_TREE_MAX_NODES + 1];  // total of round i's target weights
  int32_t hS[SPD_TREE_MAX_NODES];        // shift applied after round i
  int32_t done;                          // 1: accepted[b] / next_token[b] are final
  int32_t pad;
};
enum { SIB_PASS_TOT = 0, SIB_PASS_D = 1, SIB_PASS_A = 2 };

inline size_t sib_state_bytes(int B) { return align256((size_t)B * sizeof(SibState)); }
inline size_t sib_part_bytes(int B, int V) {
  const size_t nch = (size_t)(V + SIB_CHUNK - 1) / SIB_CHUNK;
  return (size_t)B * 4 * nch * 16;  // sa, sb, d, a partials (128-bit) per chunk
}

__device__ u128 sib_block_sum256(u128 v, u128* red) {
  uint64_t lo = (uint64_t)v, hi = (uint64_t)(v >> 64);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const uint64_t olo = shfl_xor_u64(lo, m), ohi = shfl_xor_u64(hi, m);
    const uint64_t nlo = lo + olo;
    hi = hi + ohi + (nlo < lo ? 1ull : 0ull);
    lo = nlo;
  }
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ((u128)hi << 64) | lo;
  __syncthreads();
  u128 t = 0;
  for (int w = 0; w < SIB_MB_THREADS / 64; ++w) t += red[w];
  __syncthreads();
  return t;
}

__device__ __forceinline__ void st_coh_u128(u128* p, u128 v) {
  uint64_t* q = reinterpret_cast<uint64_t*>(p);
  st_coh_u64(q, (uint64_t)v);
  st_coh_u64(q + 1, (uint64_t)(v >> 64));
}
__device__ __forceinline__ u128 ld_coh_u128(const u128* p) {
  const uint64_t* q = reinterpret_cast<const uint64_t*>(p);
  return ((u128)ld_coh_u64(q + 1) << 64) | ld_coh_u64(q);
}

struct SibMulti {
  SibState* st;      // [B]
  u128* part;        // [B][4][nch]
  unsigned* counters;  // [B]
  int nch;
};

// accept test of candidate i against round i's target (weights after i rounds)
__device__ bool sib_accept(const VerArgs& a, const SibState& s, const uint64_t* hSA, const int* hS, int b, int i) {
  const float* prow = a.p + (size_t)b * a.V;
  const float* qrow = a.q + (size_t)b * a.V;
  const uint64_t* wd = a.words + (size_t)b * (a.W + 1) * 2;
  const int x = a.draft[(size_t)b * a.W + i];
  if (x < 0 || x >= a.V) return false;
  const uint64_t bx = sib_weight(qrow[x]);
  const uint64_t ax = sib_chain(sib_weight(prow[x]), bx, i, hSA, hS, s.SB);
  const uint64_t R1 = (wd[2 * i] >> 40) + 1;
  return (u128)R1 * bx * hSA[i] <= ((u128)ax * s.SB) << 24;
}

__global__ __launch_bounds__(SIB_MB_THREADS) void sib_pass_kernel(VerArgs a, SibMulti m, int pass, int round) {
  __shared__ u128 s_red[SIB_MB_THREADS / 64];
  __shared__ uint64_t s_hSA[SPD_TREE_MAX_NODES + 1];
  __shared__ int s_hS[SPD_TREE_MAX_NODES];
  __shared__ uint64_t s_scan[SIB_MB_THREADS];
  __shared__ int s_tok;
  const int c = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  SibState* st = m.st + b;
  if (pass != SIB_PASS_TOT && st->done) return;  // written by an earlier launch
  const uint64_t SB = pass == SIB_PASS_TOT ? 0ull : st->SB;
  if (pass != SIB_PASS_TOT) {
    for (int k = t; k <= round + 1 && k <= a.W; k += SIB_MB_THREADS) s_hSA[k] = st->hSA[k];
    for (int k = t; k <= round && k < a.W; k += SIB_MB_THREADS) s_hS[k] = st->hS[k];
  }
  __syncthreads();
  const float* prow = a.p + (size_t)b * a.V;
  const float* qrow = a.q + (size_t)b * a.V;
  const int j0 = c * SIB_CHUNK + t * SIB_PER;
  u128 v0 = 0, v1 = 0;
#pragma unroll
  for (int e = 0; e < SIB_PER; ++e) {
    const int j = j0 + e;
    if (j >= a.V) break;
    const uint64_t aj = sib_weight(prow[j]), bj = sib_weight(qrow[j]);
    if (pass == SIB_PASS_TOT) {
      v0 += aj;
      v1 += bj;
    } else if (pass == SIB_PASS_D) {
      v0 += sib_resid(sib_chain(aj, bj, round, s_hSA, s_hS, SB), bj, s_hSA[round], SB);
    } else {
      v0 += sib_chain(aj, bj, round + 1, s_hSA, s_hS, SB);
    }
  }
  u128* part = m.part + (size_t)b * 4 * m.nch;
  const u128 t0 = sib_block_sum256(v0, s_red);
  const u128 t1 = pass == SIB_PASS_TOT ? sib_block_sum256(v1, s_red) : (u128)0;
  if (t == 0) {
    if (pass == SIB_PASS_TOT) {
      st_coh_u128(part + c, t0);
      st_coh_u128(part + m.nch + c, t1);
    } else {
      st_coh_u128(part + (size_t)(pass == SIB_PASS_D ? 2 : 3) * m.nch + c, t0);
    }
  }
  if (!arrive_last(m.counters + b, (unsigned)m.nch)) return;
  // last block of this sequence: the pass's scalar work, starting with the sum of
  // the chunk partials (every thread loads its share)
  u128 X, Y = 0;
  {
    u128 x = 0, y = 0;
    const u128* src = part + (size_t)(pass == SIB_PASS_TOT ? 0 : (pass == SIB_PASS_D ? 2 : 3)) * m.nch;
    for (int k = t; k < m.nch; k += SIB_MB_THREADS) {
      x += ld_coh_u128(src + k);
      if (pass == SIB_PASS_TOT) y += ld_coh_u128(part + m.nch + k);
    }
    X = sib_block_sum256(x, s_red);
    if (pass == SIB_PASS_TOT) Y = sib_block_sum256(y, s_red);
  }
  bool final_draw = false;
  int rounds = 0;
  uint64_t S = 0;
  const u128* fpart = nullptr;
  if (pass == SIB_PASS_TOT) {
    if (t == 0) {
      SibState& s = *st;
      s.SA0 = (uint64_t)X;
      s.SB = (uint64_t)Y;
      s.hSA[0] = s.SA0;
      s_hSA[0] = s.SA0;
      const bool acc = sib_accept(a, s, s_hSA, s_hS, b, 0);
      s.done = acc ? 1 : 0;
      if (acc) {
        a.n_accept[b] = 0;
        a.next_token[b] = -1;
      }
    }
    return;
  }
  if (pass == SIB_PASS_D) {
    if (t == 0) {
      const uint64_t dhi = (uint64_t)(X >> 64), dlo = (uint64_t)X;
      const int bits = dhi ? 128 - __builtin_clzll(dhi) : (dlo ? 64 - __builtin_clzll(dlo) : 0);
      st->hS[round] = bits > 52 ? bits - 52 : 0;
    }
    return;
  }
  // SIB_PASS_A: total of round (round + 1)'s target
  const uint64_t SAn = (uint64_t)X;
  if (round + 1 < a.W) {
    if (t == 0) {
      SibState& s = *st;
      s.hSA[round + 1] = SAn;
      s_hSA[round + 1] = SAn;
      const bool acc = sib_accept(a, s, s_hSA, s_hS, b, round + 1);
      s.done = acc ? 1 : 0;
      if (acc) {
        a.n_accept[b] = round + 1;
        a.next_token[b] = -1;
      }
    }
    return;
  }
  // every candidate rejected: inverse-CDF draw from the last residual (from p if empty)
  final_draw = true;
  rounds = SAn > 0 ? a.W : 0;
  S = SAn > 0 ? SAn : st->SA0;
  fpart = part + (size_t)(SAn > 0 ? 3 : 0) * m.nch;  // chunk totals of that distribution
  (void)final_draw;
  const uint64_t* wd = a.words + (size_t)b * (a.W + 1) * 2;
  const uint64_t tau = scale_u32((uint32_t)(wd[2 * a.W + 1] >> 32), S);
  // the chunk holding tau: thread t owns chunks [t*cpt, (t+1)*cpt); a block scan of
  // the threads' totals gives each range's start
  __shared__ int s_cc;
  __shared__ uint64_t s_before;
  if (t == 0) {
    s_cc = -1;
    s_tok = -1;
  }
  {
    const int cpt = (m.nch + SIB_MB_THREADS - 1) / SIB_MB_THREADS;
    uint64_t mine = 0;
    for (int k = t * cpt; k < min((t + 1) * cpt, m.nch); ++k) mine += (uint64_t)ld_coh_u128(fpart + k);
    s_scan[t] = mine;
    __syncthreads();
    for (int o = 1; o < SIB_MB_THREADS; o <<= 1) {
      const uint64_t add = t >= o ? s_scan[t - o] : 0ull;
      __syncthreads();
      s_scan[t] += add;
      __syncthreads();
    }
    uint64_t before = s_scan[t] - mine;
    if (mine > 0 && before <= tau && tau < before + mine) {  // exactly one thread
      for (int k = t * cpt; k < min((t + 1) * cpt, m.nch); ++k) {
        const uint64_t w = (uint64_t)ld_coh_u128(fpart + k);
        if (tau < before + w) {
          s_cc = k;
          s_before = before;
          break;
        }
        before += w;
      }
    }
  }
  __syncthreads();
  const int cc = s_cc;
  if (cc >= 0) {
    // the chunk holding tau: this thread's SIB_PER entries, then a block scan
    uint64_t w[SIB_PER];
    uint64_t mine = 0;
    const int jb = cc * SIB_CHUNK + t * SIB_PER;
#pragma unroll
    for (int e = 0; e < SIB_PER; ++e) {
      const int j = jb + e;
      w[e] = j < a.V ? sib_chain(sib_weight(prow[j]), sib_weight(qrow[j]), rounds, s_hSA, s_hS, SB) : 0ull;
      mine += w[e];
    }
    s_scan[t] = mine;
    __syncthreads();
    for (int o = 1; o < SIB_MB_THREADS; o <<= 1) {
      const uint64_t add = t >= o ? s_scan[t - o] : 0ull;
      __syncthreads();
      s_scan[t] += add;
      __syncthreads();
    }
    uint64_t run = s_before + s_scan[t] - mine;  // entries before this thread's first
#pragma unroll
    for (int e = 0; e < SIB_PER; ++e) {
      if (w[e] > 0 && run <= tau && tau < run + w[e]) s_tok = jb + e;  // exactly one entry
      run += w[e];
    }
  }
  __syncthreads();
  if (t == 0) {
    st->done = 1;
    a.n_accept[b] = -1;
    a.next_token[b] = s_tok >= 0 ? s_tok : 0;
  }
}

// chunk partials of every (chunk, sequence), then the sequences' first rejections
static size_t verify_part_bytes(int B, int gamma, int V) {
  const size_t nch = (size_t)(V + VER_CHUNK - 1) / VER_CHUNK;
  const size_t per = std::max((size_t)16, (size_t)(gamma + 1) * sizeof(ArgMax));
  return align256((size_t)B * nch * per);
}
size_t verify_workspace(int B, int gamma, int V) {
  // also room for the multi-block sibling verification's state and partials
  return SPD_WS_COUNTER_BYTES + std::max(verify_part_bytes(B, gamma, V) + align256((size_t)B * 4),
                                         sib_state_bytes(B) + align256(sib_part_bytes(B, V)));
}

}  // namespace spd

using namespace spd;

extern "C" int spd_verify(int32_t B, int32_t gamma, int32_t V, float temperature, int32_t bonus,
                          const float* p, const float* q, const int32_t* draft,
                          const uint64_t* words, int32_t* n_accept, int32_t* next_token, void* ws,
                          size_t ws_bytes, void* stream) {
  if (B < 1 || B > 65535 || gamma < 0 || V < 1 || (bonus != 0 && bonus != 1)) return SPD_E_INVALID;
  if (gamma + bonus < 1 || gamma + bonus > VER_MAX_ROWS) return SPD_E_INVALID;
  if (!(temperature >= 0.f)) return SPD_E_INVALID;
  if (!p || !n_accept || !next_token || !ws || (gamma > 0 && !draft)) return SPD_E_INVALID;
  if (temperature > 0.f && (!words || (gamma > 0 && !q))) return SPD_E_INVALID;
  if (!aligned16(ws)) return SPD_E_INVALID;
  if (ws_bytes < verify_workspace(B, gamma, V)) return SPD_E_WORKSPACE;
  VerArgs a;
  a.p = p;
  a.q = q;
  a.draft = draft;
  a.words = words;
  a.n_accept = n_accept;
  a.next_token = next_token;
  a.part = static_cast<char*>(ws) + SPD_WS_COUNTER_BYTES;
  a.jrej = reinterpret_cast<int32_t*>(static_cast<char*>(a.part) + verify_part_bytes(B, gamma, V));
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.bonus = bonus;
  a.nchunks = (V + VER_CHUNK - 1) / VER_CHUNK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (temperature > 0.f) {
    hipLaunchKernelGGL(verify_sums_kernel, dim3(a.nchunks, B), dim3(VER_THREADS), 0, st, a);
    int rc = check_launch();
    if (rc) return rc;
    hipLaunchKernelGGL(verify_locate_kernel, dim3(B), dim3(VER_THREADS), 0, st, a);
  } else {
    hipLaunchKernelGGL(verify_greedy_chunks_kernel, dim3(a.nchunks, B), dim3(VER_THREADS), 0, st, a);
    int rc = check_launch();
    if (rc) return rc;
    hipLaunchKernelGGL(verify_greedy_final_kernel, dim3(B), dim3(VER_THREADS), 0, st, a);
  }
  return check_launch();
}

extern "C" int spd_verify_siblings(int32_t B, int32_t W, int32_t V, float temperature,
                                   const float* p, const float* q, const int32_t* cand,
                                   const uint64_t* words, int32_t* accepted, int32_t* next_token,
                                   void* ws, size_t ws_bytes, void* stream) {
  if (B < 1 || B > 65535 || W < 1 || W > SPD_TREE_MAX_NODES || V < 1) return SPD_E_INVALID;
  if (!(temperature >= 0.f)) return SPD_E_INVALID;
  if (!p || !cand || !accepted || !next_token || !ws || !aligned16(ws)) return SPD_E_INVALID;
  if (temperature > 0.f && (!q || !words)) return SPD_E_INVALID;
  if (ws_bytes < verify_workspace(B, 0, V)) return SPD_E_WORKSPACE;
  VerArgs a{};
  a.p = p;
  a.q = q;
  a.draft = cand;
  a.words = words;
  a.n_accept = accepted;
  a.next_token = next_token;
  a.part = static_cast<char*>(ws) + SPD_WS_COUNTER_BYTES;
  a.B = B;
  a.gamma = 0;  // the greedy chunk pass reads one target row per sequence
  a.bonus = 1;
  a.V = V;
  a.nchunks = (V + VER_CHUNK - 1) / VER_CHUNK;
  a.W = W;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (temperature > 0.f) {
    if (B >= SIB_MULTI_MAX_B) {
      // enough sequences to fill the GPU with one block each
      hipLaunchKernelGGL(verify_siblings_sampled_kernel, dim3(B), dim3(SIB_THREADS), 0, st, a);
      return check_launch();
    }
    SibMulti mm;
    char* base = static_cast<char*>(ws) + SPD_WS_COUNTER_BYTES;
    mm.st = reinterpret_cast<SibState*>(base);
    mm.part = reinterpret_cast<u128*>(base + sib_state_bytes(B));
    mm.counters = static_cast<unsigned*>(ws);
    mm.nch = (V + SIB_CHUNK - 1) / SIB_CHUNK;
    const dim3 grid(mm.nch, B);
    hipLaunchKernelGGL(sib_pass_kernel, grid, dim3(SIB_MB_THREADS), 0, st, a, mm, (int)SIB_PASS_TOT, 0);
    int rc = check_launch();
    for (int i = 0; i < W && !rc; ++i) {
      hipLaunchKernelGGL(sib_pass_kernel, grid, dim3(SIB_MB_THREADS), 0, st, a, mm, (int)SIB_PASS_D, i);
      rc = check_launch();
      if (rc) break;
      hipLaunchKernelGGL(sib_pass_kernel, grid, dim3(SIB_MB_THREADS), 0, st, a, mm, (int)SIB_PASS_A, i);
      rc = check_launch();
    }
    return rc;
  }
  hipLaunchKernelGGL(verify_greedy_chunks_kernel, dim3(a.nchunks, B), dim3(VER_THREADS), 0, st, a);
  int rc = check_launch();
  if (rc) return rc;
  hipLaunchKernelGGL(verify_siblings_final_kernel, dim3(B), dim3(VER_THREADS), 0, st, a);
  return check_launch();
}
