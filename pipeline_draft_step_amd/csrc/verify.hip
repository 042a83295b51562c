// spd_verify: speculative-sampling verification of drafted tokens.
// ("Speculative Pipeline Decoding", arXiv 2605.30852, section 3.4: streaming
// verification, greedy argmax match at T = 0, standard rejection sampling at T > 0;
// the speculative-decoding explainer's four-phase loop and acceptance criterion:
// accept if r <= min(1, p/q), else resample from norm(max(0, p - q)); bonus token
// from p_{gamma+1} when every draft is accepted.)
//
// T > 0, launch 1, grid (vocabulary chunks, sequences): every block decides the
//   sequence's outcome from the 2*gamma scalars p_j(x_j), q_j(x_j) (cheap, exact),
//   so a fully accepted sequence without bonus reads no rows; otherwise it sums
//   the exact integer weights of its chunk of the row to sample from (residual
//   and target weights both, for the empty-residual fallback).
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

// first rejected position of sequence b (gamma if all accepted); one thread
__device__ int first_reject(const VerArgs& a, int b) {
  const int rowsP = a.gamma + a.bonus;
  int j = 0;
  for (; j < a.gamma; ++j) {
    const int x = a.draft[b * a.gamma + j];
    bool acc = false;
    if (x >= 0 && x < a.V) {
      const double px = (double)a.p[((size_t)b * rowsP + j) * a.V + x];
      const double qx = (double)a.q[((size_t)b * a.gamma + j) * a.V + x];
      const uint64_t R = a.words[((size_t)b * (a.gamma + 1) + j) * 2] >> 40;
      acc = (double)(R + 1) * qx <= px * 16777216.0;
    }
    if (!acc) break;
  }
  return j;
}

__global__ __launch_bounds__(VER_THREADS) void verify_sums_kernel(VerArgs a) {
  __shared__ int s_j;
  const int c = blockIdx.x, b = blockIdx.y;
  if (threadIdx.x == 0) s_j = first_reject(a, b);
  __syncthreads();
  const int j = s_j;
  const bool rejected = j < a.gamma;
  if (!rejected && !a.bonus) return;
  const int rowsP = a.gamma + a.bonus;
  const float* prow = a.p + ((size_t)b * rowsP + j) * a.V;
  const float* qrow = rejected ? a.q + ((size_t)b * a.gamma + j) * a.V : nullptr;
  uint64_t sres = 0, sp = 0;
  constexpr int PER = VER_CHUNK / VER_THREADS;
  float pv[PER], qv[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int i = c * VER_CHUNK + threadIdx.x + VER_THREADS * e;
    pv[e] = i < a.V ? prow[i] : 0.f;
    qv[e] = (rejected && i < a.V) ? qrow[i] : 0.f;
  }
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    sp += prob_weight(pv[e]);
    if (rejected) sres += res_weight(pv[e], qv[e]);
  }
  sres = wave_sum_u64(sres);
  sp = wave_sum_u64(sp);
  __shared__ uint64_t s_w[2][VER_THREADS / 64];
  if ((threadIdx.x & 63) == 0) {
    s_w[0][threadIdx.x >> 6] = sres;
    s_w[1][threadIdx.x >> 6] = sp;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t0 = 0, t1 = 0;
    for (int w = 0; w < VER_THREADS / 64; ++w) {
      t0 += s_w[0][w];
      t1 += s_w[1][w];
    }
    uint64_t* part = static_cast<uint64_t*>(a.part) + ((size_t)b * a.nchunks + c) * 2;
    part[0] = t0;
    part[1] = t1;
  }
}

__global__ __launch_bounds__(VER_THREADS) void verify_locate_kernel(VerArgs a) {
  __shared__ uint64_t sh[VER_THREADS];
  __shared__ int s_j;
  __shared__ uint64_t s_tau, s_off;
  __shared__ int s_chunk, s_found;
  __shared__ uint64_t s_t[VER_THREADS / 64];
  const int b = blockIdx.x;
  if (threadIdx.x == 0) s_j = first_reject(a, b);
  __syncthreads();
  const int j = s_j;
  const bool rejected = j < a.gamma;
  if (!rejected && !a.bonus) {
    if (threadIdx.x == 0) {
      a.n_accept[b] = a.gamma;
      a.next_token[b] = -1;
    }
    return;
  }
  const int rowsP = a.gamma + a.bonus;
  const float* prow = a.p + ((size_t)b * rowsP + j) * a.V;
  const float* qrow = rejected ? a.q + ((size_t)b * a.gamma + j) * a.V : nullptr;
  const uint64_t* pb = static_cast<const uint64_t*>(a.part) + (size_t)b * a.nchunks * 2;
  // residual if it has mass, else the target row itself
  uint64_t tr = 0;
  for (int k = threadIdx.x; k < a.nchunks; k += VER_THREADS) tr += pb[2 * k];
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
    if (k < a.nchunks) mine += pb[2 * k + which];
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
      const uint64_t w = pb[2 * k + which];
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

size_t verify_workspace(int B, int gamma, int V) {
  const size_t nch = (size_t)(V + VER_CHUNK - 1) / VER_CHUNK;
  const size_t per = std::max((size_t)16, (size_t)(gamma + 1) * sizeof(ArgMax));
  return SPD_WS_COUNTER_BYTES + align256((size_t)B * nch * per);
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
    hipLaunchKernelGGL(verify_siblings_sampled_kernel, dim3(B), dim3(SIB_THREADS), 0, st, a);
    return check_launch();
  }
  hipLaunchKernelGGL(verify_greedy_chunks_kernel, dim3(a.nchunks, B), dim3(VER_THREADS), 0, st, a);
  int rc = check_launch();
  if (rc) return rc;
  hipLaunchKernelGGL(verify_siblings_final_kernel, dim3(B), dim3(VER_THREADS), 0, st, a);
  return check_launch();
}
