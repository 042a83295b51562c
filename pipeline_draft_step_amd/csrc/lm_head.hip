// spd_lm_head: logits = W_lm h over the vocabulary, then the next-token choice.
// ("Speculative Pipeline Decoding", arXiv 2605.30852: section 3.1 Eq. (1), the PDM's
// own head drafts x_{t+1}; section 3.4, the target head forms P of the token under
// verification.)
//
// Launch 1: the skinny GEMM streams W_lm once (HBM-bound).  Its epilogue writes
//   the logits and, per 128-row block, the (max, first argmax, sum exp((l-max)/T))
//   of each row; the last block merges the block statistics in fixed order and
//   writes the greedy token and the row's (max, sum).
// Launch 2 (T > 0): per 2048-entry chunk, probabilities p = exp((l-max)/T)/sum are
//   written and their exact integer weights floor(p*2^52) summed; the last chunk
//   to finish scans the chunk sums and locates tau = floor(u*S/2^32) first among
//   the chunks, then inside the chosen chunk.
#include "spd_common.h"
#include "spd_gemm.h"
#include "spd_host.h"

namespace spd {

constexpr int SMX_CHUNK = 2048;  // vocabulary entries per softmax/sample block
constexpr int SMX_THREADS = 256;

struct BlockStat {
  float mx;
  int arg;
  float se;
};

struct EpiLogits {
  float* logits;    // [rows][V]
  BlockStat* stat;  // [nblocks][rows]
  float2* rowstat;  // [rows] (max, sum exp)
  int32_t* token;   // [rows]
  unsigned* ctr2;
  int V, rows, nblocks;
  float inv_t;      // 1/T, 0 for greedy
  template <int NT, typename Y, typename RM>
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
          if (v[u] > -INFINITY) se += expf((v[u] - am.v) * inv_t);  // NaN adds NaN: rows must be finite
        se = wave_sum(se);
      }
      if (lane == 0) stat[(size_t)nb * rows + m0 + m] = BlockStat{am.v, am.i, se};
    }
    if (!arrive_last(ctr2, (unsigned)nblocks)) return;
    // merge block statistics: strided per thread, then a fixed tree
    __shared__ float s_mx[GEMM_THREADS];
    __shared__ int s_arg[GEMM_THREADS];
    __shared__ float s_se[GEMM_THREADS];
    for (int r = 0; r < rows; ++r) {
      float mx = -INFINITY, se = 0.f;
      int arg = ARG_NONE;
      for (int b = threadIdx.x; b < nblocks; b += GEMM_THREADS) {
        const BlockStat bs = stat[(size_t)b * rows + r];
        const ArgMax mm = argmax_merge(ArgMax{mx, arg}, ArgMax{bs.mx, bs.arg});
        if (inv_t > 0.f) {
          const float nm = fmaxf(mx, bs.mx);
          float acc = 0.f;
          if (mx > -INFINITY) acc += se * expf((mx - nm) * inv_t);
          if (bs.mx > -INFINITY) acc += bs.se * expf((bs.mx - nm) * inv_t);
          se = acc;
          mx = nm;
        } else {
          mx = mm.v;
        }
        arg = mm.i;
      }
      s_mx[threadIdx.x] = mx;
      s_arg[threadIdx.x] = arg;
      s_se[threadIdx.x] = se;
      __syncthreads();
      for (int w = GEMM_THREADS / 2; w > 0; w >>= 1) {
        if ((int)threadIdx.x < w) {
          const float m1 = s_mx[threadIdx.x], m2 = s_mx[threadIdx.x + w];
          const ArgMax mm = argmax_merge(ArgMax{m1, s_arg[threadIdx.x]}, ArgMax{m2, s_arg[threadIdx.x + w]});
          if (inv_t > 0.f) {
            const float nm = fmaxf(m1, m2);
            float acc = 0.f;
            if (m1 > -INFINITY) acc += s_se[threadIdx.x] * expf((m1 - nm) * inv_t);
            if (m2 > -INFINITY) acc += s_se[threadIdx.x + w] * expf((m2 - nm) * inv_t);
            s_se[threadIdx.x] = acc;
            s_mx[threadIdx.x] = nm;
          } else {
            s_mx[threadIdx.x] = mm.v;
          }
          s_arg[threadIdx.x] = mm.i;
        }
        __syncthreads();
      }
      if (threadIdx.x == 0) {
        rowstat[r] = make_float2(s_mx[0], s_se[0]);
        if (inv_t == 0.f) token[r] = s_arg[0] == ARG_NONE ? 0 : s_arg[0];
      }
      __syncthreads();
    }
    arrival_reset(ctr2);
  }
};

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
  return sh[threadIdx.x];
}

// Locate tau among weights w(j) of indices [base, base+n): returns the smallest j
// whose inclusive prefix (starting from `offset`) exceeds tau, or -1.
template <typename W>
__device__ int block_locate(const W& wfun, int base, int n, uint64_t offset, uint64_t tau,
                            uint64_t* sh) {
  __shared__ int s_found;
  constexpr int PER = SMX_CHUNK / SMX_THREADS;
  if (threadIdx.x == 0) s_found = -1;
  uint64_t w[PER];
  uint64_t tot = 0;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int j = threadIdx.x * PER + e;
    w[e] = j < n ? wfun(base + j) : 0ull;
    tot += w[e];
  }
  const uint64_t incl = block_scan_u64(tot, sh);
  uint64_t run = offset + incl - tot;
  if (run <= tau && offset + incl > tau) {  // exactly one thread
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      run += w[e];
      if (run > tau) {
        s_found = base + threadIdx.x * PER + e;
        break;
      }
    }
  }
  __syncthreads();
  return s_found;
}

// Sum of chunk weights per block, then the elected last block locates the sample.
__global__ __launch_bounds__(SMX_THREADS) void softmax_sample_kernel(
    const float* logits, float* probs, const float2* rowstat, const uint64_t* words, int32_t* token,
    uint64_t* csum, unsigned* counters, int V, int nchunks, float inv_t) {
  __shared__ uint64_t sh[SMX_THREADS];
  const int c = blockIdx.x, r = blockIdx.y;
  const float2 rs = rowstat[r];
  const float inv_sum = 1.0f / rs.y;
  const float* lr = logits + (size_t)r * V;
  float* pr = probs + (size_t)r * V;
  const int base = c * SMX_CHUNK;
  uint64_t part = 0;
  for (int j = base + threadIdx.x; j < min(base + SMX_CHUNK, V); j += SMX_THREADS) {
    const float p = expf((lr[j] - rs.x) * inv_t) * inv_sum;
    pr[j] = p;
    part += prob_weight(p);
  }
  part = wave_sum_u64(part);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = part;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t t = 0;
    for (int w = 0; w < SMX_THREADS / 64; ++w) t += sh[w];
    csum[(size_t)r * nchunks + c] = t;
  }
  __syncthreads();
  unsigned* ctr = counters + r;
  if (!arrive_last(ctr, (unsigned)nchunks)) return;

  // chunk-level prefix: chunks are assigned to threads in order
  __shared__ uint64_t s_tau, s_off;
  __shared__ int s_chunk;
  uint64_t mine = 0;
  const int per = (nchunks + SMX_THREADS - 1) / SMX_THREADS;
  for (int e = 0; e < per; ++e) {
    const int k = threadIdx.x * per + e;
    if (k < nchunks) mine += csum[(size_t)r * nchunks + k];
  }
  const uint64_t incl = block_scan_u64(mine, sh);
  if (threadIdx.x == SMX_THREADS - 1) {
    const uint64_t S = incl;  // total weight
    s_tau = scale_u32((uint32_t)(words[r] >> 32), S);
    s_chunk = -1;
  }
  __syncthreads();
  const uint64_t tau = s_tau;
  uint64_t run = incl - mine;
  if (run <= tau && incl > tau) {
    for (int e = 0; e < per; ++e) {
      const int k = threadIdx.x * per + e;
      if (k >= nchunks) break;
      const uint64_t w = csum[(size_t)r * nchunks + k];
      if (run + w > tau) {
        s_chunk = k;
        s_off = run;
        break;
      }
      run += w;
    }
  }
  __syncthreads();
  int tok = 0;
  if (s_chunk >= 0) {
    const int b0 = s_chunk * SMX_CHUNK;
    struct { const float* p; __device__ uint64_t operator()(int j) const { return prob_weight(p[j]); } } wf{pr};
    const int j = block_locate(wf, b0, min(SMX_CHUNK, V - b0), s_off, tau, sh);
    tok = j < 0 ? 0 : j;
  }
  if (threadIdx.x == 0) token[r] = tok;
  arrival_reset(ctr);
}

struct LmPlan {
  GemmPlan gp;
  int nchunks;
  size_t off_part, off_stat, off_rowstat, off_csum, total;
};

static LmPlan plan_lm(const spd_config* c, int rows) {
  LmPlan p;
  const bool bf = c->dtype == SPD_BF16;
  p.gp = plan_gemm(c->V, c->d, rows, bf ? Mfma<bf16>::KSTEP : Mfma<float>::KSTEP, bf ? 2 : 4, 2,
                   /*target=*/1, /*min_steps=*/1 << 30);
  p.nchunks = (c->V + SMX_CHUNK - 1) / SMX_CHUNK;
  size_t off = SPD_WS_COUNTER_BYTES;
  auto take = [&](size_t b) { size_t r = off; off = align256(off + b); return r; };
  p.off_part = take(p.gp.S > 1 ? (size_t)p.gp.S * rows * c->V * 4 : 0);
  p.off_stat = take((size_t)p.gp.nblocks * rows * sizeof(BlockStat));
  p.off_rowstat = take((size_t)rows * sizeof(float2));
  p.off_csum = take((size_t)rows * p.nchunks * 8);
  p.total = off;
  return p;
}

size_t lm_head_workspace(const spd_config* cfg, int rows) { return plan_lm(cfg, rows).total; }

template <typename WT>
static int lm_impl(const spd_config* c, const void* w_lm, const float* h, int rows, float T,
                   const uint64_t* words, float* logits, float* probs, int32_t* token, void* ws,
                   hipStream_t st) {
  const LmPlan p = plan_lm(c, rows);
  char* w = static_cast<char*>(ws);
  unsigned* ctr = reinterpret_cast<unsigned*>(w);
  GemmShape g;
  g.W = w_lm;
  g.N = c->V;
  g.K = c->d;
  g.M = rows;
  g.S = p.gp.S;
  g.nsteps = p.gp.nsteps;
  g.ldx = p.gp.ldx;
  g.part = reinterpret_cast<float*>(w + p.off_part);
  g.counters = ctr;
  g.nblocks = p.gp.nblocks;
  EpiLogits epi;
  epi.logits = logits;
  epi.stat = reinterpret_cast<BlockStat*>(w + p.off_stat);
  epi.rowstat = reinterpret_cast<float2*>(w + p.off_rowstat);
  epi.token = token;
  epi.ctr2 = ctr + CTR_FINAL;
  epi.V = c->V;
  epi.rows = rows;
  epi.nblocks = p.gp.nblocks;
  epi.inv_t = T > 0.f ? 1.0f / T : 0.f;
  int rc = launch_gemm<WT, 2>(p.gp, g, InAct<WT, float>{h, c->d}, epi, RowMapStd{}, st);
  if (rc || T <= 0.f) return rc;
  hipLaunchKernelGGL(softmax_sample_kernel, dim3(p.nchunks, rows), dim3(SMX_THREADS), 0, st, logits,
                     probs, epi.rowstat, words, token, reinterpret_cast<uint64_t*>(w + p.off_csum), ctr,
                     c->V, p.nchunks, epi.inv_t);
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
  if (!aligned16(w_lm) || !aligned16(ws)) return SPD_E_INVALID;
  if (ws_bytes < lm_head_workspace(cfg, rows)) return SPD_E_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cfg->dtype == SPD_BF16)
    return lm_impl<bf16>(cfg, w_lm, h, rows, temperature, words, logits, probs, token, ws, st);
  return lm_impl<float>(cfg, w_lm, h, rows, temperature, words, logits, probs, token, ws, st);
}
