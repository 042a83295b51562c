// spd_fuse_features: depth-conditioned features g = FC(RMSNorm(Concat(anchors))).
//
// "Speculative Pipeline Decoding" (arXiv 2605.30852) section 3.2, Eq. (3): a token
// at depth k uses every anchor b_j <= l_max(k); the review blog's core formulas
// give the operator FC(norm(Concat(.))) and g^0 = FC(H^0).
//
// Two launches.  The gather kernel reads each row's eligible anchor states from
// the anchor store (empty slots are zeros; the k = 0 rows read slot 0 only,
// without gamma), writes gamma * x as the FC's input and the row's 1/rms over its
// filled slots (decode-sized calls split a row over several blocks and finish
// the sum in the last one; prefill-sized calls take one block per row).  Because FC is linear,
// W (gamma * x / rms) = (W (gamma * x)) / rms, so the row scale is applied to
// the product tile.  Decode-sized calls stream W_fc through the skinny GEMM,
// which takes the input pre-split into bf16 hi/lo parts (fp32-accurate
// activations); prefill-sized calls in bf16 run the MFMA-tiled large-M GEMM,
// which takes the bf16-rounded input as a plain bf16 operand.
//
// One launch (spd_fuse_features_scaled): with W_fc diag(gamma) prepared once
// (spd_fc_prepare), a prefill-sized call whose rows all sit at depth n, with anchor j
// in store slot j, runs only the large-M GEMM: A is the anchor store itself and the
// row scale comes from the sums of squares the product forms from its A tiles.
#include "spd_common.h"
#include "spd_gemm.h"
#include "spd_gemm_big.h"
#include "spd_host.h"

namespace spd {

constexpr int TABN = (SPD_MAX_STAGES + 1) * SPD_MAX_ANCHORS;
struct SlotTable {
  int8_t v[TABN];
};

// Pipeline depth of row r.  Chain (anc == null): the newest fully processed row(s)
// at depth n, then the a in-flight rows at a-1 .. 0.  Draft tree: node r at level
// l = popcount(anc[r]) - 1 has depth n at the root and a - l below it.
struct RowDepth {
  int M, a, n;
  const uint64_t* anc;
  __device__ __forceinline__ int operator()(int r) const {
    if (anc) {
      const int lv = __popcll(anc[r]) - 1;
      return lv <= 0 ? n : max(a - lv, 0);
    }
    return r < M - a ? n : M - 1 - r;
  }
};

constexpr int GATHER_COLS = 8 * 256;  // columns per gather block (8 per thread)

template <typename WT>
struct GatherArgs {
  const WT* store;  // [T_cap][S_store][d]
  const WT* gamma;  // [m*d]
  XSplit<WT> xo;    // [M][m*d]
  float* part;      // [ncb][M] partial sums of squares
  float* inv;       // [M] row scale
  unsigned* counters;
  int S_store, d, m, pos0, norm_k0, ncb;
  float eps;
  RowDepth depth;
  SlotTable tab;
};

// Block (column block cb, row r); each thread owns 8 consecutive columns, which
// never straddle two anchors (d % 64 == 0).
template <typename WT>
__global__ __launch_bounds__(256) void feature_gather_kernel(GatherArgs<WT> f) {
  __shared__ int8_t s_tab[TABN];
  __shared__ float s_red[4];
  __builtin_amdgcn_s_setprio(3);  // decode chain first on a shared SIMD (as in the GEMMs)
  if (threadIdx.x == 0) {
    // the table is copied with constant indices: a dynamically indexed kernel
    // argument would be copied to scratch memory
    int* dst = reinterpret_cast<int*>(s_tab);
    const int* src = reinterpret_cast<const int*>(f.tab.v);
#pragma unroll
    for (int i = 0; i < TABN / 4; ++i) dst[i] = src[i];
  }
  __syncthreads();
  const int cb = blockIdx.x, r = blockIdx.y;
  const int k = f.depth(r);
  const bool plain = (k == 0) && !f.norm_k0;
  const int K = f.m * f.d;
  const int col = cb * GATHER_COLS + 8 * threadIdx.x;
  const bool inb = col < K;
  const int a = inb ? col / f.d : 0;
  const int c = inb ? col - a * f.d : 0;
  int slot = s_tab[k * f.m + a];
  if (plain && a != 0) slot = -1;
  const bool use = inb && slot >= 0 && slot < f.S_store;
  // unconditional loads from clamped addresses, masked afterwards
  const WT* src = f.store + ((size_t)(f.pos0 + r) * f.S_store + (use ? slot : 0)) * f.d + c;
  const WT* gp = f.gamma + (inb ? col : 0);
  float x[8], gm[8];
  {
    const float4 x0 = ldg4(src), x1 = ldg4(src + 4);
    const float4 g0 = ldg4(gp), g1 = ldg4(gp + 4);
    const float xv[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] = use ? xv[e] : 0.f;
      gm[e] = plain ? 1.f : gv[e];
    }
  }
  float sq = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) sq += x[e] * x[e];
  if (inb) {
    const float4 lo4 = make_float4(x[0] * gm[0], x[1] * gm[1], x[2] * gm[2], x[3] * gm[3]);
    const float4 hi4 = make_float4(x[4] * gm[4], x[5] * gm[5], x[6] * gm[6], x[7] * gm[7]);
    f.xo.put4(r, col, lo4);
    f.xo.put4(r, col + 4, hi4);
  }
  sq = wave_sum(sq);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = sq;
  __syncthreads();
  if (threadIdx.x == 0) {
    // this block's share of the row's mean square over the eligible slots; the
    // product kernel adds the ncb shares (a row without norm leaves -1 in share 0)
    int filled = 0;
#pragma unroll
    for (int j = 0; j < SPD_MAX_ANCHORS; ++j) filled += (j < f.m && s_tab[k * f.m + j] >= 0) ? 1 : 0;
    const float blk = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    f.part[(size_t)cb * gridDim.y + r] =
        plain ? (cb == 0 ? -1.f : 0.f) : (filled > 0 ? blk / (float)(filled * f.d) : 0.f);
  }
}

// Large-M form of the gather (bf16-rounded input only): one block per row, so the
// row's sum of squares is a block reduction and no partial sums or arrival
// counters are needed.  Columns are taken in batches of GR_BATCH x 2048 whose
// loads are all issued before any of them is used.
constexpr int GR_BATCH = 4;

template <typename WT>
__global__ __launch_bounds__(256) void feature_gather_rows_kernel(GatherArgs<WT> f) {
  __shared__ int8_t s_tab[TABN];
  __shared__ float s_red[4];
  if (threadIdx.x == 0) {
    int* dst = reinterpret_cast<int*>(s_tab);
    const int* src = reinterpret_cast<const int*>(f.tab.v);
#pragma unroll
    for (int i = 0; i < TABN / 4; ++i) dst[i] = src[i];
  }
  __syncthreads();
  const int r = blockIdx.x;
  const int k = f.depth(r);
  const bool plain = (k == 0) && !f.norm_k0;
  const int K = f.m * f.d;
  const size_t row = (size_t)(f.pos0 + r) * f.S_store;
  float sq = 0.f;
  for (int base = 0; base < K; base += GR_BATCH * GATHER_COLS) {
    float4 xv[GR_BATCH][2], gv[GR_BATCH][2];
    bool use[GR_BATCH];
#pragma unroll
    for (int b = 0; b < GR_BATCH; ++b) {
      const int col = base + b * GATHER_COLS + 8 * threadIdx.x;
      const bool inb = col < K;
      const int a = inb ? col / f.d : 0;
      const int c = inb ? col - a * f.d : 0;
      int slot = s_tab[k * f.m + a];
      if (plain && a != 0) slot = -1;
      use[b] = inb && slot >= 0 && slot < f.S_store;
      const WT* src = f.store + (row + (use[b] ? slot : 0)) * f.d + c;
      const WT* gp = f.gamma + (inb ? col : 0);
      xv[b][0] = ldg4(src);
      xv[b][1] = ldg4(src + 4);
      gv[b][0] = ldg4(gp);
      gv[b][1] = ldg4(gp + 4);
    }
#pragma unroll
    for (int b = 0; b < GR_BATCH; ++b) {
      const int col = base + b * GATHER_COLS + 8 * threadIdx.x;
      const float x[8] = {xv[b][0].x, xv[b][0].y, xv[b][0].z, xv[b][0].w,
                          xv[b][1].x, xv[b][1].y, xv[b][1].z, xv[b][1].w};
      const float g[8] = {gv[b][0].x, gv[b][0].y, gv[b][0].z, gv[b][0].w,
                          gv[b][1].x, gv[b][1].y, gv[b][1].z, gv[b][1].w};
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xe = use[b] ? x[e] : 0.f;
        sq += xe * xe;
        y[e] = xe * (plain ? 1.f : g[e]);
      }
      if (col < K) {
        f.xo.put4_hi(r, col, make_float4(y[0], y[1], y[2], y[3]));
        f.xo.put4_hi(r, col + 4, make_float4(y[4], y[5], y[6], y[7]));
      }
    }
  }
  sq = wave_sum(sq);
  if ((threadIdx.x & 63) == 0) s_red[threadIdx.x >> 6] = sq;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float t = (s_red[0] + s_red[1]) + (s_red[2] + s_red[3]);
    int filled = 0;
#pragma unroll
    for (int j = 0; j < SPD_MAX_ANCHORS; ++j) filled += (j < f.m && s_tab[k * f.m + j] >= 0) ? 1 : 0;
    f.inv[r] = plain ? 1.f : (filled > 0 ? 1.0f / sqrtf(t / (float)(filled * f.d) + f.eps) : 0.f);
  }
}

// g[row][col] = y (the row scale is already applied to the tile)
struct EpiRows {
  float* g;
  int N;
  template <int MT, int NT, typename Y, typename RM>
  __device__ void run(const Y& y, int nb, int m0, int Mt, const RM&) const {
    constexpr int TC = 64 * NT;
    for (int e = threadIdx.x; e < Mt * TC; e += GEMM_THREADS) {
      const int mm = e / TC, c = e - mm * TC;
      const int col = nb * TC + c;
      if (col < N) g[(size_t)(m0 + mm) * N + col] = y(mm, c);
    }
  }
};

// Large-M path: bf16 only, for prefill-sized M, when the K range splits into
// whole 64-wide stages.
constexpr int FUSE_BIG_MIN_M = 256;

static BigPlan plan_big(const spd_config* cfg, int M) {
  if (cfg->dtype != SPD_BF16 || M < FUSE_BIG_MIN_M) return BigPlan{};
  return plan_big_gemm(M, cfg->d, cfg->m * cfg->d);
}

struct FusePlan {
  GemmPlan gp;
  BigPlan big;
  int ncb;
  size_t off_part, off_inv, off_xh, off_xl, off_gpart, off_gsq, total;
};

static FusePlan plan_fuse(const spd_config* cfg, int M) {
  FusePlan p;
  const bool bf = cfg->dtype == SPD_BF16;
  const int kstep = bf ? Mfma<bf16>::KSTEP : Mfma<float>::KSTEP;
  const int es = bf ? 2 : 4;
  const size_t K = (size_t)cfg->m * cfg->d;
  p.big = plan_big(cfg, M);
  // about one block per CU.  Tiles of up to 16 rows take 128 columns per block with K
  // split twelve ways at the 2560-wide shape (measured against 64 columns and six
  // parts: the feature call alone 1 us slower, the headline cycle 364.4 -> 361.0 us,
  // the n = 4 cycle unchanged within 0.3%); 32-row tiles keep 64 columns (128 made the
  // 29-node tree's features faster, 46 -> 35 us, but the 9B-shaped 17-row cycle
  // slower, 1091 -> 1114 us).  Measured before: 320 blocks of the 62 KB budget ran
  // the cycle 1.6% slower than 240 of the 100 KB budget.
  p.gp = plan_gemm(cfg->d, (int)K, M, kstep, es, M > 16 ? 1 : 2, 256, 8, M > 16 ? 0 : 100 * 1024);
  p.ncb = (int)((K + GATHER_COLS - 1) / GATHER_COLS);
  size_t off = SPD_WS_COUNTER_BYTES;
  auto take = [&](size_t b) { size_t r = off; off = align256(off + b); return r; };
  p.off_part = take((size_t)p.ncb * M * 4);
  p.off_inv = take((size_t)M * 4);
  p.off_xh = take((size_t)M * K * es);
  if (p.big.use) {
    p.off_xl = take(0);
    p.off_gpart = take(p.big.part_bytes);
    p.off_gsq = take(p.big.sq_bytes);
  } else {
    p.off_xl = take(bf ? (size_t)M * K * es : 0);
    p.off_gpart = take(p.gp.S > 1 ? (size_t)p.gp.S * M * cfg->d * 4 : 0);
    p.off_gsq = take(0);
  }
  p.total = off;
  return p;
}

size_t fuse_workspace(const spd_config* cfg, int M) { return plan_fuse(cfg, M).total; }

// Prefill-sized calls whose rows all sit at depth n, with every anchor j in store
// slot j at that depth: each row's concatenation is the first m d values of its
// store row, so with the weights' columns already scaled by norm_w (spd_fc_prepare)
// the product reads the store directly and forms the rows' 1/rms from the staged
// tiles (no gather launch, no staged copy of the input).
static bool direct_rows(const spd_config* cfg, const int32_t* slot_tab, int a, const uint64_t* anc,
                        const void* fc_w_scaled, const BigPlan& big) {
  if (!fc_w_scaled || !big.use || anc || a != 0 || cfg->dtype != SPD_BF16) return false;
  for (int j = 0; j < cfg->m; ++j)
    if (slot_tab[cfg->n * cfg->m + j] != j) return false;
  return true;
}

template <typename WT>
static int fuse_impl(const spd_config* cfg, const void* hstore, int64_t T_cap, int S_store,
                     const int32_t* slot_tab, int pos0, int M, int a, const uint64_t* anc,
                     const void* norm_w, const void* fc_w, const void* fc_w_scaled, float* g, void* ws,
                     hipStream_t st) {
  (void)T_cap;
  FusePlan p = plan_fuse(cfg, M);
  const int d = cfg->d, m = cfg->m, n = cfg->n;
  char* w = static_cast<char*>(ws);
  if constexpr (sizeof(WT) == 2) {
    if (direct_rows(cfg, slot_tab, a, anc, fc_w_scaled, p.big)) {
      const bf16* A = static_cast<const bf16*>(hstore) + (size_t)pos0 * S_store * d;
      launch_big_gemm(p.big, A, S_store * d, static_cast<const bf16*>(fc_w_scaled), g, d, nullptr, M, d, m * d,
                      reinterpret_cast<float*>(w + p.off_gpart), reinterpret_cast<unsigned*>(w), st, 0,
                      reinterpret_cast<float*>(w + p.off_gsq), m * d, cfg->rms_eps);
      return check_launch();
    }
  }
  GatherArgs<WT> ga;
  for (int i = 0; i < TABN; ++i) ga.tab.v[i] = -1;
  for (int k = 0; k <= n; ++k)
    for (int j = 0; j < m; ++j) ga.tab.v[k * m + j] = (int8_t)slot_tab[k * m + j];
  ga.store = static_cast<const WT*>(hstore);
  ga.gamma = static_cast<const WT*>(norm_w);
  ga.xo = XSplit<WT>{reinterpret_cast<WT*>(w + p.off_xh), reinterpret_cast<WT*>(w + p.off_xl), m * d};
  ga.part = reinterpret_cast<float*>(w + p.off_part);
  ga.inv = reinterpret_cast<float*>(w + p.off_inv);
  ga.counters = reinterpret_cast<unsigned*>(w);
  ga.S_store = S_store;
  ga.d = d;
  ga.m = m;
  ga.pos0 = pos0;
  // under the post-step schedule the staircase's depth-0 row uses depth-1 features,
  // which are normalised like every depth >= 1 row
  ga.norm_k0 = cfg->norm_k0 || cfg->feature_schedule == SPD_SCHEDULE_POST_STEP;
  ga.ncb = p.ncb;
  ga.eps = cfg->rms_eps;
  ga.depth = RowDepth{M, a, n, anc};
  if (p.big.use && !anc) {
    if constexpr (sizeof(WT) == 2) {
      hipLaunchKernelGGL((feature_gather_rows_kernel<WT>), dim3(M), dim3(256), 0, st, ga);
      int rc = check_launch();
      if (rc) return rc;
      // the gather's row counters are back at zero when it ends, so the GEMM
      // reuses the start of the counter region for its tile counters
      launch_big_gemm(p.big, reinterpret_cast<const bf16*>(ga.xo.hi), m * d, static_cast<const bf16*>(fc_w), g,
                      d, ga.inv, M, d, m * d, reinterpret_cast<float*>(w + p.off_gpart),
                      reinterpret_cast<unsigned*>(w), st);
      return check_launch();
    }
  }
  hipLaunchKernelGGL((feature_gather_kernel<WT>), dim3(p.ncb, M), dim3(256), 0, st, ga);
  int rc = check_launch();
  if (rc) return rc;

  GemmShape gs{};
  gs.W = fc_w;
  gs.N = d;
  gs.K = m * d;
  gs.M = M;
  gs.S = p.gp.S;
  gs.nsteps = p.gp.nsteps;
  gs.ldx = p.gp.ldx;
  gs.part = reinterpret_cast<float*>(w + p.off_gpart);
  gs.nblocks = p.gp.nblocks;
  gs.counters = reinterpret_cast<unsigned*>(w);
  gs.rs_ss = ga.part;
  gs.rs_P = p.ncb;
  gs.rs_M = M;
  gs.rs_K = 1;
  gs.rs_eps = cfg->rms_eps;
  InSplit<WT, RS_SSR> in{ga.xo.hi, ga.xo.lo, m * d};
  if (p.gp.NT == 2) return launch_gemm<WT, 2>(p.gp, gs, in, EpiRows{g, d}, RowMapStd{}, st);
  return launch_gemm<WT, 1>(p.gp, gs, in, EpiRows{g, d}, RowMapStd{}, st);
}

}  // namespace spd

using namespace spd;

static int fuse_entry(const spd_config* cfg, const void* hstore, int64_t T_cap, int32_t S,
                      const int32_t* slot_tab, int32_t pos0, int32_t M, int32_t a,
                      const uint64_t* anc, const void* norm_w, const void* fc_w, const void* fc_w_scaled,
                      float* g, void* ws, size_t ws_bytes, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!hstore || !slot_tab || !norm_w || !fc_w || !g || !ws) return SPD_E_INVALID;
  if (M < 1 || pos0 < 0 || T_cap < 1 || (int64_t)pos0 + M > T_cap || S < 1) return SPD_E_INVALID;
  if (a < 0 || a > cfg->n || a > M) return SPD_E_INVALID;
  if (M >= CTR_FINAL) return SPD_E_UNSUPPORTED;  // one arrival counter per row (and per GEMM tile)
  if (cfg->d % 64) return SPD_E_UNSUPPORTED;
  // the product kernel reduces at most 128 gather blocks' shares per row
  if ((int64_t)cfg->m * cfg->d > (int64_t)128 * GATHER_COLS) return SPD_E_UNSUPPORTED;
  for (int i = 0; i < (cfg->n + 1) * cfg->m; ++i)
    if (slot_tab[i] < -1 || slot_tab[i] >= S) return SPD_E_INVALID;
  if (!aligned16(hstore) || !aligned16(fc_w) || !aligned16(norm_w) || !aligned16(g) ||
      !aligned16(ws) || !aligned16(fc_w_scaled))
    return SPD_E_INVALID;
  if (ws_bytes < fuse_workspace(cfg, M)) return SPD_E_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cfg->dtype == SPD_BF16)
    return fuse_impl<bf16>(cfg, hstore, T_cap, S, slot_tab, pos0, M, a, anc, norm_w, fc_w, fc_w_scaled, g, ws,
                           st);
  return fuse_impl<float>(cfg, hstore, T_cap, S, slot_tab, pos0, M, a, anc, norm_w, fc_w, fc_w_scaled, g, ws,
                          st);
}

extern "C" int spd_fuse_features(const spd_config* cfg, const void* hstore, int64_t T_cap,
                                 int32_t S, const int32_t* slot_tab, int32_t pos0, int32_t M,
                                 int32_t a, const void* norm_w, const void* fc_w, float* g,
                                 void* ws, size_t ws_bytes, void* stream) {
  return fuse_entry(cfg, hstore, T_cap, S, slot_tab, pos0, M, a, nullptr, norm_w, fc_w, nullptr, g, ws,
                    ws_bytes, stream);
}

extern "C" int spd_fuse_features_scaled(const spd_config* cfg, const void* hstore, int64_t T_cap,
                                        int32_t S, const int32_t* slot_tab, int32_t pos0, int32_t M,
                                        int32_t a, const void* norm_w, const void* fc_w,
                                        const void* fc_w_scaled, float* g, void* ws, size_t ws_bytes,
                                        void* stream) {
  if (!fc_w_scaled) return SPD_E_INVALID;
  return fuse_entry(cfg, hstore, T_cap, S, slot_tab, pos0, M, a, nullptr, norm_w, fc_w, fc_w_scaled, g, ws,
                    ws_bytes, stream);
}

namespace {

// out[c][k] = bf16(fc_w[c][k] * norm_w[k]); the product of two bf16 values is exact
// in fp32, so the result is rounded once
__global__ __launch_bounds__(256) void fc_scale_kernel(const bf16* fc_w, const bf16* norm_w, bf16* out, int K,
                                                       int64_t n8) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < n8; e += (int64_t)gridDim.x * 256) {
    const int64_t i = e * 8;
    const int k = (int)(i % K);
    const uint4 wv = *reinterpret_cast<const uint4*>(fc_w + i);
    const uint4 gv = *reinterpret_cast<const uint4*>(norm_w + k);
    const uint32_t* wa = reinterpret_cast<const uint32_t*>(&wv);
    const uint32_t* ga = reinterpret_cast<const uint32_t*>(&gv);
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = pack2_bf16(bf2f((bf16)(wa[q] & 0xffff)) * bf2f((bf16)(ga[q] & 0xffff)),
                        bf2f((bf16)(wa[q] >> 16)) * bf2f((bf16)(ga[q] >> 16)));
    *reinterpret_cast<uint4*>(out + i) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

extern "C" int spd_fc_prepare(const spd_config* cfg, const void* norm_w, const void* fc_w, void* fc_w_scaled,
                              void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!norm_w || !fc_w || !fc_w_scaled) return SPD_E_INVALID;
  if (cfg->dtype != SPD_BF16) return SPD_E_UNSUPPORTED;
  if (!aligned16(norm_w) || !aligned16(fc_w) || !aligned16(fc_w_scaled)) return SPD_E_INVALID;
  const int K = cfg->m * cfg->d;  // d % 64 == 0: whole 8-element groups
  if (cfg->d % 64) return SPD_E_UNSUPPORTED;
  const int64_t n8 = (int64_t)cfg->d * K / 8;
  const int blocks = (int)std::min<int64_t>((n8 + 255) / 256, 4096);
  hipLaunchKernelGGL(fc_scale_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const bf16*>(fc_w), static_cast<const bf16*>(norm_w), static_cast<bf16*>(fc_w_scaled),
                     K, n8);
  return check_launch();
}

extern "C" int spd_fuse_features_tree(const spd_config* cfg, const void* hstore, int64_t T_cap,
                                      int32_t S, const int32_t* slot_tab, int32_t pos0, int32_t M,
                                      int32_t a, const uint64_t* anc, const void* norm_w,
                                      const void* fc_w, float* g, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (!anc || ((uintptr_t)anc & 7) || M > SPD_TREE_MAX_NODES || a < 1) return SPD_E_INVALID;
  return fuse_entry(cfg, hstore, T_cap, S, slot_tab, pos0, M, a, anc, norm_w, fc_w, nullptr, g, ws,
                    ws_bytes, stream);
}
