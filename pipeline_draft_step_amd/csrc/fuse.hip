// spd_fuse_features: depth-conditioned features g = FC(RMSNorm(Concat(anchors))).
//
// "Speculative Pipeline Decoding" (arXiv 2605.30852) section 3.2, Eq. (3): a token
// at depth k uses every anchor b_j <= l_max(k); the review blog's core formulas
// give the operator FC(norm(Concat(.))) and g^0 = FC(H^0).
//
// One launch of the skinny GEMM.  The input functor gathers the row's eligible
// anchor states for its K-slice straight from the anchor store into LDS (empty
// slots are zeros; gamma is applied; the k = 0 rows read slot 0 only, without
// gamma) and records the slice's sum of squares.  Because FC is linear,
// W (gamma * x / rms) = (W (gamma * x)) / rms, so the epilogue divides the
// reduced product by the row's rms once the slice sums are known.
#include "spd_common.h"
#include "spd_gemm.h"
#include "spd_host.h"

namespace spd {

struct SlotTable {
  int8_t v[(SPD_MAX_STAGES + 1) * SPD_MAX_ANCHORS];
};

struct RowDepth {
  int M, a, n;
  __device__ __forceinline__ int operator()(int r) const { return r < M - a ? n : M - 1 - r; }
};

template <typename WT>
struct InAnchor {
  const WT* store;
  const WT* gamma;
  int64_t T_cap;
  int S_store, d, m, pos0, norm_k0;
  RowDepth depth;
  SlotTable tab;
  float* xss;  // [nblocks][S][M] slice sums of squares
  __device__ void stage(const XStage<WT>& xs, int m0, int Mt, int k0, int kw, int nb, int s, int S) const {
    // StageIdx layout (d % 4 == 0, so a group of 4 never straddles two anchor slots)
    const int kv = kw >> 2;
    const StageIdx ix(Mt, kv);
    float sq[STAGE_ROWS];
#pragma unroll
    for (int j = 0; j < STAGE_ROWS; ++j) sq[j] = 0.f;
    for (int b0 = 0; b0 < ix.n; b0 += STAGE_BATCH) {
      float4 v[STAGE_BATCH], gm[STAGE_BATCH];
#pragma unroll
      for (int i = 0; i < STAGE_BATCH; ++i) {
        int j, mm, u;
        ix.at(b0 + i, j, mm, u);
        // unconditional loads from clamped addresses, masked afterwards (a
        // conditional load becomes a branch whose join waits for every load)
        const bool ok = b0 + i < ix.n && u < kv;
        const int r = m0 + (ok ? mm : 0);
        const int k = depth(r);
        const bool plain = (k == 0) && !norm_k0;
        const int col = k0 + (ok ? 4 * u : 0);
        const int a = col / d;
        const int c = col - a * d;
        int slot = tab.v[k * m + a];
        if (plain && a != 0) slot = -1;
        const bool use = ok && slot >= 0 && slot < S_store;
        const float4 x = ldg4(store + ((size_t)(pos0 + r) * S_store + (use ? slot : 0)) * d + c);
        const float4 gg = ldg4(gamma + col);
        v[i] = use ? x : make_float4(0.f, 0.f, 0.f, 0.f);
        gm[i] = (use && !plain) ? gg : make_float4(1.f, 1.f, 1.f, 1.f);
      }
#pragma unroll
      for (int i = 0; i < STAGE_BATCH; ++i) {
        int j, mm, u;
        ix.at(b0 + i, j, mm, u);
        if (b0 + i < ix.n && u < kv) {
          const float q = v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
#pragma unroll
          for (int t = 0; t < STAGE_ROWS; ++t)
            if (t == j) sq[t] += q;
          const float x[4] = {v[i].x * gm[i].x, v[i].y * gm[i].y, v[i].z * gm[i].z, v[i].w * gm[i].w};
          xs.put4(mm, 4 * u, x);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < STAGE_ROWS; ++j) {
      const int mm = ix.wave + GEMM_WAVES * j;
      const float t = wave_sum(sq[j]);
      if (mm < Mt && ix.lane == 0) st_coh(xss + ((size_t)nb * S + s) * depth.M + m0 + mm, t);
    }
  }
};

template <typename WT>
struct EpiFeature {
  float* g;
  const float* xss;
  int d, m, S, norm_k0;
  float eps;
  RowDepth depth;
  SlotTable tab;
  template <int MT, int NT, typename Y, typename RM>
  __device__ void run(const Y& y, int nb, int m0, int Mt, const RM&) const {
    constexpr int TC = 64 * NT;
    __shared__ float inv[32];
    const int wave = threadIdx.x >> 6;
    for (int mm = wave; mm < Mt; mm += GEMM_WAVES) {
      const int r = m0 + mm;
      const int k = depth(r);
      const float* xp = xss + (size_t)nb * S * depth.M + r;
      const float t = wave_sum_of(S, [&](int q) { return ld_coh(xp + (size_t)q * depth.M); });
      if ((threadIdx.x & 63) == 0) {
        if (k == 0 && !norm_k0) {
          inv[mm] = 1.f;
        } else {
          int filled = 0;
          for (int j = 0; j < m; ++j) filled += tab.v[k * m + j] >= 0;
          inv[mm] = filled > 0 ? 1.0f / sqrtf(t / (float)(filled * d) + eps) : 0.f;
        }
      }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < Mt * TC; e += GEMM_THREADS) {
      const int mm = e / TC, c = e - mm * TC;
      const int col = nb * TC + c;
      if (col < d) g[(size_t)(m0 + mm) * d + col] = y(mm, c) * inv[mm];
    }
  }
};

struct FusePlan {
  GemmPlan gp;
  size_t off_xss, off_part, total;
};

static FusePlan plan_fuse(const spd_config* cfg, int M) {
  FusePlan p;
  const bool bf = cfg->dtype == SPD_BF16;
  const int kstep = bf ? Mfma<bf16>::KSTEP : Mfma<float>::KSTEP;
  p.gp = plan_gemm(cfg->d, cfg->m * cfg->d, M, kstep, bf ? 2 : 4, 1);
  size_t off = SPD_WS_COUNTER_BYTES;
  p.off_xss = off;
  off = align256(off + (size_t)p.gp.nblocks * p.gp.S * M * sizeof(float));
  p.off_part = off;
  if (p.gp.S > 1) off = align256(off + (size_t)p.gp.S * M * cfg->d * sizeof(float));
  p.total = off > 256 ? off : 256;
  return p;
}

size_t fuse_workspace(const spd_config* cfg, int M) { return plan_fuse(cfg, M).total; }

template <typename WT>
static int fuse_impl(const spd_config* cfg, const void* hstore, int64_t T_cap, int S_store,
                     const int32_t* slot_tab, int pos0, int M, int a, const void* norm_w,
                     const void* fc_w, float* g, void* ws, hipStream_t st) {
  FusePlan p = plan_fuse(cfg, M);
  const int d = cfg->d, m = cfg->m, n = cfg->n;
  SlotTable tab;
  for (int i = 0; i < (SPD_MAX_STAGES + 1) * SPD_MAX_ANCHORS; ++i) tab.v[i] = -1;
  for (int k = 0; k <= n; ++k)
    for (int j = 0; j < m; ++j) tab.v[k * m + j] = (int8_t)slot_tab[k * m + j];
  RowDepth dep{M, a, n};
  char* w = static_cast<char*>(ws);
  float* xss = reinterpret_cast<float*>(w + p.off_xss);

  GemmShape gs{};
  gs.W = fc_w;
  gs.N = d;
  gs.K = m * d;
  gs.M = M;
  gs.S = p.gp.S;
  gs.nsteps = p.gp.nsteps;
  gs.ldx = p.gp.ldx;
  gs.part = reinterpret_cast<float*>(w + p.off_part);
  gs.nblocks = p.gp.nblocks;
  gs.counters = reinterpret_cast<unsigned*>(w);

  InAnchor<WT> in{static_cast<const WT*>(hstore), static_cast<const WT*>(norm_w), T_cap, S_store,
                  d, m, pos0, cfg->norm_k0, dep, tab, xss};
  EpiFeature<WT> epi{g, xss, d, m, p.gp.S, cfg->norm_k0, cfg->rms_eps, dep, tab};
  return launch_gemm<WT, 1>(p.gp, gs, in, epi, RowMapStd{}, st);
}

}  // namespace spd

using namespace spd;

extern "C" int spd_fuse_features(const spd_config* cfg, const void* hstore, int64_t T_cap,
                                 int32_t S, const int32_t* slot_tab, int32_t pos0, int32_t M,
                                 int32_t a, const void* norm_w, const void* fc_w, float* g,
                                 void* ws, size_t ws_bytes, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!hstore || !slot_tab || !norm_w || !fc_w || !g || !ws) return SPD_E_INVALID;
  if (M < 1 || pos0 < 0 || T_cap < 1 || (int64_t)pos0 + M > T_cap || S < 1) return SPD_E_INVALID;
  if (a < 0 || a > cfg->n || a > M) return SPD_E_INVALID;
  if (cfg->d % 64) return SPD_E_UNSUPPORTED;
  for (int i = 0; i < (cfg->n + 1) * cfg->m; ++i)
    if (slot_tab[i] < -1 || slot_tab[i] >= S) return SPD_E_INVALID;
  if (!aligned16(hstore) || !aligned16(fc_w) || !aligned16(norm_w) || !aligned16(g) ||
      !aligned16(ws))
    return SPD_E_INVALID;
  if (ws_bytes < fuse_workspace(cfg, M)) return SPD_E_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (cfg->dtype == SPD_BF16)
    return fuse_impl<bf16>(cfg, hstore, T_cap, S, slot_tab, pos0, M, a, norm_w, fc_w, g, ws, st);
  return fuse_impl<float>(cfg, hstore, T_cap, S, slot_tab, pos0, M, a, norm_w, fc_w, g, ws, st);
}
