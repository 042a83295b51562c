// spd_pdm_step: the Pipeline Draft Module, an Ls-layer Qwen3-style decoder
// ("Speculative Pipeline Decoding", arXiv 2605.30852, section 3.1) run over the
// M rows a cycle recomputes, attending to the committed key/value cache.
//
// Per layer (5 launches):
//   QKV GEMM  : X = RMSNorm(h)*attn_norm staged in LDS (bf16 hi+lo pairs); per head:
//               q/k RMSNorm, rotate-half RoPE, k/v written to the cache, q kept.
//   attention : MFMA flash-decode, one block per (128-key chunk, kv head, 16-row
//               query tile), GQA rows of a kv head together, waves merged in LDS;
//               the last chunk block of a (kv head, tile) merges the chunk partials.
//   O GEMM    : h += W_o attn                (epilogue keeps row sums of squares)
//   gate/up   : X = RMSNorm(h)*mlp_norm; epilogue silu(gate)*up
//   down GEMM : h += W_down act.
// GEMMs split over K reduce their partial tiles in the last block of each tile.
// The last layer runs its QKV GEMM over every row (the cache needs all keys and
// values) and the other four launches over the output rows only; its down
// epilogue writes h_last = RMSNorm(h[M-1]) * final_norm.
//
// Prefill-sized steps (bf16, M >= 256, hd = 128) run the products on the large-M
// MFMA GEMM with row kernels for the epilogues and causal flash attention (pdm_big).
// With weights prepared by spd_pdm_prepare (e4m3 rows with per-row power-of-two
// factors) the QKV, gate/up and down inputs are [hi | lo8] rows and the residuals'
// products run on the block-scaled fp8 MFMA (spd_pdm_step_prepared).
#include <math.h>

#include <algorithm>

#include "spd_common.h"
#include "spd_gemm.h"
#include "spd_gemm_big.h"
#include "spd_host.h"

namespace spd {

constexpr int ATT_SUB = 32;                     // keys per wave
constexpr int ATT_WAVES = 4;                    // waves per attention block
constexpr int ATT_KC = ATT_SUB * ATT_WAVES;     // keys per block (one partial per row)
constexpr int ATT_MAXCH = 256;                  // chunks per row: context up to 32768

// h = g, per-64-column partial sums of squares of every row, and the first QKV
// GEMM's input g * attn_norm as an XSplit (its RMSNorm row scale comes from ss)
// Blocks with nb == 0 also write the rotate-half RoPE table of the row's
// position, rope[r][i] = (cos, sin)(pos * theta^(-2i/hd)), i < hd/2, in fp64.
template <typename WT>
__global__ __launch_bounds__(64) void rows_init_kernel(const float* g, float* h, float* ss, int M,
                                                       int d, XSplit<WT> xo, const WT* gamma,
                                                       float2* rope, int pos0, int hd, float theta,
                                                       const uint64_t* anc) {
  __builtin_amdgcn_s_setprio(3);  // decode chain first on a shared SIMD (as in the GEMMs)
  const int nb = blockIdx.x, r = blockIdx.y, lane = threadIdx.x;
  if (nb == 0 && lane < hd / 2) {
    // a draft-tree node sits at its level (number of proper ancestors), a chain row at r
    const int off = anc ? max(__popcll(anc[r]) - 1, 0) : r;
    double sn, cs;
    sincos((double)(pos0 + off) * pow((double)theta, -2.0 * lane / hd), &sn, &cs);
    rope[(size_t)r * (hd / 2) + lane] = make_float2((float)cs, (float)sn);
  }
  const int col = nb * 64 + lane;
  const size_t i = (size_t)r * d + col;
  const float v = g[i];
  h[i] = v;
  xo.put1(r, col, v * to_f<WT>(gamma[col]));
  const float s = wave_sum(v * v);
  if (lane == 0) ss[(size_t)nb * M + r] = s;
}

// q/k RMSNorm + RoPE, cache writes.  Block columns cover whole heads (64*NT % hd == 0).
template <typename WT>
struct EpiQKV {
  float* qbuf;  // [M][Hq][hd]
  WT* kc;       // [Hkv][T_cap][hd]
  WT* vc;       // [Hkv][hd][T_cap]
  const WT* qn;
  const WT* kn;
  const float2* rope;  // [M][hd/2] (cos, sin) of each row's position
  int Hq, Hkv, hd, pos0;
  int64_t T_cap;
  float eps;
  template <int MT, int NT, typename Y, typename RM>
  __device__ void run(const Y& y, int nb, int m0, int Mt, const RM&) const {
    constexpr int TC = 64 * NT;
    const int hpb = TC / hd;
    const int nheads = Hq + 2 * Hkv;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int half = hd >> 1;
    const int fi = hd == 128 ? lane : (lane & (half - 1));  // frequency index of this lane
    const int l0 = min(lane, hd - 1), l1 = min(lane + 64, hd - 1);  // clamped: loads stay unconditional
    for (int it = wave; it < Mt * hpb; it += GEMM_WAVES) {
      const int mm = it / hpb, hl = it - mm * hpb;
      const int hh = nb * hpb + hl;
      if (hh >= nheads) continue;
      const int r = m0 + mm, pos = pos0 + r;
      const bool e0 = lane < hd, e1 = lane + 64 < hd;
      float v0 = e0 ? y(mm, hl * hd + lane) : 0.f;
      float v1 = e1 ? y(mm, hl * hd + lane + 64) : 0.f;
      if (hh < Hq + Hkv) {
        const WT* nw = hh < Hq ? qn : kn;
        const float w0 = to_f<WT>(nw[l0]), w1 = to_f<WT>(nw[l1]);
        const float2 cs = rope[(size_t)r * half + fi];
        const float inv = 1.0f / sqrtf(wave_sum(v0 * v0 + v1 * v1) / (float)hd + eps);
        v0 = e0 ? v0 * inv * w0 : 0.f;
        v1 = e1 ? v1 * inv * w1 : 0.f;
        // rotate-half: element i pairs with i + hd/2 at angle pos * theta^(-2i/hd)
        if (hd == 128) {
          const float x1 = v0, x2 = v1;
          v0 = x1 * cs.x - x2 * cs.y;
          v1 = x2 * cs.x + x1 * cs.y;
        } else {
          const float other = __shfl_xor(v0, half, WAVE);
          v0 = lane < half ? v0 * cs.x - other * cs.y : v0 * cs.x + other * cs.y;
        }
      }
      if (hh < Hq) {
        float* qp = qbuf + ((size_t)r * Hq + hh) * hd;
        if (e0) qp[lane] = v0;
        if (e1) qp[lane + 64] = v1;
      } else if (hh < Hq + Hkv) {
        WT* kp = kc + ((size_t)(hh - Hq) * T_cap + pos) * hd;
        if (e0) kp[lane] = from_f<WT>(v0);
        if (e1) kp[lane + 64] = from_f<WT>(v1);
      } else {
        WT* vp = vc + (size_t)(hh - Hq - Hkv) * hd * T_cap + pos;
        if (e0) vp[(size_t)lane * T_cap] = from_f<WT>(v0);
        if (e1) vp[(size_t)(lane + 64) * T_cap] = from_f<WT>(v1);
      }
    }
  }
};

struct AttnArgs {
  const float* q;  // [M][Hq][hd]
  const void* kc;  // [Hkv][T_cap][hd]
  const void* vc;  // [Hkv][hd][T_cap]
  float* po;       // [Hkv][QR][nch][hd]
  float2* pml;     // [Hkv][QR][nch]  (chunk max, chunk sum of exp)
  void* xh;        // attention output [M][Hq*hd] as the O projection's XSplit input
  void* xl;
  int xld;         // row stride of xh / xl (elements)
  unsigned* counters;  // [Hkv][nqt]
  const uint64_t* anc;  // draft-tree ancestor masks [M], or null for causal rows
  int M, Hq, Hkv, pos0, nch, nqt;
  int r0;  // query rows r0 .. M-1 (local rows 0 .. M-1-r0 of the output); keys of all M rows
  int64_t T_cap;
  float scale;
};

// One block: kv head h (blockIdx.y), keys [ATT_KC c, ATT_KC (c+1)) (blockIdx.x),
// one 16-row tile of the head's GQA query rows (blockIdx.z).  Wave w owns ATT_SUB
// keys: S^T = K Q^T and O^T = V^T P^T on MFMA (Q and P as bf16 hi + lo pairs),
// softmax over its keys; the four waves are merged in LDS (log-sum-exp) into one
// partial per query.  The K rows of S^T tile ks are taken in the order
// key(ks, r) = KSTEP (v / KPL) + KPL (r / 4) + v % KPL with v = 4 ks + r % 4, so
// that the lane holding query c of tile rows 4 g .. 4 g + 3 holds exactly the
// keys of its P^T operand (keys KSTEP kt + KPL g + j): P stays in registers.
template <typename WT, int HD>
__global__ __launch_bounds__(256) void attn_partial_kernel(AttnArgs a) {
  typedef Mfma<WT> F;
  typedef typename F::frag frag;
  constexpr int KS = ATT_SUB / 16;
  constexpr int DS = HD / F::KSTEP;
  constexpr int KT = ATT_SUB / F::KSTEP;
  constexpr int DT = HD / 16;
  constexpr int KPL = F::KPL;
  constexpr bool SPLIT = sizeof(WT) == 2;
  static_assert(KS == 2 && KT * KPL == 4 * KS, "a lane holds 4 KS scores = the KT KPL keys of its P^T");
  __shared__ __align__(16) float Ob[ATT_WAVES][16][HD + 4];
  __shared__ float2 Ml[ATT_WAVES][16];

  __builtin_amdgcn_s_setprio(3);  // decode chain first on a shared SIMD (as in the GEMMs)
  const int c = blockIdx.x, h = blockIdx.y, qt = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int G = a.Hq / a.Hkv, QR = (a.M - a.r0) * G;
  const int nkeys = a.pos0 + a.M;
  const int qpos0 = a.pos0 + a.r0;  // position of local query row 0
  const int r_last = (min(QR, 16 * qt + 16) - 1) / G;
  if (c * ATT_KC > qpos0 + r_last) return;  // every row of the tile is masked here
  const int key0 = c * ATT_KC + wave * ATT_SUB;
  // key offset (within the wave's keys) of S^T tile ks, row r
  auto key_of = [](int ks, int r) {
    const int v = 4 * ks + (r & 3);
    return F::KSTEP * (v / KPL) + KPL * (r >> 2) + v % KPL;
  };

  const WT* K = static_cast<const WT*>(a.kc) + (size_t)h * a.T_cap * HD;
  const WT* Vt = static_cast<const WT*>(a.vc) + (size_t)h * HD * a.T_cap;
  // All loads are unconditional (a conditional load becomes a branch whose join
  // waits for every outstanding load) and issued in the order they are needed:
  // Q, K, then V.  Query = 16*qt + lr (clamped; rows past QR are zeroed).
  const int qi = 16 * qt + lr;
  const bool qv = qi < QR;
  const float* qp = a.q + ((size_t)(a.r0 + (qv ? qi / G : 0)) * a.Hq + h * G + (qv ? qi % G : 0)) * HD;
  float qraw[DS][KPL];
#pragma unroll
  for (int ds = 0; ds < DS; ++ds)
#pragma unroll
    for (int e = 0; e < KPL; ++e) qraw[ds][e] = qp[ds * F::KSTEP + lg * KPL + e];
  frag kf[KS][DS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int key = min(key0 + key_of(ks, lr), nkeys - 1);
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) kf[ks][ds] = F::load(K + (size_t)key * HD + ds * F::KSTEP + lg * KPL);
  }
  // V^T (A operand): this lane's KPL keys start at kb; kb + KPL <= T_cap whenever
  // kb < nkeys (both multiples of KPL), so the clamp only moves fully masked fragments
  frag vf[KT][DT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int kb = key0 + kt * F::KSTEP + lg * KPL;
    const int kbc = min(kb, (int)a.T_cap - KPL);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[kt][dt] = F::load(Vt + (size_t)(dt * 16 + lr) * a.T_cap + kbc);
  }
  __builtin_amdgcn_sched_barrier(0);  // keep V in flight with Q and K
  // Q fragments (B operand), pre-scaled by 1/sqrt(hd), as hi + lo pairs
  frag qf[DS], ql[DS];
  const float qs = qv ? a.scale : 0.f;  // clamped rows (finite values) become zero
#pragma unroll
  for (int ds = 0; ds < DS; ++ds) {
    float tmp[KPL], rem[KPL];
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
      tmp[e] = qraw[ds][e] * qs;  // used unconditionally: no load is sunk into a branch
      rem[e] = tmp[e] - to_f<WT>(from_f<WT>(tmp[e]));
    }
    qf[ds] = F::pack(tmp);
    ql[ds] = F::pack(rem);
  }
  f32x4 sc[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    sc[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < DS; ++ds) {
      sc[ks] = F::mma(kf[ks][ds], qf[ds], sc[ks]);
      if constexpr (SPLIT) sc[ks] = F::mma(kf[ks][ds], ql[ds], sc[ks]);
    }
  }
  // lane holds S^T[key_of(ks, 4 lg + e)][query lr]
  const int lim = qv ? qpos0 + qi / G : -1;
  // draft tree: a row reads the new keys of its own root path only
  const uint64_t am = a.anc ? a.anc[a.r0 + min(qi, QR - 1) / G] : ~0ull;
  float mx = -INFINITY;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int key = key0 + key_of(ks, 4 * lg + e);
      // key <= lim keeps the shift below the row index (< 64 for tree rows)
      const bool off_path = a.anc && key >= a.pos0 && key <= lim && !((am >> ((key - a.pos0) & 63)) & 1ull);
      if (key > lim || key >= nkeys || off_path) sc[ks][e] = -INFINITY;
      mx = fmaxf(mx, sc[ks][e]);
    }
  // the query's other keys sit in lanes lr + 16 j; the butterfly gives all four the same value
  mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
  mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
  float sm = 0.f;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float p = sc[ks][e] == -INFINITY ? 0.f : expf(sc[ks][e] - mx);
      sc[ks][e] = p;
      sm += p;
    }
  sm += __shfl_xor(sm, 16, WAVE);
  sm += __shfl_xor(sm, 32, WAVE);
  if (lg == 0) Ml[wave][lr] = make_float2(mx, sm);
  // zero the V elements of keys >= nkeys (their P is 0, but the cache past the
  // committed rows may hold anything)
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const int kb = key0 + kt * F::KSTEP + lg * KPL;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vf[kt][dt] = F::mask_from(vf[kt][dt], nkeys - kb);
  }
  // O^T = V^T P^T: the B operand of key step kt is this lane's own P of keys
  // KSTEP kt + KPL lg + j, i.e. scores v = KPL kt + j (tile v / 4, row v % 4)
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    float ph[KPL], pl[KPL];
#pragma unroll
    for (int j = 0; j < KPL; ++j) {
      const int v = KPL * kt + j;
      ph[j] = sc[v >> 2][v & 3];
      pl[j] = ph[j] - to_f<WT>(from_f<WT>(ph[j]));
    }
    const frag bh = F::pack(ph);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = F::mma(vf[kt][dt], bh, o[dt]);
    if constexpr (SPLIT) {
      const frag bl = F::pack(pl);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] = F::mma(vf[kt][dt], bl, o[dt]);
    }
  }
  __syncthreads();  // Ml of every wave
  // merge the four waves: rescale to the block maximum of each query; lane holds
  // O[query lr][16 dt + 4 lg + e]
  {
    float mb = -INFINITY;
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) mb = fmaxf(mb, Ml[w][lr].x);
    const float f = mx == -INFINITY ? 0.f : expf(mx - mb);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(&Ob[wave][lr][16 * dt + 4 * lg]) =
          make_float4(o[dt][0] * f, o[dt][1] * f, o[dt][2] * f, o[dt][3] * f);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 16 * HD; e += 256) {
    const int row = e / HD, dim = e - row * HD;
    const int qr = 16 * qt + row;
    if (qr >= QR) continue;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) v += Ob[w][row][dim];
    st_coh(a.po + (((size_t)h * QR + qr) * a.nch + c) * HD + dim, v);
  }
  if (threadIdx.x < 16) {
    const int row = threadIdx.x, qr = 16 * qt + row;
    if (qr < QR) {
      float mb = -INFINITY;
#pragma unroll
      for (int w = 0; w < ATT_WAVES; ++w) mb = fmaxf(mb, Ml[w][row].x);
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < ATT_WAVES; ++w)
        if (Ml[w][row].x > -INFINITY) L += Ml[w][row].y * expf(Ml[w][row].x - mb);
      float* ml = reinterpret_cast<float*>(a.pml + ((size_t)h * QR + qr) * a.nch + c);
      st_coh(ml, mb);
      st_coh(ml + 1, L);
    }
  }
  // the last chunk block of (kv head, query tile) merges the chunk partials of its rows
  const int nchunk_tile = min(a.nch, (qpos0 + r_last) / ATT_KC + 1);
  if (!arrive_last(a.counters + h * a.nqt + qt, (unsigned)nchunk_tile)) {
    return;
  }
  // chunk weights exp(m_c - max) of each row: 16 threads per row, chunks strided
  __shared__ float s_w[16][ATT_MAXCH];
  __shared__ float s_L[16];
  {
    constexpr int CPT = ATT_MAXCH / 16;  // chunks per thread at most
    const int row = threadIdx.x >> 4, j = threadIdx.x & 15;
    const int qr = 16 * qt + row;
    const int nv = qr < QR ? (qpos0 + qr / G) / ATT_KC + 1 : 0;
    const uint64_t* ml = reinterpret_cast<const uint64_t*>(a.pml + ((size_t)h * QR + (qr < QR ? qr : 0)) * a.nch);
    float2 v[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cc = j + 16 * i;
      const float2 t = __builtin_bit_cast(float2, ld_coh_u64(ml + (cc < nv ? cc : 0)));
      v[i] = cc < nv ? t : make_float2(-INFINITY, 0.f);
    }
    float mmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < CPT; ++i) mmax = fmaxf(mmax, v[i].x);
    mmax = row16_max(mmax);
    float L = 0.f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      const int cc = j + 16 * i;
      const float wgt = cc < nv ? expf(v[i].x - mmax) : 0.f;
      s_w[row][cc] = wgt;
      L += v[i].y * wgt;
    }
    L = row16_sum(L);
    if (j == 0) s_L[row] = L;
  }
  __syncthreads();
  // output: a thread owns NI items of 4 consecutive dims of a row; the partials of up
  // to CB chunks of all its items are in flight together (one round trip for
  // contexts up to CB * ATT_KC keys)
  constexpr int D4 = HD / 4;
  constexpr int NI = (16 * D4 + 255) / 256;
  constexpr int CB = 16;
  int rowv[NI], nvv[NI], dimv[NI], qrv[NI];
  uint32_t basev[NI];
  int nvmax = 0;
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int e = threadIdx.x + 256 * ii;
    const int row = e / D4, dim = (e - row * D4) * 4;
    const int qr = 16 * qt + row;
    const bool ok = e < 16 * D4 && qr < QR;
    const int qc = ok ? qr : 16 * qt;  // a valid row of the tile for the unused items
    rowv[ii] = ok ? row : 0;
    dimv[ii] = ok ? dim : 0;
    qrv[ii] = ok ? qr : -1;
    nvv[ii] = ok ? (qpos0 + qr / G) / ATT_KC + 1 : 0;
    basev[ii] = (uint32_t)(((((size_t)h * QR + qc) * a.nch) * HD + (ok ? dim : 0)) * 4);
    nvmax = max(nvmax, nvv[ii]);
  }
  float4 acc[NI];
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) acc[ii] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < nvmax; c0 += CB) {
    float4 pv[NI][CB];
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
      for (int i = 0; i < CB; ++i)
        pv[ii][i] = ld_coh4(a.po, basev[ii] + (uint32_t)((c0 + i < nvv[ii] ? c0 + i : 0) * HD * 4));
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
      for (int i = 0; i < CB; ++i) {
        const float wgt = c0 + i < nvv[ii] ? s_w[rowv[ii]][c0 + i] : 0.f;
        acc[ii].x += pv[ii][i].x * wgt;
        acc[ii].y += pv[ii][i].y * wgt;
        acc[ii].z += pv[ii][i].z * wgt;
        acc[ii].w += pv[ii][i].w * wgt;
      }
  }
  const XSplit<WT> xo{static_cast<WT*>(a.xh), static_cast<WT*>(a.xl), a.xld};
#pragma unroll
  for (int ii = 0; ii < NI; ++ii) {
    const int qr = qrv[ii];
    if (qr < 0) continue;
    const float il = 1.0f / s_L[rowv[ii]];
    xo.put4(qr / G, (h * G + qr % G) * HD + dimv[ii],
            make_float4(acc[ii].x * il, acc[ii].y * il, acc[ii].z * il, acc[ii].w * il));
  }
}

// ---------------------------------------------------------------------------
// Prefill-sized steps (bf16, M >= 256, hd = 128): the four products of a layer
// run on the large-M MFMA GEMM and write fp32 rows; the row kernels below apply
// what the decode path's GEMM epilogues do.
// ---------------------------------------------------------------------------
constexpr int PDM_BIG_MIN_M = 256;

// block sum of a value every thread holds (256 threads)
__device__ __forceinline__ float block_sum256(float v) {
  __shared__ float s_part[4];
  v = wave_sum(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = v;
  __syncthreads();
  return (s_part[0] + s_part[1]) + (s_part[2] + s_part[3]);
}

// four values as bf16 hi parts at p and the lo parts (v - hi) at p + K
__device__ __forceinline__ void put4_hilo(bf16* p, int K, float4 v) {
  const uint32_t h0 = pack2_bf16(v.x, v.y), h1 = pack2_bf16(v.z, v.w);
  const uint32_t l0 = pack2_bf16(v.x - __uint_as_float(h0 << 16), v.y - __uint_as_float(h0 & 0xffff0000u));
  const uint32_t l1 = pack2_bf16(v.z - __uint_as_float(h1 << 16), v.w - __uint_as_float(h1 & 0xffff0000u));
  *reinterpret_cast<uint2*>(p) = make_uint2(h0, h1);
  *reinterpret_cast<uint2*>(p + K) = make_uint2(l0, l1);
}

// four values as bf16 hi parts at p and their lo8 bytes (e4m3 of 256 (v - hi)) at q
__device__ __forceinline__ void put4_hilo8(bf16* p, unsigned char* q, float4 v) {
  const uint32_t h0 = pack2_bf16(v.x, v.y), h1 = pack2_bf16(v.z, v.w);
  *reinterpret_cast<uint2*>(p) = make_uint2(h0, h1);
  *reinterpret_cast<uint32_t*>(q) =
      lo8_word(v.x - __uint_as_float(h0 << 16), v.y - __uint_as_float(h0 & 0xffff0000u),
               v.z - __uint_as_float(h1 << 16), v.w - __uint_as_float(h1 & 0xffff0000u));
}

// A row of the next large-M product's input: [hi | lo] (2d bf16), or with LO8
// [hi | lo8] (d bf16 hi parts, then d lo8 bytes: 3d bytes); with LO8 row M - 1 also
// goes to xlast as [hi | lo] (the output row's query product on the decode kernels).
template <bool LO8>
__device__ __forceinline__ void put4_row(bf16* xa, bf16* xlast, int r, int M, int d, int c, float4 v) {
  if constexpr (LO8) {
    bf16* row = xa + (size_t)r * (3 * d / 2);
    put4_hilo8(row + c, reinterpret_cast<unsigned char*>(row + d) + c, v);
    if (r == M - 1) put4_hilo(xlast + c, d, v);
  } else {
    put4_hilo(xa + (size_t)r * 2 * d + c, d, v);
  }
}

// h = g, the row's 1/rms, the first QKV input g * attn_norm as a row of the next
// product's input (put4_row), and the rotate-half RoPE table of the row's position
// (fp64 angles)
template <typename WT, bool LO8>
__global__ __launch_bounds__(256) void big_rows_init_kernel(const float* g, float* h, float* rs, WT* xa,
                                                            const WT* gamma, float2* rope, int d, int pos0,
                                                            int hd, float theta, float eps, WT* xlast, int M) {
  const int r = blockIdx.x;
  if (threadIdx.x < hd / 2) {
    double sn, cs;
    sincos((double)(pos0 + r) * pow((double)theta, -2.0 * threadIdx.x / hd), &sn, &cs);
    rope[(size_t)r * (hd / 2) + threadIdx.x] = make_float2((float)cs, (float)sn);
  }
  float sq = 0.f;
  for (int c = 4 * threadIdx.x; c < d; c += 4 * 256) {
    const size_t i = (size_t)r * d + c;
    const float4 v = *reinterpret_cast<const float4*>(g + i);
    *reinterpret_cast<float4*>(h + i) = v;
    sq += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
    put4_row<LO8>(xa, xlast, r, M, d, c,
                  make_float4(v.x * to_f<WT>(gamma[c]), v.y * to_f<WT>(gamma[c + 1]), v.z * to_f<WT>(gamma[c + 2]),
                              v.w * to_f<WT>(gamma[c + 3])));
  }
  const float t = block_sum256(sq);
  if (threadIdx.x == 0) rs[r] = 1.0f / sqrtf(t / (float)d + eps);
}

// q and k heads of one row: per-head RMSNorm with q_norm / k_norm, rotate-half
// RoPE (element i pairs with i + 64), q to the attention buffer, k to the cache.
template <typename WT>
__global__ __launch_bounds__(64) void qk_post_kernel(const float* C, int ldc, float* qbuf, WT* kc, const WT* qn,
                                                     const WT* kn, const float2* rope, int Hq, int pos0,
                                                     int64_t T_cap, float eps) {
  const int hh = blockIdx.x, r = blockIdx.y, lane = threadIdx.x;
  const float* y = C + (size_t)r * ldc + hh * 128;
  float v0 = y[lane], v1 = y[lane + 64];
  const WT* nw = hh < Hq ? qn : kn;
  const float inv = 1.0f / sqrtf(wave_sum(v0 * v0 + v1 * v1) / 128.f + eps);
  v0 *= inv * to_f<WT>(nw[lane]);
  v1 *= inv * to_f<WT>(nw[lane + 64]);
  const float2 cs = rope[(size_t)r * 64 + lane];
  const float x1 = v0, x2 = v1;
  v0 = x1 * cs.x - x2 * cs.y;
  v1 = x2 * cs.x + x1 * cs.y;
  if (hh < Hq) {
    float* qp = qbuf + ((size_t)r * Hq + hh) * 128;
    qp[lane] = v0;
    qp[lane + 64] = v1;
  } else {
    WT* kp = kc + ((size_t)(hh - Hq) * T_cap + pos0 + r) * 128;
    kp[lane] = from_f<WT>(v0);
    kp[lane + 64] = from_f<WT>(v1);
  }
}

// v heads into the position-minor cache [Hkv][hd][T_cap]: a block writes 64
// consecutive positions of every dimension of one head.
template <typename WT>
__global__ __launch_bounds__(256) void v_post_kernel(const float* C, int ldc, WT* vc, int col0, int pos0,
                                                     int64_t T_cap, int M) {
  const int vh = blockIdx.x, r = blockIdx.y * 64 + (threadIdx.x & 63);
  if (r >= M) return;
  const float* y = C + (size_t)r * ldc + col0 + vh * 128;
  WT* vp = vc + (size_t)vh * 128 * T_cap + pos0 + r;
  for (int dim = threadIdx.x >> 6; dim < 128; dim += 4) vp[(size_t)dim * T_cap] = from_f<WT>(y[dim]);
}

// h += y, the row's 1/rms and the next GEMM's input h * gnext (put4_row)
template <typename WT, bool LO8>
__global__ __launch_bounds__(256) void resid_post_kernel(const float* C, int ldc, float* h, float* rs, WT* xa,
                                                         const WT* gnext, int d, float eps, WT* xlast, int M) {
  const int r = blockIdx.x;
  float sq = 0.f;
  for (int c = 4 * threadIdx.x; c < d; c += 4 * 256) {
    const size_t i = (size_t)r * d + c;
    float4 v = *reinterpret_cast<const float4*>(h + i);
    const float4 y = *reinterpret_cast<const float4*>(C + (size_t)r * ldc + c);
    v.x += y.x;
    v.y += y.y;
    v.z += y.z;
    v.w += y.w;
    *reinterpret_cast<float4*>(h + i) = v;
    sq += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
    put4_row<LO8>(xa, xlast, r, M, d, c,
                  make_float4(v.x * to_f<WT>(gnext[c]), v.y * to_f<WT>(gnext[c + 1]), v.z * to_f<WT>(gnext[c + 2]),
                              v.w * to_f<WT>(gnext[c + 3])));
  }
  const float t = block_sum256(sq);
  if (threadIdx.x == 0) rs[r] = 1.0f / sqrtf(t / (float)d + eps);
}


// Causal attention for prefill-sized steps (bf16, hd = 128), flash style: a block
// owns 64 of a kv head's GQA query rows (query index qi = row * G + head in the
// group, as in the decode kernel) and walks the keys in blocks of 64 up to its
// causal limit.  Per key block the K tile (key-major) and the V tile (from the
// position-minor cache, dimension-major) are staged in LDS; the next block's tiles
// are loaded into registers while the current one is multiplied.  Each wave owns
// 16 queries and computes S^T = K Q^T on MFMA (Q as bf16 hi + lo pairs, the B
// operand), keeps a running maximum and sum per query, and accumulates
// O^T += V^T P^T (P rounded to bf16).  The K rows of S^T tile ks are read in the
// order key(ks, r) = 32 (ks / 2) + 8 (r / 4) + 4 (ks % 2) + r % 4: the lane that
// holds query c of tile rows 4 g .. 4 g + 3 then holds that query's keys
// 8 g .. 8 g + 7 (tiles 0, 1) and 32 + 8 g .. + 7 (tiles 2, 3), which is exactly
// its B operand of the P^T V^T product, so P never leaves the registers.  The
// output is written once, as the O projection's [hi | lo] input rows.
constexpr int FA_KB = 64;               // keys per step
constexpr int FA_ROWS = 64;             // query rows per block (16 per wave)
constexpr int FA_KSTR = 128 + 8;        // padded LDS row strides (bf16 elements)
constexpr int FA_VSTR = FA_KB + 8;

struct FlashArgs {
  const float* q;  // [M][Hq][128]
  const bf16* kc;  // [Hkv][T_cap][128] of this layer
  const bf16* vc;  // [Hkv][128][T_cap]
  bf16* xh;        // output hi parts, row stride xld
  bf16* xl;        // output lo parts
  int xld;
  int M, Hq, Hkv, pos0, nqt;
  int64_t T_cap;
  float scale;
};

__global__ __launch_bounds__(256) void attn_flash_kernel(FlashArgs a) {
  typedef Mfma<bf16> F;
  typedef F::frag frag;
  __shared__ __align__(16) bf16 Ks[FA_KB * FA_KSTR];
  __shared__ __align__(16) bf16 Vs[128 * FA_VSTR];
  const int h = blockIdx.y;
  const int qt = a.nqt - 1 - blockIdx.x;  // the longest (latest) tiles start first
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lr = lane & 15, lg = lane >> 4;
  const int G = a.Hq / a.Hkv, QR = a.M * G;
  const int nkeys = a.pos0 + a.M;
  const int r_last = (min(QR, FA_ROWS * qt + FA_ROWS) - 1) / G;  // last position of the tile
  const int nkb = (a.pos0 + r_last) / FA_KB + 1;
  const bf16* K = a.kc + (size_t)h * a.T_cap * 128;
  const bf16* Vt = a.vc + (size_t)h * 128 * a.T_cap;

  // Q fragments of this lane's query (B operand), pre-scaled, as hi + lo pairs
  const int qi = FA_ROWS * qt + 16 * wave + lr;
  const bool qv = qi < QR;
  const float* qp = a.q + ((size_t)(qv ? qi / G : 0) * a.Hq + h * G + (qv ? qi % G : 0)) * 128;
  frag qf[4], ql[4];
  {
    const float qs = qv ? a.scale : 0.f;
#pragma unroll
    for (int ds = 0; ds < 4; ++ds) {
      const float4 x0 = *reinterpret_cast<const float4*>(qp + ds * 32 + lg * 8);
      const float4 x1 = *reinterpret_cast<const float4*>(qp + ds * 32 + lg * 8 + 4);
      float tmp[8] = {x0.x * qs, x0.y * qs, x0.z * qs, x0.w * qs, x1.x * qs, x1.y * qs, x1.z * qs, x1.w * qs};
      float rem[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) rem[e] = tmp[e] - to_f<bf16>(from_f<bf16>(tmp[e]));
      qf[ds] = F::pack(tmp);
      ql[ds] = F::pack(rem);
    }
  }
  const int lim = a.pos0 + (qv ? qi / G : 0);  // causal limit of this lane's query
  float mrow = -INFINITY, lrow = 0.f;
  f32x4 o[8];  // O^T: lane holds O[query][16 dt + 4 lg + e]
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The K and V tiles of key block kb + 1 are loaded into registers while block kb
  // is multiplied (unconditionally: the last block is loaded again at the end).
  u32x4 kreg[4], vreg[4];  // native vectors: an array of HIP's uint4 structs is kept in memory
  auto load_tiles = [&](int key0) {
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int idx = pass * 256 + threadIdx.x;
      // K: row = key, 16 chunks of 8 dims; keys past the cache end read its last row
      const int kr = idx >> 4, kc = idx & 15;
      const int key = min(key0 + kr, (int)a.T_cap - 1);
      kreg[pass] = *reinterpret_cast<const u32x4*>(K + (size_t)key * 128 + kc * 8);
      // V: row = dimension, 8 chunks of 8 keys; keys past the last written one are zeroed
      const int vr = idx >> 3, vcn = idx & 7;
      const int kk = key0 + vcn * 8;
      vreg[pass] = *reinterpret_cast<const u32x4*>(Vt + (size_t)vr * a.T_cap + min(kk, (int)a.T_cap - 8));
    }
  };
  load_tiles(0);
  for (int kb = 0; kb < nkb; ++kb) {
    const int key0 = kb * FA_KB;
    __syncthreads();  // the previous tiles are consumed
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int idx = pass * 256 + threadIdx.x;
      const int kr = idx >> 4, kc = idx & 15;
      *reinterpret_cast<u32x4*>(Ks + kr * FA_KSTR + kc * 8) = kreg[pass];
      const int vr = idx >> 3, vcn = idx & 7;
      *reinterpret_cast<uint4*>(Vs + vr * FA_VSTR + vcn * 8) =
          F::mask_from(__builtin_bit_cast(uint4, vreg[pass]), nkeys - (key0 + vcn * 8));
    }
    __syncthreads();
    load_tiles(min(kb + 1, nkb - 1) * FA_KB);
    // S^T = K Q^T: tile ks, lane holds S^T[key(ks, 4 lg + e)][lr]
    f32x4 sc[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int kr = 32 * (ks >> 1) + 8 * (lr >> 2) + 4 * (ks & 1) + (lr & 3);  // key(ks, lr)
      sc[ks] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ds = 0; ds < 4; ++ds) {
        const frag kf = *reinterpret_cast<const frag*>(Ks + kr * FA_KSTR + ds * 32 + lg * 8);
        sc[ks] = F::mma(kf, qf[ds], sc[ks]);
        sc[ks] = F::mma(kf, ql[ds], sc[ks]);
      }
    }
    // online softmax of this lane's query: its 16 keys, then the 3 other lanes of
    // the query (lanes lr + 16 j); the butterfly gives all four the same sums
    float mx = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = key0 + 32 * (ks >> 1) + 8 * lg + 4 * (ks & 1) + e;
        if (key > lim) sc[ks][e] = -INFINITY;
        mx = fmaxf(mx, sc[ks][e]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, WAVE));
    mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
    const float mnew = fmaxf(mrow, mx);  // finite: key 0 is inside every query's limit
    const float scl = expf(mrow - mnew);
    float sm = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float pv = sc[ks][e] == -INFINITY ? 0.f : expf(sc[ks][e] - mnew);
        sc[ks][e] = pv;
        sm += pv;
      }
    sm += __shfl_xor(sm, 16, WAVE);
    sm += __shfl_xor(sm, 32, WAVE);
    lrow = lrow * scl + sm;
    mrow = mnew;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[dt][e] *= scl;
    // O^T += V^T P^T: the B operand of key step kt is this lane's own P of keys
    // 32 kt + 8 lg + j (tiles 2 kt and 2 kt + 1), rounded to bf16 once (P is in
    // [0, 1]; a lo part moved no cache row of the headline prefill)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float ph[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) ph[j] = sc[2 * kt + (j >> 2)][j & 3];
      const frag bh = F::pack(ph);
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const frag vf = *reinterpret_cast<const frag*>(Vs + (16 * dt + lr) * FA_VSTR + kt * 32 + lg * 8);
        o[dt] = F::mma(vf, bh, o[dt]);
      }
    }
  }
  // O / l as [hi | lo] parts: this lane's query, dimensions 16 dt + 4 lg .. + 3
  if (qv) {
    const float inv = 1.0f / lrow;
    const size_t base = (size_t)(qi / G) * a.xld + (size_t)(h * G + qi % G) * 128 + 4 * lg;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const float v0 = o[dt][0] * inv, v1 = o[dt][1] * inv, v2 = o[dt][2] * inv, v3 = o[dt][3] * inv;
      const uint32_t h01 = pack2_bf16(v0, v1), h23 = pack2_bf16(v2, v3);
      const uint32_t l01 = pack2_bf16(v0 - __uint_as_float(h01 << 16), v1 - __uint_as_float(h01 & 0xffff0000u));
      const uint32_t l23 = pack2_bf16(v2 - __uint_as_float(h23 << 16), v3 - __uint_as_float(h23 & 0xffff0000u));
      *reinterpret_cast<uint2*>(a.xh + base + 16 * dt) = make_uint2(h01, h23);
      *reinterpret_cast<uint2*>(a.xl + base + 16 * dt) = make_uint2(l01, l23);
    }
  }
}

struct PdmPlan {
  GemmPlan qkv, o, gu, down;
  int nch, QR;
  size_t off_h, off_ss, off_q, off_rope, off_po, off_pml, off_x0h, off_x0l, off_x1h, off_x1l, off_part, total;
  int ld1;  // row stride of the second XSplit buffer
  size_t part_bytes;  // split-K partials of the decode-shaped products
  // large-M path
  bool big;
  BigPlan bqkv, bkv, bo, bgu, bdown;  // bkv: the key/value columns of W_qkv only
  size_t off_C, off_rs, off_bpart, off_xa, off_xb;
  // the same products with [hi | lo8] inputs (prepared e4m3 weights), and the output
  // row's [hi | lo] copy for its query product
  bool big8;
  BigPlan b8qkv, b8kv, b8gu, b8down;
  size_t off_xlast;
};

// Prepared e4m3 copies (spd_pdm_prepare) of the weights of the products that take
// [hi | lo] inputs on the large-M path: per layer W_qkv, W_gate_up and W_down as
// [rows][K] bytes, then their per-row E8M0 scale bytes, each 256-byte aligned.
struct PrepLayout {
  size_t qkv8, gu8, dn8, qkv_s, gu_s, dn_s, layer_bytes, total;
};
static PrepLayout prep_layout(const spd_config* c) {
  PrepLayout L{};
  const size_t nq = (size_t)(c->Hq + 2 * c->Hkv) * c->hd, d = c->d, dff = c->dff;
  size_t off = 0;
  auto take = [&](size_t b) { size_t r = off; off = align256(off + b); return r; };
  L.qkv8 = take(nq * d);
  L.gu8 = take(2 * dff * d);
  L.dn8 = take(d * dff);
  L.qkv_s = take(nq);
  L.gu_s = take(2 * dff);
  L.dn_s = take(d);
  L.layer_bytes = off;
  L.total = off * (size_t)c->Ls;
  return L;
}
// the configurations whose large-M products take prepared weights
static bool prep_supported(const spd_config* c) {
  return c->dtype == SPD_BF16 && c->hd == 128 && c->d % 128 == 0 && c->dff % 128 == 0;
}

// Products of the large-M step that take the activations as bf16 hi + lo pairs
// (bit i: QKV, O, gate/up, down); the others take the bf16-rounded activations.
// Measured on the 2039-row headline prefill against the fp64 oracle (max error /
// rms): every product rounded once gives keys 0.0217-0.0235, QKV alone in hi + lo
// still 0.0203 on the second layer's keys, gate/up in hi + lo is what brings them
// to 0.0157; the O projection's lo half moves no tensor by more than 0.0004.
constexpr int PDM_BIG_LO = 0xD;
static inline int big_k(int prod, int K) { return ((PDM_BIG_LO >> prod) & 1) ? 2 * K : K; }
// With prepared weights exactly these products (QKV, gate/up, down) take [hi | lo8] rows.
static_assert(PDM_BIG_LO == 0xD, "the lo8 form covers QKV, gate/up and down");

// The decode-shaped products for M rows.  Grid targets measured at the 2560-wide
// shape: about one block per CU for the products over the hidden size, two for the
// down projection (rows of dff).
struct RowPlans {
  GemmPlan qkv, o, gu, down;
};
static RowPlans plan_rows(const spd_config* c, int M) {
  const bool bf = c->dtype == SPD_BF16;
  const int ks = bf ? Mfma<bf16>::KSTEP : Mfma<float>::KSTEP;
  const int es = bf ? 2 : 4;
  RowPlans r;
  r.qkv = plan_gemm((c->Hq + 2 * c->Hkv) * c->hd, c->d, M, ks, es, 2, 256);
  r.o = plan_gemm(c->d, c->Hq * c->hd, M, ks, es, 1, 256);
  r.gu = plan_gemm(2 * c->dff, c->d, M, ks, es, 2, 256);
  r.down = plan_gemm(c->d, c->dff, M, ks, es, 1, 512);
  return r;
}

// the query heads of one row (the first Hq hd rows of W_qkv)
static GemmPlan plan_q_row(const spd_config* c) {
  const bool bf = c->dtype == SPD_BF16;
  return plan_gemm(c->Hq * c->hd, c->d, 1, bf ? Mfma<bf16>::KSTEP : Mfma<float>::KSTEP, bf ? 2 : 4, 2, 256);
}

// split-K partial floats of the O, gate/up and down products over M rows
static size_t tail_part_bytes(const spd_config* c, const RowPlans& r, int M) {
  size_t b = 0;
  if (r.o.S > 1) b = std::max(b, (size_t)r.o.S * M * c->d * 4);
  if (r.gu.S > 1) b = std::max(b, (size_t)r.gu.S * M * 2 * c->dff * 4);
  if (r.down.S > 1) b = std::max(b, (size_t)r.down.S * M * c->d * 4);
  return b;
}

static PdmPlan plan_pdm(const spd_config* c, int M, int64_t T_cap) {
  PdmPlan p;
  const bool bf = c->dtype == SPD_BF16;
  const int es = bf ? 2 : 4;
  {
    const RowPlans r = plan_rows(c, M);
    p.qkv = r.qkv;
    p.o = r.o;
    p.gu = r.gu;
    p.down = r.down;
  }
  p.nch = (int)((T_cap + ATT_KC - 1) / ATT_KC);
  p.QR = M * (c->Hq / c->Hkv);
  size_t off = SPD_WS_COUNTER_BYTES;
  auto take = [&](size_t bytes) { size_t r = off; off = align256(off + bytes); return r; };
  p.off_h = take((size_t)M * c->d * 4);
  p.off_ss = take((size_t)(c->d / 64) * M * 4);
  p.off_q = take((size_t)M * c->Hq * c->hd * 4);
  p.off_rope = take((size_t)M * (c->hd / 2) * 8);
  p.off_po = take((size_t)c->Hkv * p.QR * p.nch * c->hd * 4);
  p.off_pml = take((size_t)c->Hkv * p.QR * p.nch * 8);
  // XSplit GEMM inputs: x0 feeds QKV and gate/up (width d), x1 feeds O and down
  p.ld1 = std::max(c->Hq * c->hd, c->dff);
  p.off_x0h = take((size_t)M * c->d * es);
  p.off_x0l = take((size_t)M * c->d * es);
  p.off_x1h = take((size_t)M * p.ld1 * es);
  p.off_x1l = take((size_t)M * p.ld1 * es);
  size_t part = 0;
  const GemmPlan* gps[4] = {&p.qkv, &p.o, &p.gu, &p.down};
  const size_t Ns[4] = {(size_t)(c->Hq + 2 * c->Hkv) * c->hd, (size_t)c->d, (size_t)2 * c->dff,
                        (size_t)c->d};
  for (int i = 0; i < 4; ++i)
    if (gps[i]->S > 1) part = std::max(part, (size_t)gps[i]->S * M * Ns[i] * 4);
  // the one-row tail of the last layer (the chain's h_last) and, on the large-M
  // path, the output row's query product
  part = std::max(part, tail_part_bytes(c, plan_rows(c, 1), 1));
  {
    const GemmPlan q1 = plan_q_row(c);
    if (q1.S > 1) part = std::max(part, (size_t)q1.S * c->Hq * c->hd * 4);
  }
  p.part_bytes = part;
  p.off_part = take(part);
  p.big = bf && M >= PDM_BIG_MIN_M && c->hd == 128;
  p.big8 = false;
  p.off_xlast = 0;
  if (p.big) {
    // activations enter as [hi | lo] rows; a product in PDM_BIG_LO runs over all 2K
    // columns, the others over the K hi columns only
    const int nq = (c->Hq + 2 * c->Hkv) * c->hd;
    p.bqkv = plan_big_gemm(M, nq, big_k(0, c->d));
    p.bkv = plan_big_gemm(M, 2 * c->Hkv * c->hd, big_k(0, c->d));
    p.bo = plan_big_gemm(M, c->d, big_k(1, c->Hq * c->hd));
    p.bgu = plan_big_swiglu(M, c->dff, big_k(2, c->d));
    p.bdown = plan_big_gemm(M, c->d, big_k(3, c->dff));
    p.big = p.bqkv.use && p.bkv.use && p.bo.use && p.bgu.use && p.bdown.use;
  }
  if (p.big) {
    const int nq = (c->Hq + 2 * c->Hkv) * c->hd;
    p.off_C = take((size_t)M * std::max(nq, c->d) * 4);  // gate/up writes its activations directly
    p.off_rs = take((size_t)M * 4);
    p.off_xa = take((size_t)M * 2 * c->d * 2);
    p.off_xb = take((size_t)M * 2 * p.ld1 * 2);
    p.big8 = prep_supported(c);
    if (p.big8) {
      p.b8qkv = plan_big_lo8(M, nq, c->d);
      p.b8kv = plan_big_lo8(M, 2 * c->Hkv * c->hd, c->d);
      p.b8gu = plan_big_swiglu_lo8(M, c->dff, c->d);
      p.b8down = plan_big_lo8(M, c->d, c->dff);
      p.big8 = p.b8qkv.use && p.b8kv.use && p.b8gu.use && p.b8down.use;
    }
    size_t bp = std::max(std::max(std::max(p.bqkv.part_bytes, p.bkv.part_bytes), p.bo.part_bytes),
                         std::max(p.bgu.part_bytes, p.bdown.part_bytes));
    if (p.big8)
      bp = std::max(bp, std::max(std::max(p.b8qkv.part_bytes, p.b8kv.part_bytes),
                                 std::max(p.b8gu.part_bytes, p.b8down.part_bytes)));
    p.off_bpart = take(bp);
    p.off_xlast = take((size_t)2 * c->d * 2);
  }
  p.total = off;
  return p;
}

size_t pdm_workspace(const spd_config* cfg, int M, int64_t T_cap) {
  return plan_pdm(cfg, M, T_cap).total;
}

static GemmShape shape_of(const GemmPlan& gp, const void* W, int N, int K, int M, float* part,
                          unsigned* ctr, const float* rs_ss = nullptr, int rs_P = 0, float eps = 0.f) {
  GemmShape g{};
  g.rs_ss = rs_ss;
  g.rs_P = rs_P;
  g.rs_M = M;
  g.rs_K = K;
  g.rs_eps = eps;
  g.W = W;
  g.N = N;
  g.K = K;
  g.M = M;
  g.S = gp.S;
  g.nsteps = gp.nsteps;
  g.ldx = gp.ldx;
  g.part = part;
  g.nblocks = gp.nblocks;
  g.counters = ctr;
  return g;
}

template <typename WT, int HD>
static int launch_attention(const AttnArgs& aa, hipStream_t st) {
  if constexpr (HD % Mfma<WT>::KSTEP != 0) {
    return SPD_E_UNSUPPORTED;  // head dim below one MFMA k-step of this dtype
  } else {
    hipLaunchKernelGGL((attn_partial_kernel<WT, HD>), dim3(aa.nch, aa.Hkv, aa.nqt), dim3(256), 0, st,
                       aa);
    return check_launch();
  }
}

// Attention, O projection, gate/up and down of one layer for the query rows
// r0 .. M-1, once the layer's QKV product has put the keys and values of all M
// rows in the cache and their queries in the attention buffer.  Rows r0 .. M-1 of
// h are updated in place; x0, x1 and the row statistics hold them from local row
// 0.  The last layer (next == null) final-norms local rows Mq - n_out .. Mq - 1
// into h_last, Mq = M - r0.  P returns the partial count of the row statistics
// the down projection leaves for the next layer's QKV product.
template <typename WT>
static int layer_rows(const spd_config* c, const PdmPlan& p, const spd_layer_weights& lw,
                      const spd_layer_weights* next, const void* final_norm, int M, int r0, int n_out,
                      float* h_last, char* w, AttnArgs aa, int& P, hipStream_t st) {
  const int d = c->d, hd = c->hd, Hq = c->Hq, dff = c->dff;
  const int Mq = M - r0;
  const RowPlans rp = r0 == 0 ? RowPlans{p.qkv, p.o, p.gu, p.down} : plan_rows(c, Mq);
  float* h = reinterpret_cast<float*>(w + p.off_h) + (size_t)r0 * d;
  float* ss = reinterpret_cast<float*>(w + p.off_ss);
  float* part = reinterpret_cast<float*>(w + p.off_part);
  unsigned* ctr = reinterpret_cast<unsigned*>(w);
  const XSplit<WT> x0{reinterpret_cast<WT*>(w + p.off_x0h), reinterpret_cast<WT*>(w + p.off_x0l), d};
  const XSplit<WT> x1{reinterpret_cast<WT*>(w + p.off_x1h), reinterpret_cast<WT*>(w + p.off_x1l), p.ld1};
  const XSplit<WT> none{nullptr, nullptr, 0};
  int rc;
  // attention -> x1
  aa.r0 = r0;
  aa.nqt = (Mq * (Hq / c->Hkv) + 15) / 16;
  switch (hd) {
    case 16: rc = launch_attention<WT, 16>(aa, st); break;
    case 32: rc = launch_attention<WT, 32>(aa, st); break;
    case 64: rc = launch_attention<WT, 64>(aa, st); break;
    default: rc = launch_attention<WT, 128>(aa, st); break;
  }
  if (rc) return rc;
  // O projection + residual; x0 = h * mlp_norm
  {
    InSplit<WT> in{x1.hi, x1.lo, p.ld1};
    EpiResid<WT> epi{h, ss, d, Mq, 0, nullptr, nullptr, ctr + CTR_FINAL, rp.o.nblocks, c->rms_eps,
                     x0, static_cast<const WT*>(lw.mlp_norm)};
    rc = launch_gemm<WT, 1>(rp.o, shape_of(rp.o, lw.wo, d, Hq * hd, Mq, part, ctr), in, epi,
                            RowMapStd{}, st);
    if (rc) return rc;
  }
  // gate/up + silu*mul -> x1; row scale = 1 / rms(h)
  {
    InSplit<WT, RS_SS> in{x0.hi, x0.lo, d};
    EpiSilu<WT> epi{x1, dff};
    rc = launch_gemm<WT, 2>(rp.gu, shape_of(rp.gu, lw.w_gate_up, 2 * dff, d, Mq, part, ctr, ss,
                                            rp.o.nblocks, c->rms_eps),
                            in, epi, RowMapGateUp{dff}, st);
    if (rc) return rc;
  }
  // down + residual; x0 = h * next attn_norm; after the last layer h_last
  {
    InSplit<WT> in{x1.hi, x1.lo, p.ld1};
    const bool last = next == nullptr;
    EpiResid<WT> epi{h, ss, d, Mq, last ? 1 : 0, static_cast<const WT*>(final_norm), h_last,
                     ctr + CTR_FINAL, rp.down.nblocks, c->rms_eps, last ? none : x0,
                     last ? nullptr : static_cast<const WT*>(next->attn_norm), n_out};
    rc = launch_gemm<WT, 1>(rp.down, shape_of(rp.down, lw.w_down, d, dff, Mq, part, ctr), in, epi,
                            RowMapStd{}, st);
    if (rc) return rc;
    P = rp.down.nblocks;
  }
  return SPD_OK;
}

// First query row of the last layer: only the rows that are final-normed into the
// output need that layer's attention, O projection and MLP (the others' outputs
// feed nothing; their keys and values come from the QKV product).  Falls back to
// every row when the tail's split-K partials would not fit the workspace.
static int last_layer_r0(const spd_config* c, const PdmPlan& p, int M, int n_out) {
  const int r0 = M - n_out;
  if (r0 <= 0) return 0;
  return tail_part_bytes(c, plan_rows(c, n_out), n_out) <= p.part_bytes ? r0 : 0;
}

// Large-M step.  Buffers: xa = [hi | lo] input of QKV and gate/up (2d wide), xb =
// attention output and SwiGLU activations, C = one GEMM's fp32 output, rs = the
// row scales 1/rms(h).  The last layer runs its QKV product over every row (the
// cache needs all keys and values) and the rest for the output row only, on the
// decode-shaped kernels.
// With prepared weights (prep, lo8) the QKV, gate/up and down products take their
// inputs as [hi | lo8] rows and multiply the lo8 parts on the block-scaled fp8 MFMA.
template <bool LO8>
static int pdm_big(const spd_config* c, const spd_layer_weights* layers, const void* final_norm, void* k_cache,
                   void* v_cache, int64_t T_cap, const float* g, int pos0, int M, float* h_last, char* w,
                   const PdmPlan& p, AttnArgs aa, const unsigned char* prep, hipStream_t st) {
  typedef bf16 WT;
  const int d = c->d, hd = c->hd, Hq = c->Hq, Hkv = c->Hkv, dff = c->dff;
  const int nq = (Hq + 2 * Hkv) * hd;
  float* h = reinterpret_cast<float*>(w + p.off_h);
  float* qb = reinterpret_cast<float*>(w + p.off_q);
  float* C = reinterpret_cast<float*>(w + p.off_C);
  float* rs = reinterpret_cast<float*>(w + p.off_rs);
  float* bpart = reinterpret_cast<float*>(w + p.off_bpart);
  unsigned* ctr = reinterpret_cast<unsigned*>(w);
  WT* xa = reinterpret_cast<WT*>(w + p.off_xa);  // [M][2d]: QKV and gate/up input
  WT* xb = reinterpret_cast<WT*>(w + p.off_xb);  // [M][2 K]: O (K = Hq hd) and down (K = dff) input
  const int ko = Hq * hd;
  float2* rope = reinterpret_cast<float2*>(w + p.off_rope);
  WT* xlast = reinterpret_cast<WT*>(w + p.off_xlast);  // [hi | lo] copy of row M - 1 (LO8)
  const int lda = LO8 ? 3 * d / 2 : 2 * d;              // xa row stride (bf16 elements)
  const int ldact = LO8 ? 3 * dff / 2 : 2 * dff;        // row stride of the SwiGLU output in xb
  const PrepLayout PL = prep_layout(c);
  hipLaunchKernelGGL((big_rows_init_kernel<WT, LO8>), dim3(M), dim3(256), 0, st, g, h, rs, xa,
                     static_cast<const WT*>(layers[0].attn_norm), rope, d, pos0, hd, c->rope_theta, c->rms_eps,
                     xlast, M);
  int rc = check_launch();
  if (rc) return rc;
  for (int l = 0; l < c->Ls; ++l) {
    const spd_layer_weights& lw = layers[l];
    WT* kc = static_cast<WT*>(k_cache) + (size_t)l * Hkv * T_cap * hd;
    WT* vc = static_cast<WT*>(v_cache) + (size_t)l * Hkv * hd * T_cap;
    const unsigned char* pl = LO8 ? prep + (size_t)l * PL.layer_bytes : nullptr;
    if (l == c->Ls - 1) {
      // Last layer: every row's keys and values (the key/value columns of W_qkv on
      // the large-M GEMM), then the output row alone on the decode-shaped kernels:
      // its queries, attention, O and MLP (the other rows' outputs of this layer
      // feed nothing).
      const int nkv = 2 * Hkv * hd;
      if constexpr (LO8)
        launch_big_gemm_lo8(p.b8kv, xa, lda, static_cast<const WT*>(lw.wqkv) + (size_t)Hq * hd * d,
                            pl + PL.qkv8 + (size_t)Hq * hd * d, pl + PL.qkv_s + (size_t)Hq * hd, C, nkv, rs, M,
                            nkv, d, bpart, ctr, st);
      else
        launch_big_gemm(p.bkv, xa, 2 * d, static_cast<const WT*>(lw.wqkv) + (size_t)Hq * hd * d, C, nkv, rs, M,
                        nkv, big_k(0, d), bpart, ctr, st, d);
      // C holds key heads then value heads: no query heads in front of the keys
      hipLaunchKernelGGL((qk_post_kernel<WT>), dim3(Hkv, M), dim3(64), 0, st, C, nkv, qb, kc,
                         static_cast<const WT*>(lw.q_norm), static_cast<const WT*>(lw.k_norm), rope, 0, pos0,
                         T_cap, c->rms_eps);
      hipLaunchKernelGGL((v_post_kernel<WT>), dim3(Hkv, (M + 63) / 64), dim3(256), 0, st, C, nkv, vc, Hkv * hd,
                         pos0, T_cap, M);
      rc = check_launch();
      if (rc) return rc;
      const int r = M - 1;
      {
        const GemmPlan qp = plan_q_row(c);
        GemmShape gs = shape_of(qp, lw.wqkv, Hq * hd, d, 1, reinterpret_cast<float*>(w + p.off_part), ctr);
        gs.rs_inv = rs + r;
        const WT* xr = LO8 ? xlast : xa + (size_t)r * 2 * d;
        InSplit<WT, RS_INV> in{xr, xr + d, 2 * d};
        EpiQKV<WT> epi{qb + (size_t)r * Hq * hd, kc, vc, static_cast<const WT*>(lw.q_norm),
                       static_cast<const WT*>(lw.k_norm), rope + (size_t)r * (hd / 2), Hq, Hkv, hd, pos0 + r,
                       T_cap, c->rms_eps};
        rc = launch_gemm<WT, 2>(qp, gs, in, epi, RowMapStd{}, st);
        if (rc) return rc;
      }
      // (the workspace always holds the one-row tail's partials: r0 = M - 1)
      aa.kc = kc;
      aa.vc = vc;
      int P = 0;
      return layer_rows<WT>(c, p, lw, nullptr, final_norm, M, r, 1, h_last, w, aa, P, st);
    }
    if constexpr (LO8)
      launch_big_gemm_lo8(p.b8qkv, xa, lda, static_cast<const WT*>(lw.wqkv), pl + PL.qkv8, pl + PL.qkv_s, C, nq,
                          rs, M, nq, d, bpart, ctr, st);
    else
      launch_big_gemm(p.bqkv, xa, 2 * d, static_cast<const WT*>(lw.wqkv), C, nq, rs, M, nq, big_k(0, d), bpart,
                      ctr, st, d);
    hipLaunchKernelGGL((qk_post_kernel<WT>), dim3(Hq + Hkv, M), dim3(64), 0, st, C, nq, qb, kc,
                       static_cast<const WT*>(lw.q_norm), static_cast<const WT*>(lw.k_norm), rope, Hq, pos0,
                       T_cap, c->rms_eps);
    hipLaunchKernelGGL((v_post_kernel<WT>), dim3(Hkv, (M + 63) / 64), dim3(256), 0, st, C, nq, vc,
                       (Hq + Hkv) * hd, pos0, T_cap, M);
    rc = check_launch();
    if (rc) return rc;
    {
      FlashArgs fa;
      fa.q = qb;
      fa.kc = kc;
      fa.vc = vc;
      fa.xh = xb;  // the attention output as [hi | lo] rows of 2 Hq hd
      fa.xl = xb + ko;
      fa.xld = 2 * ko;
      fa.M = M;
      fa.Hq = Hq;
      fa.Hkv = Hkv;
      fa.pos0 = pos0;
      fa.nqt = (M * (Hq / Hkv) + FA_ROWS - 1) / FA_ROWS;
      fa.T_cap = T_cap;
      fa.scale = aa.scale;
      hipLaunchKernelGGL(attn_flash_kernel, dim3(fa.nqt, Hkv), dim3(256), 0, st, fa);
      rc = check_launch();
      if (rc) return rc;
    }
    launch_big_gemm(p.bo, xb, 2 * ko, static_cast<const WT*>(lw.wo), C, d, nullptr, M, d, big_k(1, ko), bpart, ctr,
                    st, ko);
    hipLaunchKernelGGL((resid_post_kernel<WT, LO8>), dim3(M), dim3(256), 0, st, C, d, h, rs, xa,
                       static_cast<const WT*>(lw.mlp_norm), d, c->rms_eps, xlast, M);
    if constexpr (LO8) {
      launch_big_swiglu_lo8(p.b8gu, xa, lda, static_cast<const WT*>(lw.w_gate_up), pl + PL.gu8, pl + PL.gu_s, xb,
                            ldact, dff, rs, M, d, bpart, ctr, st);
      launch_big_gemm_lo8(p.b8down, xb, ldact, static_cast<const WT*>(lw.w_down), pl + PL.dn8, pl + PL.dn_s, C, d,
                          nullptr, M, d, dff, bpart, ctr, st);
    } else {
      launch_big_swiglu(p.bgu, xa, 2 * d, static_cast<const WT*>(lw.w_gate_up), xb, 2 * dff, dff, rs, M,
                        big_k(2, d), bpart, ctr, st, d);
      launch_big_gemm(p.bdown, xb, 2 * dff, static_cast<const WT*>(lw.w_down), C, d, nullptr, M, d, big_k(3, dff),
                      bpart, ctr, st, dff);
    }
    hipLaunchKernelGGL((resid_post_kernel<WT, LO8>), dim3(M), dim3(256), 0, st, C, d, h, rs, xa,
                       static_cast<const WT*>(layers[l + 1].attn_norm), d, c->rms_eps, xlast, M);
    rc = check_launch();
    if (rc) return rc;
  }
  return SPD_E_UNSUPPORTED;  // Ls == 0 (rejected by the caller)
}

template <typename WT>
static int pdm_impl(const spd_config* c, const spd_layer_weights* layers, const void* final_norm,
                    void* k_cache, void* v_cache, int64_t T_cap, const float* g, int pos0, int M,
                    const uint64_t* anc, int n_out, float* h_last, void* ws, const void* prep,
                    hipStream_t st) {
  const PdmPlan p = plan_pdm(c, M, T_cap);
  char* w = static_cast<char*>(ws);
  float* h = reinterpret_cast<float*>(w + p.off_h);
  float* ss = reinterpret_cast<float*>(w + p.off_ss);
  float* qb = reinterpret_cast<float*>(w + p.off_q);
  float* part = reinterpret_cast<float*>(w + p.off_part);
  unsigned* ctr = reinterpret_cast<unsigned*>(w);
  const int d = c->d, hd = c->hd, Hq = c->Hq, Hkv = c->Hkv, dff = c->dff;
  const int nq = (Hq + 2 * Hkv) * hd;
  // XSplit buffers: x0 = input of QKV and gate/up, x1 = input of O and down
  const XSplit<WT> x0{reinterpret_cast<WT*>(w + p.off_x0h), reinterpret_cast<WT*>(w + p.off_x0l), d};
  const XSplit<WT> x1{reinterpret_cast<WT*>(w + p.off_x1h), reinterpret_cast<WT*>(w + p.off_x1l), p.ld1};
  const XSplit<WT> none{nullptr, nullptr, 0};

  float2* rope = reinterpret_cast<float2*>(w + p.off_rope);
  int rc;
  AttnArgs aa;
  aa.q = qb;
  aa.po = reinterpret_cast<float*>(w + p.off_po);
  aa.pml = reinterpret_cast<float2*>(w + p.off_pml);
  aa.M = M;
  aa.Hq = Hq;
  aa.Hkv = Hkv;
  aa.pos0 = pos0;
  aa.nch = (pos0 + M + ATT_KC - 1) / ATT_KC;
  aa.xh = x1.hi;
  aa.xl = x1.lo;
  aa.xld = p.ld1;
  aa.counters = ctr;
  aa.nqt = (p.QR + 15) / 16;
  aa.T_cap = T_cap;
  aa.scale = 1.0f / sqrtf((float)hd);
  aa.anc = anc;
  aa.r0 = 0;

  if constexpr (sizeof(WT) == 2) {
    if (p.big && !anc) {
      if (prep && p.big8)
        return pdm_big<true>(c, layers, final_norm, k_cache, v_cache, T_cap, g, pos0, M, h_last, w, p, aa,
                             static_cast<const unsigned char*>(prep), st);
      return pdm_big<false>(c, layers, final_norm, k_cache, v_cache, T_cap, g, pos0, M, h_last, w, p, aa, nullptr,
                            st);
    }
  }
  hipLaunchKernelGGL((rows_init_kernel<WT>), dim3(d / 64, M), dim3(64), 0, st, g, h, ss, M, d, x0,
                     static_cast<const WT*>(layers[0].attn_norm), rope, pos0, hd, c->rope_theta, anc);
  rc = check_launch();
  if (rc) return rc;
  int P = d / 64;  // partial count of ss
  for (int l = 0; l < c->Ls; ++l) {
    const spd_layer_weights& lw = layers[l];
    WT* kc = static_cast<WT*>(k_cache) + (size_t)l * Hkv * T_cap * hd;
    WT* vc = static_cast<WT*>(v_cache) + (size_t)l * Hkv * hd * T_cap;
    // QKV: x0 = h * attn_norm, row scale = 1 / rms(h)
    {
      InSplit<WT, RS_SS> in{x0.hi, x0.lo, d};
      EpiQKV<WT> epi{qb, kc, vc, static_cast<const WT*>(lw.q_norm), static_cast<const WT*>(lw.k_norm),
                     rope, Hq, Hkv, hd, pos0, T_cap, c->rms_eps};
      rc = launch_gemm<WT, 2>(p.qkv, shape_of(p.qkv, lw.wqkv, nq, d, M, part, ctr, ss, P, c->rms_eps),
                              in, epi, RowMapStd{}, st);
      if (rc) return rc;
    }
    // attention, O, MLP; the last layer only for the output rows
    aa.kc = kc;
    aa.vc = vc;
    const bool last = l == c->Ls - 1;
    rc = layer_rows<WT>(c, p, lw, last ? nullptr : &layers[l + 1], final_norm, M,
                        last ? last_layer_r0(c, p, M, n_out) : 0, n_out, h_last, w, aa, P, st);
    if (rc) return rc;
  }
  if (c->Ls == 0) return SPD_E_UNSUPPORTED;
  return SPD_OK;
}

}  // namespace spd

using namespace spd;

static int pdm_entry(const spd_config* cfg, const spd_layer_weights* layers, const void* final_norm,
                     void* k_cache, void* v_cache, int64_t T_cap, const float* g, int32_t pos0,
                     int32_t M, const uint64_t* anc, int32_t n_out, float* h_last, void* ws,
                     size_t ws_bytes, void* stream, const void* prep = nullptr) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!layers || !final_norm || !k_cache || !v_cache || !g || !h_last || !ws) return SPD_E_INVALID;
  if (cfg->Ls < 1 || cfg->Hq < 1 || cfg->Hkv < 1 || cfg->hd < 1 || cfg->dff < 1) return SPD_E_INVALID;
  if (M < 1 || pos0 < 0 || (int64_t)pos0 + M > T_cap) return SPD_E_INVALID;
  if (cfg->Hq % cfg->Hkv) return SPD_E_UNSUPPORTED;
  const int hd = cfg->hd;
  if (hd != 16 && hd != 32 && hd != 64 && hd != 128) return SPD_E_UNSUPPORTED;
  if (cfg->d % 64 || cfg->dff % 64 || T_cap % 8) return SPD_E_UNSUPPORTED;
  if (cfg->d > 8192) return SPD_E_UNSUPPORTED;  // row statistics come in <= 128 partial sums
  if (((int64_t)pos0 + M + ATT_KC - 1) / ATT_KC > ATT_MAXCH) return SPD_E_UNSUPPORTED;
  {
    const int G = cfg->Hq / cfg->Hkv;
    if ((int64_t)cfg->Hkv * ((M * G + 15) / 16) >= CTR_FINAL) return SPD_E_UNSUPPORTED;
  }
  if (((int64_t)cfg->Hq * hd) % 32) return SPD_E_UNSUPPORTED;
  for (int l = 0; l < cfg->Ls; ++l) {
    const spd_layer_weights& w = layers[l];
    if (!w.attn_norm || !w.wqkv || !w.q_norm || !w.k_norm || !w.wo || !w.mlp_norm || !w.w_gate_up ||
        !w.w_down)
      return SPD_E_INVALID;
    if (!aligned16(w.wqkv) || !aligned16(w.wo) || !aligned16(w.w_gate_up) || !aligned16(w.w_down) ||
        !aligned16(w.attn_norm) || !aligned16(w.mlp_norm) || !aligned16(w.q_norm) ||
        !aligned16(w.k_norm))
      return SPD_E_INVALID;
  }
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(ws) || !aligned16(g) ||
      !aligned16(final_norm))
    return SPD_E_INVALID;
  if (ws_bytes < pdm_workspace(cfg, M, T_cap)) return SPD_E_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (prep && (!prep_supported(cfg) || !aligned16(prep))) return SPD_E_INVALID;
  if (cfg->dtype == SPD_BF16)
    return pdm_impl<bf16>(cfg, layers, final_norm, k_cache, v_cache, T_cap, g, pos0, M, anc, n_out,
                          h_last, ws, prep, st);
  return pdm_impl<float>(cfg, layers, final_norm, k_cache, v_cache, T_cap, g, pos0, M, anc, n_out,
                         h_last, ws, nullptr, st);
}

extern "C" int spd_pdm_step(const spd_config* cfg, const spd_layer_weights* layers,
                            const void* final_norm, void* k_cache, void* v_cache, int64_t T_cap,
                            const float* g, int32_t pos0, int32_t M, float* h_last, void* ws,
                            size_t ws_bytes, void* stream) {
  return pdm_entry(cfg, layers, final_norm, k_cache, v_cache, T_cap, g, pos0, M, nullptr, 1, h_last,
                   ws, ws_bytes, stream);
}

extern "C" int spd_pdm_step_tree(const spd_config* cfg, const spd_layer_weights* layers,
                                 const void* final_norm, void* k_cache, void* v_cache,
                                 int64_t T_cap, const float* g, int32_t pos0, int32_t M,
                                 const uint64_t* anc, int32_t n_out, float* h_out, void* ws,
                                 size_t ws_bytes, void* stream) {
  if (!anc || ((uintptr_t)anc & 7) || M > SPD_TREE_MAX_NODES || n_out < 1 || n_out > M)
    return SPD_E_INVALID;
  return pdm_entry(cfg, layers, final_norm, k_cache, v_cache, T_cap, g, pos0, M, anc, n_out, h_out,
                   ws, ws_bytes, stream);
}

// e4m3 copy of weight rows with a per-row power-of-two factor: row n's largest
// magnitude m = f 2^E (0.5 <= f < 1) becomes f 2^8 in [128, 256) by 2^e, e = 8 - E
// (e = 0 for a row of zeros); s8[n] = 127 - e is the E8M0 scale that undoes the
// factor in the block-scaled MFMA.  Rows with non-finite values keep them (NaN).
__global__ __launch_bounds__(256) void fp8_rows_kernel(const bf16* W, int K, unsigned char* W8, unsigned char* s8) {
  const int n = blockIdx.x;
  const bf16* row = W + (size_t)n * K;
  float m = 0.f;
  for (int k = 8 * threadIdx.x; k < K; k += 8 * 256) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + k);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m = fmaxf(m, fmaxf(fabsf(__uint_as_float(u[i] << 16)), fabsf(__uint_as_float(u[i] & 0xffff0000u))));
  }
  __shared__ float s_m[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) s_m[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
  int e = 0;
  if (m > 0.f && m <= 3.402823466e38f) {
    int E;
    frexpf(m, &E);
    e = 8 - E;
  }
  if (threadIdx.x == 0) s8[n] = (unsigned char)(127 - e);
  for (int k = 8 * threadIdx.x; k < K; k += 8 * 256) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + k);
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float a0 = ldexpf(__uint_as_float(u[2 * i] << 16), e), a1 = ldexpf(__uint_as_float(u[2 * i] & 0xffff0000u), e);
      const float a2 = ldexpf(__uint_as_float(u[2 * i + 1] << 16), e),
                  a3 = ldexpf(__uint_as_float(u[2 * i + 1] & 0xffff0000u), e);
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
      x = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, x, true);
      o[i] = (uint32_t)x;
    }
    *reinterpret_cast<uint2*>(W8 + (size_t)n * K + k) = make_uint2(o[0], o[1]);
  }
}

extern "C" size_t spd_pdm_prepared_bytes(const spd_config* cfg) {
  if (check_config(cfg) || cfg->Ls < 1 || cfg->Hq < 1 || cfg->Hkv < 1 || !prep_supported(cfg)) return 0;
  return prep_layout(cfg).total;
}

extern "C" int spd_pdm_prepare(const spd_config* cfg, const spd_layer_weights* layers, void* prep,
                               size_t prep_bytes, void* stream) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!layers || !prep) return SPD_E_INVALID;
  if (cfg->Ls < 1 || cfg->Hq < 1 || cfg->Hkv < 1 || cfg->hd < 1 || cfg->dff < 1) return SPD_E_INVALID;
  if (!prep_supported(cfg)) return SPD_E_UNSUPPORTED;
  if (!aligned16(prep)) return SPD_E_INVALID;
  const PrepLayout L = prep_layout(cfg);
  if (prep_bytes < L.total) return SPD_E_WORKSPACE;
  for (int l = 0; l < cfg->Ls; ++l)
    if (!layers[l].wqkv || !layers[l].w_gate_up || !layers[l].w_down || !aligned16(layers[l].wqkv) ||
        !aligned16(layers[l].w_gate_up) || !aligned16(layers[l].w_down))
      return SPD_E_INVALID;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int d = cfg->d, dff = cfg->dff, nq = (cfg->Hq + 2 * cfg->Hkv) * cfg->hd;
  for (int l = 0; l < cfg->Ls; ++l) {
    unsigned char* base = static_cast<unsigned char*>(prep) + (size_t)l * L.layer_bytes;
    hipLaunchKernelGGL(fp8_rows_kernel, dim3(nq), dim3(256), 0, st, static_cast<const bf16*>(layers[l].wqkv), d,
                       base + L.qkv8, base + L.qkv_s);
    hipLaunchKernelGGL(fp8_rows_kernel, dim3(2 * dff), dim3(256), 0, st,
                       static_cast<const bf16*>(layers[l].w_gate_up), d, base + L.gu8, base + L.gu_s);
    hipLaunchKernelGGL(fp8_rows_kernel, dim3(d), dim3(256), 0, st, static_cast<const bf16*>(layers[l].w_down), dff,
                       base + L.dn8, base + L.dn_s);
    rc = check_launch();
    if (rc) return rc;
  }
  return SPD_OK;
}

extern "C" int spd_pdm_step_prepared(const spd_config* cfg, const spd_layer_weights* layers, const void* prep,
                                     size_t prep_bytes, const void* final_norm, void* k_cache, void* v_cache,
                                     int64_t T_cap, const float* g, int32_t pos0, int32_t M, float* h_last,
                                     void* ws, size_t ws_bytes, void* stream) {
  if (prep) {
    const int rc = check_config(cfg);
    if (rc) return rc;
    if (cfg->Ls < 1 || cfg->Hq < 1 || cfg->Hkv < 1 || cfg->hd < 1 || cfg->dff < 1) return SPD_E_INVALID;
    if (!prep_supported(cfg)) return SPD_E_INVALID;
    if (prep_bytes < prep_layout(cfg).total) return SPD_E_WORKSPACE;
  }
  return pdm_entry(cfg, layers, final_norm, k_cache, v_cache, T_cap, g, pos0, M, nullptr, 1, h_last, ws,
                   ws_bytes, stream, prep);
}
