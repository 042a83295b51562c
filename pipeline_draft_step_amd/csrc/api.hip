// Host helpers of the C ABI (eligibility table, cycle layout, workspace sizes,
// status strings) and spd_rollback, the end-of-cycle state transition.
#include <string.h>

#include "spd_common.h"
#include "spd_host.h"

namespace spd {

int& last_hip_error_ref() {
  static thread_local int e = 0;
  return e;
}

// One thread.  "Speculative Pipeline Decoding" (arXiv 2605.30852) section 3.4: the
// oldest in-flight token exits when the pipeline is saturated; a rejected successor
// truncates the sequence to t-n+1 and the corrected token enters stage 1; otherwise
// the new draft enters stage 1.
__global__ void rollback_kernel(spd_seq_state* st, int n, const int32_t* drafted,
                                const int32_t* n_accept, const int32_t* next_token, int32_t* tokens,
                                int64_t T_cap) {
  spd_seq_state s = *st;
  s.cycles += 1;
  if (s.a == n) {
    s.commits += 1;
    if (n_accept[0] == 0) {
      const int keep = s.t - n + 1;
      if (keep >= 0 && keep < T_cap) tokens[keep] = next_token[0];
      s.t = keep + 1;
      s.a = 1;
      *st = s;
      return;
    }
  }
  if (s.t >= 0 && s.t < T_cap) tokens[s.t] = drafted[0];
  s.t += 1;
  s.a = s.a + 1 < n ? s.a + 1 : n;
  *st = s;
}

}  // namespace spd

using namespace spd;

extern "C" int spd_slot_table(const spd_config* cfg, const int32_t* anchors, int32_t* slot_tab,
                              int32_t* store_layers, int32_t* n_store) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!anchors || !slot_tab || !store_layers || !n_store) return SPD_E_INVALID;
  const int L = cfg->L, n = cfg->n, m = cfg->m;
  if (anchors[0] != 0) return SPD_E_INVALID;
  for (int j = 1; j < m; ++j)
    if (anchors[j] <= anchors[j - 1]) return SPD_E_INVALID;
  if (anchors[m - 1] > L) return SPD_E_INVALID;
  // layer read by (depth k, slot j) for depths 0..n, -1 when the slot is empty
  int layer[SPD_MAX_STAGES + 1][SPD_MAX_ANCHORS];
  for (int k = 0; k <= n; ++k) {
    const int lmax = (int)(((int64_t)k * L) / n) < L ? (int)(((int64_t)k * L) / n) : L;
    for (int j = 0; j < m; ++j) {
      if (k == 0) {
        layer[k][j] = j == 0 ? 0 : -1;
      } else if (cfg->anchor_mode == SPD_ANCHOR_ZERO_MASK) {
        layer[k][j] = anchors[j] <= lmax ? anchors[j] : -1;
      } else {
        layer[k][j] = anchors[j] < lmax ? anchors[j] : lmax;
      }
    }
  }
  // distinct layers of the anchor mode, sorted
  char used[4097];
  if (L > 4096) return SPD_E_UNSUPPORTED;
  memset(used, 0, sizeof(used));
  for (int k = 0; k <= n; ++k)
    for (int j = 0; j < m; ++j)
      if (layer[k][j] >= 0) used[layer[k][j]] = 1;
  int index[4097];
  int S = 0;
  for (int l = 0; l <= L; ++l) {
    index[l] = -1;
    if (used[l]) {
      store_layers[S] = l;
      index[l] = S++;
    }
  }
  *n_store = S;
  // the row at staircase depth k reads the features of depth e(k)
  for (int k = 0; k <= n; ++k) {
    const int e = cfg->feature_schedule == SPD_SCHEDULE_POST_STEP    ? (k + 1 < n ? k + 1 : n)
                  : cfg->feature_schedule == SPD_SCHEDULE_FIRST_STAGE ? (k < 1 ? k : 1)
                                                                      : k;
    for (int j = 0; j < m; ++j) slot_tab[k * m + j] = layer[e][j] >= 0 ? index[layer[e][j]] : -1;
  }
  return SPD_OK;
}

extern "C" int spd_layout(int32_t t, int32_t a, int32_t n, int32_t* pos, int32_t* depth) {
  if (!pos || !depth || n < 1 || a < 1 || a > n || t < a + 1) return SPD_E_INVALID;
  const int M = a + 1, pos0 = t - 1 - a;
  for (int r = 0; r < M; ++r) {
    pos[r] = pos0 + r;
    depth[r] = r == 0 ? n : a - r;
  }
  return M;
}

extern "C" int spd_cycle_plan(int32_t t, int32_t a, int32_t n, spd_cycle_info* out) {
  if (!out || n < 1 || a < 1 || a > n || t < a + 1) return SPD_E_INVALID;
  // with one stage the token under verification would be this cycle's own draft
  if (n < 2) return SPD_E_UNSUPPORTED;
  spd_cycle_info p;
  p.pos0 = t - 1 - a;
  p.M = a + 1;
  p.verifies = a == n ? 1 : 0;
  p.exiting = p.verifies ? t - n : -1;
  p.cand = p.verifies ? t - n + 1 : -1;
  p.draft_pos = t;
  p.ring_draft = t % n;
  p.ring_cand = p.verifies ? p.cand % n : -1;
  *out = p;
  return SPD_OK;
}

extern "C" size_t spd_workspace_size(int32_t call, const spd_config* cfg, int32_t rows,
                                     int32_t gamma, int64_t T_cap) {
  if (rows < 1) return 0;
  switch (call) {
    case SPD_CALL_FUSE:
      return cfg ? fuse_workspace(cfg, rows) : 0;
    case SPD_CALL_PDM:
      return cfg ? pdm_workspace(cfg, rows, T_cap > 0 ? T_cap : 1) : 0;
    case SPD_CALL_LM_HEAD:
      return cfg ? lm_head_workspace(cfg, rows) : 0;
    case SPD_CALL_VERIFY:
      return cfg ? verify_workspace(rows, gamma, cfg->V) : 0;
    default:
      return 0;
  }
}

extern "C" int spd_rollback(spd_seq_state* st, int32_t n, const int32_t* drafted,
                            const int32_t* n_accept, const int32_t* next_token, int32_t* tokens,
                            int64_t T_cap, void* stream) {
  if (!st || !drafted || !n_accept || !next_token || !tokens || n < 1 || T_cap < 1)
    return SPD_E_INVALID;
  hipLaunchKernelGGL(rollback_kernel, dim3(1), dim3(1), 0, static_cast<hipStream_t>(stream), st, n,
                     drafted, n_accept, next_token, tokens, T_cap);
  return check_launch();
}

extern "C" const char* spd_status_string(int status) {
  switch (status) {
    case SPD_OK: return "ok";
    case SPD_E_INVALID: return "invalid argument";
    case SPD_E_UNSUPPORTED: return "unsupported shape or dtype";
    case SPD_E_WORKSPACE: return "workspace too small";
    case SPD_E_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

extern "C" int spd_last_hip_error(void) { return last_hip_error_ref(); }

extern "C" int spd_version(void) { return 3; }
