/*
 * spd.h -- C ABI of the SPD draft-and-verify cycle for AMD Instinct MI355X (gfx950).
 *
 * Speculative Pipeline Decoding ("Speculative Pipeline Decoding: Higher-Accuracy
 * Drafting with Hidden Latency via Pipeline Parallelism", arXiv 2605.30852) drafts
 * one token per pipeline cycle from depth-conditioned features of the tokens in
 * flight, and verifies one in-flight token per cycle.  One cycle on the draft
 * rank is:
 *
 *   spd_fuse_features   anchor gather + RMSNorm + FC  -> features g   (section 3.2)
 *   spd_pdm_step        L_s-layer Qwen3-style decoder  -> h_last       (section 3.1)
 *   spd_lm_head         draft head, argmax or sample   -> x_hat, q row (section 3.1, Eq. (1))
 *   spd_lm_head         target head on the exiting token's last state  (section 3.4)
 *   spd_verify          greedy match / rejection sampling             (section 3.4)
 *   spd_rollback        commit, or truncate to t-n+1 and reseed        (section 3.4)
 *
 * Conventions shared by every call
 *  - Pointers marked DEVICE are device pointers owned by the caller; pointers marked
 *    HOST are read during the call only.  Nothing is retained after return.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue kernels on it
 *    and return without synchronising; they never allocate or free memory.
 *  - Every device pointer must be 16-byte aligned (torch allocations are).
 *  - Argument errors are detected on the host and returned before anything is
 *    enqueued.  Values held in device memory (tokens, probabilities) are not
 *    inspected on the host; kernels clamp out-of-range indices so that no access
 *    leaves the buffers described below.
 *  - Workspaces: `ws` is a DEVICE buffer of at least spd_workspace_size(...) bytes,
 *    16-byte aligned, holding partial results of one call.  Its first
 *    SPD_WS_COUNTER_BYTES bytes are arrival counters that must be zero before the
 *    workspace is first used (allocate it zero-filled); every completed call leaves
 *    them zero again.  Calls that share a workspace must not run concurrently (use
 *    one workspace per stream).
 *  - dtype SPD_BF16: weights, anchors and the key/value cache are bfloat16 (bit
 *    pattern in uint16); SPD_F32: all of them are float32.  Features, hidden rows,
 *    logits and probabilities are always float32.
 *  - Return value: SPD_OK (0) or a negative status; spd_status_string() names it.
 */
#ifndef SPD_H
#define SPD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SPD_OK = 0,
  SPD_E_INVALID = -1,     /* null pointer, bad size or inconsistent arguments */
  SPD_E_UNSUPPORTED = -2, /* valid but not implemented shape/dtype combination */
  SPD_E_WORKSPACE = -3,   /* ws_bytes below spd_workspace_size()               */
  SPD_E_HIP = -4          /* a HIP launch failed; see spd_last_hip_error()      */
};

enum { SPD_F32 = 0, SPD_BF16 = 1 };
enum { SPD_ANCHOR_ZERO_MASK = 0, SPD_ANCHOR_CLAMP_MIN = 1 };
/* Feature schedules (section 3.3 and 4.5; PPSD in section 2): which depth's features
 * a row at staircase depth k uses.  PRE_STEP (the method's own): depth k.  POST_STEP:
 * depth min(n, k+1), every in-flight position one stage deeper (the newest token uses
 * g^1 instead of g^0).  FIRST_STAGE: depth min(k, 1), nothing deeper than the first
 * stage (PPSD's features). */
enum { SPD_SCHEDULE_PRE_STEP = 0, SPD_SCHEDULE_POST_STEP = 1, SPD_SCHEDULE_FIRST_STAGE = 2 };
enum { SPD_CALL_FUSE = 0, SPD_CALL_PDM = 1, SPD_CALL_LM_HEAD = 2, SPD_CALL_VERIFY = 3 };

#define SPD_WS_COUNTER_BYTES 65536
#define SPD_MAX_ANCHORS 8
#define SPD_MAX_STAGES 32
#define SPD_TOP_K_MAX 256
#define SPD_TREE_MAX_NODES 64

/* Sizes of the target, the PDM and the heads (section 3.1-3.2, section 4 setup). */
typedef struct spd_config {
  int32_t L;           /* target layers                                          */
  int32_t n;           /* pipeline stages (1..SPD_MAX_STAGES)                    */
  int32_t m;           /* anchors (1..SPD_MAX_ANCHORS)                           */
  int32_t d;           /* hidden size of target and PDM                          */
  int32_t Ls;          /* PDM decoder layers                                     */
  int32_t Hq, Hkv, hd; /* PDM query heads, key/value heads, head size (16..128)  */
  int32_t dff;         /* PDM MLP width                                          */
  int32_t V;           /* vocabulary                                             */
  int32_t dtype;       /* SPD_F32 or SPD_BF16                                    */
  int32_t anchor_mode; /* SPD_ANCHOR_ZERO_MASK (default) or SPD_ANCHOR_CLAMP_MIN  */
  int32_t norm_k0;     /* 0: g^0 = FC(H^0) without norm (default); 1: normalise  */
  float rms_eps;       /* 1e-6                                                   */
  float rope_theta;    /* 1e6                                                    */
  int32_t feature_schedule; /* SPD_SCHEDULE_PRE_STEP (default), _POST_STEP, _FIRST_STAGE */
  int32_t top_k;       /* sampling filter of spd_lm_head at T > 0: 0 = off, else   */
                       /* 1..SPD_TOP_K_MAX (section 4 evaluation setting: 50)      */
  float top_p;         /* nucleus mass, used when 0 < top_p < 1 (0 and 1 = off;   */
                       /* section 4 evaluation setting: 1.0); spd_lm_head applies */
                       /* it after top-k and returns SPD_E_UNSUPPORTED for        */
                       /* 0 < top_p < 1 with top_k = 0 at T > 0                    */
  int32_t head_workgroups; /* spd_lm_head's vocabulary GEMV (bf16, one row): 0 = one */
                       /* workgroup per 32 rows; else at most this many, each looping */
                       /* over row groups with one row's loads in flight per wave (a */
                       /* head streaming beside latency-bound work); results are   */
                       /* bit-identical for every value                            */
} spd_config;

/* One PDM decoder layer (DEVICE pointers, cfg.dtype).  Row-major [rows][cols]. */
typedef struct spd_layer_weights {
  const void *attn_norm; /* [d]                                              */
  const void *wqkv;      /* [(Hq+2*Hkv)*hd][d]: q heads, then k heads, then v  */
  const void *q_norm;    /* [hd]                                             */
  const void *k_norm;    /* [hd]                                             */
  const void *wo;        /* [d][Hq*hd]                                       */
  const void *mlp_norm;  /* [d]                                              */
  const void *w_gate_up; /* [2*dff][d]: gate rows, then up rows              */
  const void *w_down;    /* [d][dff]                                         */
} spd_layer_weights;

/* Sequence state kept in DEVICE memory by spd_rollback. */
typedef struct spd_seq_state {
  int32_t t;       /* sequence length (verified prefix + in-flight tokens) */
  int32_t a;       /* tokens in flight, 1..n                               */
  int32_t commits; /* N: tokens that exited the last stage                  */
  int32_t cycles;  /* K: executed cycles                                    */
} spd_seq_state;

/* ---------------------------------------------------------------- host helpers */

/* Anchor eligibility (section 3.2, Eq. (3); the review blog's core formulas for the
 * clamped variant).  l_max(k) = min(L, floor(k*L/n)).  For every staircase depth k in
 * 0..n and anchor j, writes slot_tab[k*m + j] = index into `store_layers` of the
 * target layer slot j reads, or -1 for an empty slot.  With e = the feature depth of
 * k under cfg->feature_schedule (k, min(n, k+1) or min(k, 1)):
 *   ZERO_MASK: layer b_j if b_j <= l_max(e), else empty;
 *   CLAMP_MIN: layer min(b_j, l_max(e));
 *   e = 0 (both modes): slot 0 reads layer 0 (the embedding), the rest are empty.
 * store_layers (HOST, capacity L+1) receives the sorted distinct layers an anchor
 * store must hold for the anchor mode (every schedule reads a subset of them);
 * *n_store their count.  anchors (HOST [m]) must be strictly increasing with
 * anchors[0] = 0 and anchors[m-1] <= L.
 */
int spd_slot_table(const spd_config *cfg, const int32_t *anchors, int32_t *slot_tab,
                   int32_t *store_layers, int32_t *n_store);

/* Rows one cycle recomputes (section 3.1 Eq. (2), section 3.2 partial fill, section 3.3
 * pre-step depths).  With t tokens and a in flight (1 <= a <= n, a < t): M = a+1 rows
 * at positions pos0 = t-1-a .. t-1; the first is fully processed (depth n) and the
 * in-flight ones have depths a-1 .. 0.  Writes pos[M], depth[M] (HOST) and returns M,
 * or SPD_E_INVALID. */
int spd_layout(int32_t t, int32_t a, int32_t n, int32_t *pos, int32_t *depth);

/* Everything the host needs to issue one cycle (section 3.1 Eq. (2); section 3.4
 * streaming verification), from the state (t tokens, a of them in flight) the
 * cycle starts from; positions are 0-based (position i holds x_{i+1}).
 *   pos0, M      rows the cycle recomputes, as spd_layout: pos0 = t-1-a, M = a+1
 *   verifies     1 iff a == n: the pipeline is saturated, the token at `exiting`
 *                leaves the last stage and its successor `cand` is verified
 *   exiting      t-n (the target head reads its last-layer state), else -1
 *   cand         t-n+1, drafted n-1 cycles earlier (x_{t-n+2}), else -1
 *   draft_pos    t: the position this cycle's draft fills
 *   ring_draft   t mod n: row of an n-row ring that keeps this cycle's q
 *   ring_cand    cand mod n: the ring row holding cand's q (the row written when
 *                cand was drafted; the n-1 drafts since used the other rows), else -1
 * Returns SPD_OK, SPD_E_INVALID (out NULL, a outside 1..n, t < a+1) or
 * SPD_E_UNSUPPORTED for n < 2, where cand would be this cycle's own draft. */
typedef struct spd_cycle_info {
  int32_t pos0, M, verifies, exiting, cand, draft_pos, ring_draft, ring_cand;
} spd_cycle_info;
int spd_cycle_plan(int32_t t, int32_t a, int32_t n, spd_cycle_info *out);

/* Bytes of workspace a call needs.  call: SPD_CALL_*; rows = M for FUSE and PDM, the
 * number of head rows for LM_HEAD, B for VERIFY (then gamma and cfg->V are used);
 * T_cap is the key/value cache capacity of the PDM call (ignored by the others).
 * Returns 0 for invalid arguments. */
size_t spd_workspace_size(int32_t call, const spd_config *cfg, int32_t rows, int32_t gamma,
                          int64_t T_cap);

/* ---------------------------------------------------------------- cycle calls */

/* Depth-conditioned features (section 3.2 Eq. (3); review blog core formulas:
 * g = FC(norm(Concat(anchors)))).
 * Rows are positions pos0 .. pos0+M-1; the last `a` of them have depths a-1 .. 0 and
 * the others depth n (so a = 0 means all rows are fully processed, e.g. prefill).
 * For a row at position i and depth k:
 *   k = 0, !norm_k0 and not POST_STEP: g = W_fc[:, 0:d] . H_i^{layer 0}  (no norm, no gamma)
 *   otherwise: x = Concat_j (slot_tab[k*m+j] >= 0 ? H_i^{store slot} : 0),
 *              rms = sqrt(sum(x^2) / (#filled * d) + eps),  g = W_fc (norm_w * x / rms)
 * (under SPD_SCHEDULE_POST_STEP the depth-0 row uses depth-1 features, normalised).
 * The large-M path (bf16, M >= 256) feeds the product the bf16-rounded norm_w * x.
 * hstore  DEVICE [T_cap][S][d]  anchor hidden states, slot s holds store_layers[s]
 * slot_tab HOST [(n+1)*m]       as written by spd_slot_table (any table of slots < S)
 * norm_w  DEVICE [m*d]; fc_w DEVICE [d][m*d]; g DEVICE float [M][d] (output).
 * Requires d % 64 == 0, pos0 >= 0, pos0+M <= T_cap, 0 <= a <= min(n, M); SPD_E_UNSUPPORTED
 * when d % 64 != 0 or m*d > 262144.
 */
int spd_fuse_features(const spd_config *cfg, const void *hstore, int64_t T_cap, int32_t S,
                      const int32_t *slot_tab, int32_t pos0, int32_t M, int32_t a,
                      const void *norm_w, const void *fc_w, float *g,
                      void *ws, size_t ws_bytes, void *stream);

/* FC weights with the norm folded in, for spd_fuse_features_scaled (section 3.2 Eq. (3):
 * W_fc (norm_w * x) / rms = (W_fc diag(norm_w)) x / rms).  Writes
 *   fc_w_scaled[c][j] = bf16(fc_w[c][j] * norm_w[j])   (the product is exact in fp32,
 *                                                         rounded once)
 * norm_w DEVICE bf16 [m*d]; fc_w, fc_w_scaled DEVICE bf16 [d][m*d] (caller-owned, 16-byte
 * aligned, not overlapping).  bf16 only (SPD_E_UNSUPPORTED otherwise); d % 64 == 0. */
int spd_fc_prepare(const spd_config *cfg, const void *norm_w, const void *fc_w, void *fc_w_scaled,
                   void *stream);

/* spd_fuse_features with the prepared weights of spd_fc_prepare.  A bf16 call with
 * M >= 256, a == 0 and every anchor j in store slot j at depth n (each row's
 * concatenation is then the first m*d values of its store row) runs one launch: the
 * product reads the anchor store directly, multiplies by fc_w_scaled and scales each
 * row by 1/rms of its store values; any other call is spd_fuse_features (fc_w_scaled is
 * not read).  Same arguments and workspace as spd_fuse_features, plus fc_w_scaled
 * DEVICE bf16 [d][m*d] (required). */
int spd_fuse_features_scaled(const spd_config *cfg, const void *hstore, int64_t T_cap, int32_t S,
                             const int32_t *slot_tab, int32_t pos0, int32_t M, int32_t a,
                             const void *norm_w, const void *fc_w, const void *fc_w_scaled,
                             float *g, void *ws, size_t ws_bytes, void *stream);

/* PDM step (section 3.1: f_theta is an Ls-layer decoder with Qwen3-style attention; the
 * draft reads its last-position output).  Each layer (pre-norm):
 *   h += W_o . Attn(RoPE(qnorm(W_q n1)), RoPE(knorm(W_k n1)), W_v n1),  n1 = RMSNorm(h)
 *   h += W_down (silu(W_gate n2) * (W_up n2)),                           n2 = RMSNorm(h)
 * with GQA (query head h reads kv head h / (Hq/Hkv)), rotate-half RoPE at 0-based
 * positions, scale 1/sqrt(hd), and a causal mask.  Input rows h = g at positions
 * pos0 .. pos0+M-1 attend to cached positions < pos0 and to each other.  The call
 * writes this call's keys/values at positions pos0 .. pos0+M-1 (later cycles treat
 * positions below their own pos0 as committed).
 * layers   HOST [Ls]; final_norm DEVICE [d]
 * k_cache  DEVICE [Ls][Hkv][T_cap][hd]      keys (normed, rotated)
 * v_cache  DEVICE [Ls][Hkv][hd][T_cap]      values, position-minor
 * g        DEVICE float [M][d]; h_last DEVICE float [d] = final RMSNorm of row M-1.
 * Requires d % 64 == 0, hd in {16,32,64,128}, Hq % Hkv == 0, dff % 64 == 0,
 * T_cap % 8 == 0, pos0 + M <= T_cap.
 */
int spd_pdm_step(const spd_config *cfg, const spd_layer_weights *layers, const void *final_norm,
                 void *k_cache, void *v_cache, int64_t T_cap, const float *g, int32_t pos0,
                 int32_t M, float *h_last, void *ws, size_t ws_bytes, void *stream);

/* Prepared weights for prefill-sized PDM steps (the same decoder as spd_pdm_step, section
 * 3.1).  Those steps carry each activation feeding the QKV, gate/up and down products as
 * a bf16 part plus its residual; with prepared weights the residual's product runs on the
 * block-scaled e4m3 MFMA instead of a second bf16 pass (about 2^-12 of the activation
 * against 2^-9 for the bf16 part alone).  spd_pdm_prepare writes, per layer, e4m3 copies
 * of W_qkv, W_gate_up and W_down with one power-of-two factor per row (the row's largest
 * magnitude scaled into [128, 256)) and that row's E8M0 scale byte.
 * spd_pdm_prepared_bytes: the buffer size, 0 when the configuration takes no prepared
 *   weights (they need bf16, hd == 128, d % 128 == 0 and dff % 128 == 0).
 * spd_pdm_prepare: prep DEVICE, 16-byte aligned, prep_bytes >= that size; layers as in
 *   spd_pdm_step (the three matrices are read).  SPD_E_UNSUPPORTED for other
 *   configurations, SPD_E_WORKSPACE if prep_bytes is short.  Run it again whenever the
 *   weights change.
 * spd_pdm_step_prepared: spd_pdm_step with prep (written by spd_pdm_prepare for these
 *   weights, prep_bytes its size), used by steps with M >= 256; prep == NULL is
 *   spd_pdm_step.  SPD_E_INVALID when prep is given for a configuration that takes none.
 *   Same workspace as spd_pdm_step. */
size_t spd_pdm_prepared_bytes(const spd_config *cfg);
int spd_pdm_prepare(const spd_config *cfg, const spd_layer_weights *layers, void *prep,
                    size_t prep_bytes, void *stream);
int spd_pdm_step_prepared(const spd_config *cfg, const spd_layer_weights *layers, const void *prep,
                          size_t prep_bytes, const void *final_norm, void *k_cache, void *v_cache,
                          int64_t T_cap, const float *g, int32_t pos0, int32_t M, float *h_last,
                          void *ws, size_t ws_bytes, void *stream);

/* LM head and next-token choice (section 3.1 Eq. (1); section 3.4 target head).
 * logits[r] = W_lm . h[r] for r < rows (rows <= 16).
 * temperature == 0: token[r] = lowest index of the maximum logit (NaN never wins);
 *   probs may be NULL and words is unused.  With cfg.top_k >= 2 (the children of a
 *   greedy draft-tree node) token is [rows][top_k] instead: the indices of the top_k
 *   largest logits in descending order (equal logits by ascending index, NaN last),
 *   -1 past the vocabulary.
 * temperature > 0: probs[r] = softmax(logits[r] / T) (float32) and
 *   token[r] = inverse-CDF draw from the integer weights w_j = floor(probs_j * 2^52):
 *   u = words[r] >> 32, tau = floor(u * sum(w) / 2^32), token = smallest j whose
 *   inclusive prefix sum of w exceeds tau.
 *   With cfg.top_k >= 1 (section 4 evaluation setting: T = 1, top-k = 50, top-p = 1)
 *   the softmax is taken over the cfg.top_k largest logits only (equal logits rank by
 *   ascending index, NaN last) and probs is 0 elsewhere; with 0 < cfg.top_p < 1 it is
 *   further restricted to the shortest run of those, in descending logit order, whose
 *   top-k probability (computed in float64) reaches top_p, and renormalised.  The draw
 *   is the same inverse CDF over the filtered probs.  A nucleus without top-k
 *   (cfg.top_k = 0, 0 < cfg.top_p < 1, T > 0) is not offered: SPD_E_UNSUPPORTED.
 * w_lm DEVICE [V][d] (cfg.dtype); h DEVICE float [rows][d]; words DEVICE uint64 [rows];
 * logits, probs DEVICE float [rows][V]; token DEVICE int32 [rows].
 */
int spd_lm_head(const spd_config *cfg, const void *w_lm, const float *h, int32_t rows,
                float temperature, const uint64_t *words, float *logits, float *probs,
                int32_t *token, void *ws, size_t ws_bytes, void *stream);

/* Verification (section 3.4 streaming verify; the speculative-decoding explainer's
 * four-phase loop and acceptance criterion).  For each sequence b < B and drafted
 * positions j = 0 .. gamma-1 in order, until the first rejection:
 *   T == 0: accept iff draft[b][j] is the argmax of p[b][j] (p holds logits); on a
 *           mismatch the argmax is the next token.
 *   T > 0:  R = words[b][j][0] >> 40; accept iff (R+1) * q(x) <= p(x) * 2^24, i.e.
 *           r <= min(1, p/q) for r = (R+1)/2^24, decided exactly.  On rejection the
 *           next token is drawn (as in spd_lm_head, with u = words[b][j][1] >> 32)
 *           from the integer residual max(0, P_i - Q_i), P = floor(p*2^52),
 *           Q = floor(q*2^52); from P itself if that residual is all zero.
 * If all gamma drafts are accepted: next = bonus ? draw from p[b][gamma] (argmax at
 * T == 0; u = words[b][gamma][1] >> 32) : -1.
 * p DEVICE float [B][gamma+bonus][V]; q DEVICE float [B][gamma][V] (unused at T == 0);
 * draft DEVICE int32 [B][gamma]; words DEVICE uint64 [B][gamma+1][2];
 * n_accept, next_token DEVICE int32 [B] (outputs).  SPD streaming verify is
 * B = 1, gamma = 1, bonus = 0.
 */
int spd_verify(int32_t B, int32_t gamma, int32_t V, float temperature, int32_t bonus,
               const float *p, const float *q, const int32_t *draft, const uint64_t *words,
               int32_t *n_accept, int32_t *next_token, void *ws, size_t ws_bytes,
               void *stream);

/* End-of-cycle commit or rollback (section 3.4; review blog, synchronous rollback),
 * one thread on the device, reading the state the cycle started from:
 *   a == n (the cycle verified; n_accept[0], next_token[0] are its outcome):
 *     commits += 1;
 *     rejected (n_accept[0] == 0): keep x_1..x_{t-n+1}, discard the n-1 younger
 *       in-flight tokens and this cycle's draft, append next_token[0] at depth 0:
 *       tokens[t-n+1] = next_token[0]; t = t-n+2; a = 1.
 *     accepted: tokens[t] = drafted[0]; t += 1 (a stays n).
 *   a < n: tokens[t] = drafted[0]; t += 1; a += 1.
 *   cycles += 1 in every case.  Writes at or beyond T_cap are dropped.
 * st DEVICE; drafted, n_accept, next_token DEVICE int32 [1]; tokens DEVICE int32 [T_cap].
 */
int spd_rollback(spd_seq_state *st, int32_t n, const int32_t *drafted, const int32_t *n_accept,
                 const int32_t *next_token, int32_t *tokens, int64_t T_cap, void *stream);

/* ---------------------------------------------------------------- draft trees */

/* Width-W draft trees (section 4, draft-tree paragraph, and Appendix B: trees raise
 * acceptance; the pages measure them in theory only and leave branched key/value
 * caches and tree attention masks open).  A tree's M <= SPD_TREE_MAX_NODES nodes are
 * rows in topological order; anc DEVICE uint64 [M]: bit j of anc[i] is set iff node
 * j is node i or one of its ancestors.  Node 0 is the root, the newest fully
 * processed token (anc[0] = 1); every other node's mask is its parent's plus its own
 * bit.  level(i) = popcount(anc[i]) - 1.  Node i reads anchor-store row pos0 + i
 * (its own branch's target states), sits at position pos0 + level(i) and keeps its
 * keys/values in cache slot pos0 + i.  The masks are read on the device and not
 * validated; a malformed mask changes results but no access leaves the buffers. */

/* spd_fuse_features over a tree: node i has depth n at level 0 and a - level(i)
 * below it (the in-flight levels 1..a); otherwise as spd_fuse_features.
 * Requires 1 <= a <= n, M <= SPD_TREE_MAX_NODES; anc 8-byte aligned. */
int spd_fuse_features_tree(const spd_config *cfg, const void *hstore, int64_t T_cap, int32_t S,
                           const int32_t *slot_tab, int32_t pos0, int32_t M, int32_t a,
                           const uint64_t *anc, const void *norm_w, const void *fc_w, float *g,
                           void *ws, size_t ws_bytes, void *stream);

/* spd_pdm_step over a tree: node i attends to the cached positions < pos0 and to the
 * nodes on its own root path, with RoPE at position pos0 + level(i); its keys/values
 * go to slot pos0 + i.  h_out DEVICE float [n_out][d] receives the final-normed rows
 * M - n_out .. M - 1 (the deepest level's nodes when they come last), 1 <= n_out <= M.
 * Workspace as spd_pdm_step. */
int spd_pdm_step_tree(const spd_config *cfg, const spd_layer_weights *layers,
                      const void *final_norm, void *k_cache, void *v_cache, int64_t T_cap,
                      const float *g, int32_t pos0, int32_t M, const uint64_t *anc, int32_t n_out,
                      float *h_out, void *ws, size_t ws_bytes, void *stream);

/* Verification of sibling candidates: W candidates for one position per sequence (a
 * draft-tree level whose nodes share one parent).  Returns accepted[b] = index of the
 * accepted candidate, or -1 with next_token[b] = the token that replaces them (else -1).
 * temperature == 0 (section 3.4, greedy): p DEVICE float [B][V] holds target logits;
 *   best = argmax (lowest index on ties); the first i with cand[b][i] == best is
 *   accepted, else next_token = best.  q and words are unused.
 * temperature > 0 (multi-round form of the speculative-decoding explainer's acceptance
 *   criterion; the candidates must be independent draws from q): p, q DEVICE float
 *   [B][V] probability rows (sums near 1), words DEVICE uint64 [B][W+1][2].  With
 *   A = floor(p 2^51), B = floor(q 2^51) (integers): round i accepts cand[b][i] = x iff
 *   (R_i + 1) B(x) sum(A) <= 2^24 A(x) sum(B), R_i = words[b][i][0] >> 40 (x outside the
 *   vocabulary is rejected); on rejection A <- max(0, A sum(B) - B sum(A)) >> s with
 *   s = max(0, bitlength of its sum - 52), the residual max(0, p_i - q) as the next
 *   target.  After W rejections next_token is the inverse-CDF draw from A with
 *   u = words[b][W][1] >> 32 (from floor(p 2^51) if A is empty).  The output token is
 *   distributed as p.  Batches of fewer than 64 sequences spread every pass over the
 *   vocabulary across many workgroups (one launch per pass, 1 + 2W launches; a sequence
 *   that is decided makes the remaining launches return at once); larger batches use
 *   one workgroup per sequence.  The decisions are the same either way.
 * cand DEVICE int32 [B][W] (W <= SPD_TREE_MAX_NODES); accepted, next_token DEVICE int32
 * [B].  ws >= spd_workspace_size(SPD_CALL_VERIFY, cfg with this V, B, 0, 0).  The W
 * candidates of a greedy tree node come from spd_lm_head at T = 0 with cfg.top_k = W. */
int spd_verify_siblings(int32_t B, int32_t W, int32_t V, float temperature, const float *p,
                        const float *q, const int32_t *cand, const uint64_t *words,
                        int32_t *accepted, int32_t *next_token, void *ws, size_t ws_bytes,
                        void *stream);

/* ---------------------------------------------------------------- no allocation */

/* For callers that cannot allocate device memory or pass a workspace (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call as spd_lm_head, with its workspace in a device array of
 * SPD_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends.  It allocates and frees nothing.  The GPU is the one `stream`
 * belongs to (the current device for NULL).  The first call on a GPU looks up the
 * array's address with that GPU current and clears its arrival counters with a
 * kernel on `stream` (make that first call outside graph capture).  Returns
 * SPD_E_WORKSPACE when spd_workspace_size(SPD_CALL_LM_HEAD, cfg, rows) exceeds
 * SPD_NOALLOC_SCRATCH_BYTES (64 MiB: up to 16 rows with top_k <= 256 at V = 151936
 * and d <= 4096 fit; a vocabulary of millions does not), else as spd_lm_head.  Every call on a
 * GPU shares that GPU's array: calls that may overlap on one GPU (other streams,
 * other host threads) race and must not be issued; the array keeps the last
 * call's contents. */
#define SPD_NOALLOC_SCRATCH_BYTES (64u << 20)
int spd_lm_head_noalloc(const spd_config *cfg, const void *w_lm, const float *h, int32_t rows,
                        float temperature, const uint64_t *words, float *logits, float *probs,
                        int32_t *token, void *stream);

const char *spd_status_string(int status);
int spd_last_hip_error(void);
/* Version of this interface: 3 (2: spd_config gained top_k, top_p and head_workgroups;
 * 3: spd_cycle_plan). */
int spd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPD_H */
