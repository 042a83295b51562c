"""Plain CPU oracle of one Speculative Pipeline Decoding (SPD) draft-and-verify cycle.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The product path
(``pipeline_draft_step_amd``) never imports it, and this module imports nothing
from the product path: the two share no code, constants or tables.

Everything is numpy in float64 (inputs are the bf16- or fp32-valued arrays the
device sees, widened to float64).  Integer decisions (argmax, sampling, the
accept test) are exact.  It is written to be read against the pages, not to be
fast.

Pages cited (by title and section; the text of each page is the authority):

* [SPD]   "Speculative Pipeline Decoding: Higher-Accuracy Drafting with Hidden
          Latency via Pipeline Parallelism" (arXiv 2605.30852), sections 3.1-3.4
          and 4 (metrics).  Its display equations were lost in extraction; each
          function below states the reading of the prose it takes.
* [REV]   The xllm-io paper-review blog post on the same paper, section
          "核心公式" (core formulas) and "验证与回滚机制" (verification and rollback).
* [SD]    "Speculative Decoding: How Draft-Model Parallelism Cuts LLM Inference
          Latency", sections "The four-phase loop", "The acceptance criterion and
          why it is exact", "Acceptance rate equals 1 minus total variation
          distance", "Theoretical speedup".

Parity status per function: every function below is pinned by a ``-m "not gpu"``
test in ``tests/test_oracle_pins.py`` except where its docstring says
"parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

ZERO_MASK = 0
CLAMP_MIN = 1

# feature schedules ([SPD] 3.3 and 4.5; [SPD] 2 for PPSD)
PRE_STEP = 0     # the pages' choice: features present before the current pipeline forward
POST_STEP = 1    # features after the forward: every in-flight position one stage deeper
FIRST_STAGE = 2  # PPSD's features: nothing deeper than the first stage (l <= L/n)

_TWO52 = float(2 ** 52)


# --------------------------------------------------------------------------
# Layout and eligibility  ([SPD] 3.1 Eq. (2), 3.2 Eq. (3) and the partial-fill
# equation; [REV] core formulas)
# --------------------------------------------------------------------------

def l_max(k: int, L: int, n: int) -> int:
    """Deepest target layer available to a token that has completed k of n stages.

    [SPD] 3.2: l_max(k) = min(L, k*L/n).  Stages are whole layers (uniform L/n
    splits, [SPD] 4 setup), so a non-integral k*L/n is floored.
    """
    if not 0 <= k <= n:
        raise ValueError("depth k must lie in 0..n")
    return min(L, (k * L) // n)


def slot_layers(k: int, L: int, n: int, anchors, mode: int = ZERO_MASK):
    """Target layer read by each of the m anchor slots at depth k (-1 = empty slot).

    [SPD] 3.2 Eq. (3): a depth-k token consumes every anchor b_j <= l_max(k);
    the others are left out (ZERO_MASK: their slot of the concatenation is 0).
    [REV] core formulas, 0<k<n case: the clamped variant reads layer
    min(b_j, l_max(k)) in every slot (CLAMP_MIN).
    Both sources give k = 0 its own rule, g^0 = FC(H^0): only slot 0 (b_0 = 0,
    the embedding) is read.
    """
    anchors = [int(b) for b in anchors]
    if anchors[0] != 0:
        raise ValueError("the first anchor must be the embedding layer 0")
    if k == 0:
        return [0] + [-1] * (len(anchors) - 1)
    lm = l_max(k, L, n)
    if mode == ZERO_MASK:
        return [b if b <= lm else -1 for b in anchors]
    if mode == CLAMP_MIN:
        return [min(b, lm) for b in anchors]
    raise ValueError("unknown anchor mode")


def feature_depth(k: int, n: int, schedule: int = PRE_STEP) -> int:
    """Depth whose features a row uses when the staircase puts it at depth k.

    [SPD] 3.3: the pre-step schedule conditions on the intermediates present
    before the current pipeline forward; relative to a post-step schedule every
    in-flight position is one stage shallower (its example: the newest token
    uses g^0 instead of g^1), so post-step = min(n, k + 1).  The verified prefix
    (k = n) is the same in both.  [SPD] 2: PPSD uses only first-stage features,
    read here as depth min(k, 1): the embedding alone for a token that has not
    entered a stage yet, the first stage's output (l <= L/n) for all others.
    """
    if not 0 <= k <= n:
        raise ValueError("depth k must lie in 0..n")
    if schedule == PRE_STEP:
        return k
    if schedule == POST_STEP:
        return min(n, k + 1)
    if schedule == FIRST_STAGE:
        return min(k, 1)
    raise ValueError("unknown feature schedule")


def store_layers_for(L: int, n: int, anchors, mode: int = ZERO_MASK):
    """Sorted list of target layers an anchor store must hold for this mode (every
    feature schedule reads a subset of them)."""
    layers = set()
    for k in range(n + 1):
        layers.update(l for l in slot_layers(k, L, n, anchors, mode) if l >= 0)
    return sorted(layers)


def depths(t: int, a: int, n: int):
    """Pipeline depth of positions 0..t-1 when a tokens are in flight.

    [SPD] 3.1 Eq. (2) (a = n) and 3.2's partial-fill layout (a < n): positions
    before the trailing a are fully processed (k = n); the in-flight tokens form
    a staircase from the oldest (depth a-1) down to the newest (depth 0, the
    embedding-only input), the pre-step reading of [SPD] 3.3.
    """
    if not 1 <= a <= n or a > t:
        raise ValueError("need 1 <= a <= min(n, t)")
    return [n if i < t - a else t - 1 - i for i in range(t)]


def cycle_rows(t: int, a: int, n: int):
    """Rows recomputed by one cycle: the newest fully-processed position plus the
    a in-flight ones.  Returns (pos0, positions, depths).  Positions before pos0
    keep the key/value entries computed when they last changed depth."""
    if t < a + 1:
        raise ValueError("need at least one fully processed position")
    dep = depths(t, a, n)
    pos0 = t - 1 - a
    pos = list(range(pos0, t))
    return pos0, pos, [dep[i] for i in pos]


# --------------------------------------------------------------------------
# Feature fusion  ([SPD] 3.2; [REV] core formulas)
# --------------------------------------------------------------------------

def fuse_features(store, store_layers, pos, depth, gamma, w_fc, *, L, n, anchors,
                  mode=ZERO_MASK, eps=1e-6, norm_k0=False, schedule=PRE_STEP):
    """Depth-conditioned feature g_i^k for each requested row.

    store:  [T][S][d]  hidden states H_i^l of every layer listed in store_layers.
    gamma:  [m*d]      RMSNorm weight of the concatenation.
    w_fc:   [d][m*d]   FC projection (no bias).
    For k >= 1: x = Concat over slots (zeros in empty slots), RMS over the filled
    slots only, u = gamma * x / rms, g = W_fc u.  For k = 0: g = W_fc[:, :d] H^0
    (no norm, no gamma) unless norm_k0 asks for the uniform rule.  `depth` is
    the staircase depth; the feature schedule maps it to the depth whose
    features the row uses (feature_depth), and the k = 0 rule applies when that
    depth is 0.
    """
    store = np.asarray(store, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    w_fc = np.asarray(w_fc, dtype=np.float64)
    d = store.shape[2]
    m = len(anchors)
    index_of = {l: s for s, l in enumerate(store_layers)}
    out = np.zeros((len(pos), d))
    for r, (i, k_row) in enumerate(zip(pos, depth)):
        k = feature_depth(k_row, n, schedule)
        layers = slot_layers(k, L, n, anchors, mode)
        if k == 0 and not norm_k0:
            out[r] = w_fc[:, :d] @ store[i, index_of[0]]
            continue
        x = np.zeros(m * d)
        filled = 0
        for j, l in enumerate(layers):
            if l >= 0:
                x[j * d:(j + 1) * d] = store[i, index_of[l]]
                filled += 1
        rms = math.sqrt(float(np.dot(x, x)) / (filled * d) + eps)
        u = gamma * x / rms
        out[r] = w_fc @ u
    return out


# --------------------------------------------------------------------------
# Pipeline Draft Module: Qwen3-style decoder ([SPD] 3.1)
# --------------------------------------------------------------------------

def rms_norm(x, w, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


def silu(x):
    return x / (1.0 + np.exp(-x))


def rope(x, positions, theta):
    """Rotate-half rotary embedding of x [T][H][hd] at the given 0-based positions."""
    x = np.asarray(x, dtype=np.float64)
    hd = x.shape[-1]
    half = hd // 2
    inv_freq = theta ** (-np.arange(half, dtype=np.float64) * 2.0 / hd)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv_freq[None, :]
    cos = np.cos(ang)[:, None, :]
    sin = np.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x2 * cos + x1 * sin], axis=-1)


@dataclass
class PdmConfig:
    d: int
    Hq: int
    Hkv: int
    hd: int
    dff: int
    eps: float = 1e-6
    rope_theta: float = 1e6


def _split_qkv(qkv, c: PdmConfig):
    T = qkv.shape[0]
    nq, nk = c.Hq * c.hd, c.Hkv * c.hd
    q = qkv[:, :nq].reshape(T, c.Hq, c.hd)
    k = qkv[:, nq:nq + nk].reshape(T, c.Hkv, c.hd)
    v = qkv[:, nq + nk:].reshape(T, c.Hkv, c.hd)
    return q, k, v


def _attend(q, k_all, v_all, q_pos, k_pos, c: PdmConfig, allowed=None):
    """GQA softmax attention: query head h reads key/value head h // (Hq/Hkv).
    Causal by position unless `allowed` [queries][keys] gives the mask."""
    group = c.Hq // c.Hkv
    out = np.zeros((q.shape[0], c.Hq, c.hd))
    scale = 1.0 / math.sqrt(c.hd)
    if allowed is None:
        allowed = np.asarray(k_pos)[None, :] <= np.asarray(q_pos)[:, None]
    for h in range(c.Hq):
        kh = k_all[:, h // group, :]
        vh = v_all[:, h // group, :]
        s = (q[:, h, :] @ kh.T) * scale
        s = np.where(allowed, s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p = p / p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ vh
    return out


def decoder_layer(h, positions, lw, c: PdmConfig, kv_prefix=None, allowed=None):
    """One pre-norm decoder layer over rows h [T][d] at `positions`.

    lw: dict of float64 arrays attn_norm [d], wqkv [(Hq+2Hkv)*hd][d] (q heads,
    then k heads, then v heads), q_norm [hd], k_norm [hd], wo [d][Hq*hd],
    mlp_norm [d], w_gate_up [2*dff][d] (gate rows, then up rows), w_down [d][dff].
    kv_prefix: optional (K [P][Hkv][hd], V [P][Hkv][hd], positions [P]) of earlier
    rows (already normed and rotated).  allowed: optional attention mask [rows]
    [prefix + rows] (default: causal by position).  Returns (h_out, K_rows,
    V_rows) where K_rows/V_rows are this call's rows' keys/values as they enter
    attention.
    """
    n1 = rms_norm(h, lw["attn_norm"], c.eps)
    q, k, v = _split_qkv(n1 @ lw["wqkv"].T, c)
    q = rope(rms_norm(q, lw["q_norm"], c.eps), positions, c.rope_theta)
    k = rope(rms_norm(k, lw["k_norm"], c.eps), positions, c.rope_theta)
    if kv_prefix is not None:
        kp, vp, pp = kv_prefix
        k_all = np.concatenate([kp, k], axis=0)
        v_all = np.concatenate([vp, v], axis=0)
        k_pos = list(pp) + list(positions)
    else:
        k_all, v_all, k_pos = k, v, list(positions)
    att = _attend(q, k_all, v_all, positions, k_pos, c, allowed)
    h = h + att.reshape(h.shape[0], -1) @ lw["wo"].T
    n2 = rms_norm(h, lw["mlp_norm"], c.eps)
    gu = n2 @ lw["w_gate_up"].T
    act = silu(gu[:, :c.dff]) * gu[:, c.dff:]
    h = h + act @ lw["w_down"].T
    return h, k, v


def pdm_forward(G, layers, final_norm, c: PdmConfig):
    """Definitional PDM: run f_theta over the whole feature sequence G [t][d]
    with a causal mask and return the final-normed last row ([SPD] 3.1 Eq. (1):
    the draft reads the last-position representation).  No token embedding
    enters: the input rows are the features themselves."""
    h = np.asarray(G, dtype=np.float64)
    positions = list(range(h.shape[0]))
    for lw in layers:
        h, _, _ = decoder_layer(h, positions, lw, c)
    return rms_norm(h[-1], final_norm, c.eps)


class PdmCache:
    """Key/value entries per layer for positions 0..len-1 (float64)."""

    def __init__(self, n_layers: int, c: PdmConfig):
        self.k = [np.zeros((0, c.Hkv, c.hd)) for _ in range(n_layers)]
        self.v = [np.zeros((0, c.Hkv, c.hd)) for _ in range(n_layers)]

    def length(self) -> int:
        return self.k[0].shape[0]

    def truncate(self, n: int) -> None:
        self.k = [x[:n] for x in self.k]
        self.v = [x[:n] for x in self.v]


def pdm_step(g_rows, pos0, cache: PdmCache, layers, final_norm, c: PdmConfig):
    """Incremental PDM: rows pos0..pos0+M-1 attend to the cached positions
    < pos0 and causally to each other.  Afterwards the cache holds exactly the
    positions 0..pos0+M-1 (this call's rows overwrite any older entries at those
    positions).  Returns (final-normed last row, un-normed output rows [M][d])."""
    h = np.asarray(g_rows, dtype=np.float64)
    M = h.shape[0]
    positions = list(range(pos0, pos0 + M))
    for li, lw in enumerate(layers):
        kp, vp = cache.k[li][:pos0], cache.v[li][:pos0]
        if kp.shape[0] != pos0:
            raise ValueError("cache does not cover the positions before pos0")
        h, k, v = decoder_layer(h, positions, lw, c, (kp, vp, range(pos0)))
        cache.k[li] = np.concatenate([kp, k], axis=0)
        cache.v[li] = np.concatenate([vp, v], axis=0)
    return rms_norm(h[-1], final_norm, c.eps), h


# --------------------------------------------------------------------------
# Draft trees ([SPD] 4, draft-tree paragraph, and Appendix B: width-W trees raise
# acceptance; [REV] draft-tree paragraphs).  The pages measure trees only in
# theory and leave branched KV caches and tree attention masks open; the
# readings below are this oracle's own: the tree is the staircase with branches
# (level l holds in-flight tokens at depth a - l), each node keeps its own
# key/value slot, and a node attends to the committed prefix and its root path.
# --------------------------------------------------------------------------

def tree_levels(anc):
    """Level of every node of a draft tree given by ancestor masks.

    Rows are the nodes in topological order.  Bit j of anc[i] is set iff node j
    is node i or one of its ancestors; node 0 is the root (anc[0] = 1).  Every
    other node's parent p is its highest ancestor below it, and
    anc[i] = anc[p] | 2^i.  Returns the number of proper ancestors of each node.
    """
    anc = [int(x) for x in anc]
    if not anc or anc[0] != 1:
        raise ValueError("node 0 must be the root, with mask 1")
    for i in range(1, len(anc)):
        a = anc[i]
        if not (a >> i) & 1 or a >> (i + 1):
            raise ValueError("a node's mask holds itself and only earlier nodes")
        rest = a & ~(1 << i)
        if rest == 0 or anc[rest.bit_length() - 1] != rest:
            raise ValueError("a node's mask is its parent's mask plus itself")
    return [bin(x).count("1") - 1 for x in anc]


def tree_rows(anc, a: int, n: int, pos0: int):
    """Anchor-store rows, pipeline depths and positions of a draft tree's nodes.

    Node i reads store row pos0 + i (the target states of its own branch) and
    sits at position pos0 + level(i).  The root (level 0) is the newest fully
    processed token (depth n); level l = 1..a holds in-flight tokens at depth
    a - l, the tree form of [SPD] 3.1 Eq. (2) and 3.3 (pre-step depths).
    """
    lv = tree_levels(anc)
    if not 1 <= a <= n or max(lv) > a:
        raise ValueError("need 1 <= a <= n and no level deeper than a")
    rows = [pos0 + i for i in range(len(anc))]
    depth = [n if l == 0 else a - l for l in lv]
    pos = [pos0 + l for l in lv]
    return rows, depth, pos


def pdm_step_tree(g_rows, pos0, cache: PdmCache, layers, final_norm, c: PdmConfig, anc):
    """Tree-masked incremental PDM.  Node i sits at position pos0 + level(i) and
    attends to the cached positions < pos0 and to the nodes on its own root
    path (anc[i]); its key/value entries occupy cache slot pos0 + i (a branched
    cache: siblings share a position but not a slot).  Afterwards the cache holds
    slots 0..pos0+M-1.  Returns (final-normed rows [M][d], un-normed rows)."""
    h = np.asarray(g_rows, dtype=np.float64)
    M = h.shape[0]
    lv = tree_levels(anc)
    if len(lv) != M:
        raise ValueError("one mask per row")
    positions = [pos0 + l for l in lv]
    allowed = np.array([[True] * pos0 + [bool((int(anc[i]) >> j) & 1) for j in range(M)]
                        for i in range(M)])
    for li, lw in enumerate(layers):
        kp, vp = cache.k[li][:pos0], cache.v[li][:pos0]
        if kp.shape[0] != pos0:
            raise ValueError("cache does not cover the positions before pos0")
        h, k, v = decoder_layer(h, positions, lw, c, (kp, vp, range(pos0)), allowed=allowed)
        cache.k[li] = np.concatenate([kp, k], axis=0)
        cache.v[li] = np.concatenate([vp, v], axis=0)
    return rms_norm(h, final_norm, c.eps), h


def top_k_list(logits, k):
    """The k largest logits' indices in descending order (equal values by
    ascending index, NaN last): the W children a greedy draft tree gives a
    node (EAGLE-style top-k expansion, [SPD] 4 draft-tree paragraph)."""
    x = np.asarray(logits, dtype=np.float64)
    nan = np.isnan(x)
    order = np.lexsort((np.arange(len(x)), -np.where(nan, 0.0, x), nan))
    return [int(i) for i in order[:max(int(k), 1)]]


def verify_siblings(p_logits, cand):
    """Greedy verification of sibling candidates for one position ([SPD] 3.4 at
    T = 0 applied to a tree level): the sibling equal to the target argmax is
    accepted.  Returns (index of the accepted sibling, -1) or, when none
    matches, (-1, the argmax as the corrected token)."""
    best = argmax_first(p_logits)
    for i, x in enumerate(cand):
        if int(x) == best:
            return i, -1
    return -1, best


def sibling_weights(p32):
    """floor(p * 2^51) of an fp32 probability row as Python integers (entries
    that are not positive, NaN included, weigh 0)."""
    p = np.asarray(p32, dtype=np.float32).astype(np.float64)
    p = np.where(p > 0, p, 0.0)
    return [int(v) for v in np.floor(p * 2.0 ** 51)]


def verify_siblings_sampled(p32, q32, cand, words):
    """Stochastic verification of W sibling candidates drawn independently from q
    (the multi-round form of [SD]'s acceptance criterion, as in SpecInfer's
    multi-candidate speculative sampling): round i tests candidate x_i against the
    current target p_i with r <= min(1, p_i(x)/q(x)); a rejection replaces the
    target by the normalised residual max(0, p_i - q); after W rejections the token
    is drawn from the last residual.  The output is distributed as p.

    Integer form, exact on both sides: A = floor(p 2^51), B = floor(q 2^51),
    p_i = A/sum(A), q = B/sum(B).  Round i accepts x_i iff
    (R_i + 1) B(x_i) sum(A) <= 2^24 A(x_i) sum(B) with R_i = words[i][0] >> 40
    (a candidate outside the vocabulary is rejected).  On rejection
    D = max(0, A sum(B) - B sum(A)) and A = D >> s, s = max(0, bitlength(sum D) - 52),
    which keeps sum(A) below 2^52.  After W rejections the token is the inverse-CDF
    draw from A with u = words[W][1] >> 32 (from floor(p 2^51) if A sums to 0).
    Returns (index of the accepted candidate, -1) or (-1, drawn token).
    """
    A = sibling_weights(p32)
    B = sibling_weights(q32)
    SB = sum(B)
    V = len(A)
    for i, x in enumerate(cand):
        SA = sum(A)
        x = int(x)
        R1 = (int(words[i][0]) >> 40) + 1
        if 0 <= x < V and R1 * B[x] * SA <= (1 << 24) * A[x] * SB:
            return i, -1
        D = [max(0, a * SB - b * SA) for a, b in zip(A, B)]
        s = max(0, sum(D).bit_length() - 52)
        A = [d >> s for d in D]
    if sum(A) == 0:
        A = sibling_weights(p32)
    t = sample_weights(np.array(A, dtype=np.uint64), int(words[len(cand)][1]) >> 32)
    return -1, 0 if t is None else t


# --------------------------------------------------------------------------
# Heads, sampling and verification ([SPD] 3.1, 3.4; [SD] four-phase loop and
# acceptance criterion)
# --------------------------------------------------------------------------

def lm_logits(w_lm, h):
    """logits = W_lm h for a final-normed hidden row h."""
    return np.asarray(w_lm, dtype=np.float64) @ np.asarray(h, dtype=np.float64)


def argmax_first(x):
    """Greedy choice: the lowest index attaining the maximum; NaN never wins."""
    x = np.asarray(x, dtype=np.float64)
    x = np.where(np.isnan(x), -np.inf, x)
    return int(np.argmax(x))


def softmax(logits, temperature):
    z = np.asarray(logits, dtype=np.float64) / float(temperature)
    z = z - z.max()
    e = np.exp(z)
    return e / e.sum()


def top_k_set(logits, k):
    """Ascending indices of the top-k filter's support ([SPD] 4, evaluation
    setting: sampling runs use top-k = 50).

    The k largest logits, a total order on (value descending, index ascending),
    NaN below every number; -0 and +0 are equal values.  k <= 0 or k >= V keeps
    every index.
    """
    x = np.asarray(logits, dtype=np.float64)
    V = len(x)
    if k <= 0 or k >= V:
        return np.arange(V)
    nan = np.isnan(x)
    key = np.where(nan, 0.0, x)
    order = np.lexsort((np.arange(V), -key, nan))   # last key is the primary one
    return np.sort(order[:k])


def filtered_softmax(logits, temperature, top_k=0, top_p=1.0):
    """Sampling distribution after the top-k and top-p filters, zero outside
    the kept set ([SPD] 4 evaluation setting: T = 1, top-k = 50, top-p = 1.0).

    top-k: softmax(logits / T) restricted to top_k_set(logits, top_k) and
    renormalised (top_k = 0: no filter).
    top-p (nucleus, when 0 < top_p < 1; applied after top-k, or over the whole
    vocabulary when top_k = 0): order the kept tokens by probability (descending;
    probability is increasing in the logit, so this is the logit order, equal
    logits by ascending index), keep the shortest prefix whose mass reaches
    top_p, renormalise over it.
    """
    x = np.asarray(logits, dtype=np.float64)
    keep = top_k_set(x, top_k)
    z = x[keep] / float(temperature)
    e = np.exp(z - z.max())
    pk = e / e.sum()
    if 0.0 < top_p < 1.0:
        order = np.lexsort((keep, -x[keep]))         # logit desc, index asc
        before = np.concatenate(([0.0], np.cumsum(pk[order])[:-1]))
        m = int(np.count_nonzero(before < top_p))    # prefix mass before a kept token < top_p
        sub = np.sort(order[:m])
        keep, e = keep[sub], e[sub]
        pk = e / e.sum()
    p = np.zeros(len(x))
    p[keep] = pk
    return p


def prob_weights(p32):
    """Exact integer weights of an fp32 probability row: floor(p * 2^52).
    Non-positive and NaN entries weigh 0."""
    p = np.asarray(p32, dtype=np.float32).astype(np.float64)
    p = np.where(p > 0, p, 0.0)  # NaN compares false -> 0
    return np.floor(p * _TWO52).astype(np.uint64)


def sample_weights(w, u32):
    """Inverse-CDF draw from non-negative integer weights with a 32-bit uniform.

    tau = floor(u * S / 2^32); the result is the smallest j whose inclusive
    prefix sum exceeds tau.  Returns None when every weight is zero.
    Each j is returned for exactly the u in an interval of length ~w_j*2^32/S.
    """
    w = np.asarray(w, dtype=np.uint64)
    total = int(w.sum(dtype=np.uint64))
    if total == 0:
        return None
    tau = (int(u32) * total) >> 32
    csum = np.cumsum(w, dtype=np.uint64)
    return int(np.searchsorted(csum, np.uint64(tau), side="right"))


def sample_probs(p32, u32):
    """Draw from an fp32 probability row (O7 of the design: integer weights)."""
    j = sample_weights(prob_weights(p32), u32)
    if j is None:
        raise ValueError("probability row has no positive entry")
    return j


def accept_test(p_x, q_x, r24):
    """Exact form of 'accept iff r <= min(1, p(x)/q(x))' with r = (R + 1) / 2^24.

    R is a 24-bit integer, so r is uniform on the lattice (0, 1]: p >= q always
    accepts and p = 0 never does.  (R+1)*q (25 x 24 bits) fits a double's
    mantissa exactly, so (R+1)*q <= p*2^24 is decided without rounding.
    q(x) = 0 accepts.
    """
    R1 = float(int(r24) + 1)
    q = float(np.float32(q_x))
    p = float(np.float32(p_x))
    return R1 * q <= p * 16777216.0


def residual_weights(p32, q32):
    """Integer residual max(0, P - Q) of the fp32 rows ([SD] residual p')."""
    P = prob_weights(p32)
    Q = prob_weights(q32)
    return np.where(P > Q, P - Q, np.uint64(0)).astype(np.uint64)


def verify(p, q, draft, words, *, temperature, bonus):
    """Speculative-sampling verify of one sequence.

    p:     [gamma+bonus][V] fp32 target probabilities (T>0) or target logits (T=0)
    q:     [gamma][V]       fp32 draft probabilities (unused at T=0)
    draft: [gamma]          drafted tokens
    words: [gamma+1][2]     uint64 random words; word 0 of row j gives the
                            accept uniform of position j (its top 24 bits),
                            word 1 gives the resample/bonus uniform (top 32 bits).
    Returns (n_accept, next_token) with next_token = -1 when none is produced.

    T = 0 ([SPD] 3.4): accept iff the drafted token is the target argmax; on the
    first mismatch the argmax is the corrected token.
    T > 0 ([SD] acceptance criterion): accept position j iff
    r_j <= min(1, p_j(x_j)/q_j(x_j)); at the first rejection j*, the next token
    is drawn from norm(max(0, p_j* - q_j*)) (from p_j* if that residual is
    empty); if all gamma are accepted and a bonus row is present, the next
    token is drawn from p_gamma.
    """
    gamma = len(draft)
    words = np.asarray(words, dtype=np.uint64)
    for j in range(gamma):
        x = int(draft[j])
        if temperature == 0:
            best = argmax_first(p[j])
            if x != best:
                return j, best
        else:
            r24 = int(words[j, 0]) >> 40
            if not accept_test(p[j][x], q[j][x], r24):
                u = int(words[j, 1]) >> 32
                t = sample_weights(residual_weights(p[j], q[j]), u)
                if t is None:
                    t = sample_probs(p[j], u)
                return j, t
    if not bonus:
        return gamma, -1
    if temperature == 0:
        return gamma, argmax_first(p[gamma])
    return gamma, sample_probs(p[gamma], int(words[gamma, 1]) >> 32)


# --------------------------------------------------------------------------
# Cycle state machine ([SPD] 3.4 streaming verification and rollback; metrics
# of [SPD] 4 and the acceptance-length formula of [REV])
# --------------------------------------------------------------------------

@dataclass
class SeqState:
    t: int            # sequence length x_1..x_t
    a: int            # tokens in flight (1..n)
    commits: int = 0  # N: tokens that exited the last stage
    cycles: int = 0   # K: executed pipeline steps
    tokens: list = field(default_factory=list)


def transition(st: SeqState, n: int, drafted: int, verified: bool,
               n_accept: int, next_token: int) -> SeqState:
    """End-of-cycle update.

    Saturated cycle (a = n): the oldest in-flight token exits and is committed
    (N += 1) and its successor was verified.  Accept: the new draft enters
    stage 1 (t += 1, a stays n).  Reject: keep x_1..x_{t-n+1}, discard the n-1
    younger in-flight tokens and this cycle's draft, append the corrected
    token at depth 0 (t = t-n+2, a = 1).
    Partial cycle (a < n): nothing exits or is verified; the draft joins.
    """
    st.cycles += 1
    if verified:
        if st.a != n:
            raise ValueError("only a saturated pipeline verifies")
        st.commits += 1
        if n_accept == 0:
            keep = st.t - n + 1
            del st.tokens[keep:]
            st.tokens.append(int(next_token))
            st.t = keep + 1
            st.a = 1
            return st
    st.tokens.append(int(drafted))
    st.t += 1
    st.a = min(st.a + 1, n)
    return st


def step_acceptance(st: SeqState) -> float:
    """alpha = N / K ([SPD] 4 metrics)."""
    return st.commits / st.cycles


def acceptance_length(st: SeqState, n: int) -> float:
    """L_acc' = (N / K) * n, the zero-draft-cost theoretical speedup ([REV] core
    formulas; [SPD] 4)."""
    return step_acceptance(st) * n


def expected_speedup(alpha: float, gamma: int, c: float) -> float:
    """[SD] theoretical speedup (i.i.d. acceptance alpha, cost ratio c)."""
    return (1.0 - alpha ** (gamma + 1)) / ((1.0 - alpha) * (gamma * c + 1.0))
