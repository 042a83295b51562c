"""One SPD cycle and a trajectory of cycles, composed from oracle.spd.

TEST INFRASTRUCTURE ONLY (same rule as oracle.spd).

The cycle follows "Speculative Pipeline Decoding" (arXiv 2605.30852):
section 3.3 (pre-step features: the PDM runs on the current depth staircase),
section 3.1 Eq. (1) (one next-token draft from the last position), section 3.4
(when the pipeline is saturated the oldest in-flight token exits, the target LM
head forms P of its successor, which is verified; a rejection truncates to
t-n+1 and reseeds stage 1 with the corrected token).  The synthetic target is a
store of per-position hidden states: a position's states do not depend on the
token it holds (there is no target model), and the target's last-layer states
are taken as already final-normed.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import spd as O


@dataclass
class OracleModel:
    """float64 copies of the weights and synthetic target states."""
    L: int
    n: int
    anchors: tuple
    mode: int
    norm_k0: bool
    eps: float
    store_layers: list
    store: np.ndarray        # [T][S][d]
    h_final: np.ndarray      # [T][d]
    fc_norm: np.ndarray
    w_fc: np.ndarray
    layers: list
    final_norm: np.ndarray
    w_dlm: np.ndarray
    w_tlm: np.ndarray
    pdm: O.PdmConfig
    schedule: int = O.PRE_STEP
    top_k: int = 0           # sampling filters of both heads (T > 0)
    top_p: float = 1.0


@dataclass
class CycleOut:
    pos0: int
    depths: list
    g: np.ndarray
    h_last: np.ndarray
    draft_logits: np.ndarray
    q: np.ndarray            # fp32 draft probabilities (T > 0) or None
    drafted: int
    verified: bool
    target_logits: np.ndarray = None
    p: np.ndarray = None
    n_accept: int = -1
    next_token: int = -1
    q_verified: np.ndarray = None   # the q row the verification used (T > 0)


def run_cycle(om: OracleModel, st: O.SeqState, cache: O.PdmCache, ring: dict,
              temperature: float, words: np.ndarray, *, q_override=None,
              probs_from=None) -> CycleOut:
    """Run one cycle from state `st` and apply the end-of-cycle transition.

    words: [4] uint64 block of this cycle: word 0 accept uniform (top 24 bits),
    word 1 resample uniform (top 32 bits), word 2 draft-sampling uniform (top 32
    bits).
    ring: position -> fp32 draft row q of the token drafted at that position.
    q_override: fp32 row to verify against instead of the ring's (independent
    cycles have no ring history).
    probs_from: optional dict with fp32 'q' / 'p' rows to use in place of this
    cycle's own softmax outputs (teacher forcing of the decision functions).
    """
    n = om.n
    pos0, pos, dep = O.cycle_rows(st.t, st.a, n)
    g = O.fuse_features(om.store, om.store_layers, pos, dep, om.fc_norm, om.w_fc,
                        L=om.L, n=n, anchors=om.anchors, mode=om.mode, eps=om.eps,
                        norm_k0=om.norm_k0, schedule=om.schedule)
    h_last, _ = O.pdm_step(g, pos0, cache, om.layers, om.final_norm, om.pdm)
    dl = O.lm_logits(om.w_dlm, h_last)
    if temperature == 0:
        q = None
        drafted = O.argmax_first(dl)
    else:
        q = O.filtered_softmax(dl, temperature, om.top_k, om.top_p).astype(np.float32)
        if probs_from is not None and "q" in probs_from:
            q = probs_from["q"]
        drafted = O.sample_probs(q, int(words[2]) >> 32)
        ring[st.t] = q
    out = CycleOut(pos0=pos0, depths=dep, g=g, h_last=h_last, draft_logits=dl, q=q,
                   drafted=drafted, verified=(st.a == n))
    if out.verified:
        exiting = st.t - n                  # 0-based position of x_{t-n+1}
        cand = exiting + 1                  # the token under verification
        tl = O.lm_logits(om.w_tlm, om.h_final[exiting])
        out.target_logits = tl
        x = st.tokens[cand]
        vwords = np.asarray(words, dtype=np.uint64).reshape(2, 2)
        if temperature == 0:
            na, nt = O.verify([tl], None, [x], vwords, temperature=0, bonus=False)
        else:
            p = O.filtered_softmax(tl, temperature, om.top_k, om.top_p).astype(np.float32)
            if probs_from is not None and "p" in probs_from:
                p = probs_from["p"]
            out.p = p
            # the token under verification was drafted n-1 cycles ago, at the cycle
            # whose length was cand; its draft distribution is the row kept then
            qrow = q_override if q_override is not None else ring[cand]
            out.q_verified = qrow
            na, nt = O.verify([p], [qrow], [x], vwords, temperature=temperature,
                              bonus=False)
        out.n_accept, out.next_token = na, nt
    O.transition(st, n, drafted, out.verified, out.n_accept, out.next_token)
    return out


def prefill(om: OracleModel, t: int, a: int):
    """Build the PDM cache of positions 0..t-a-2 (all at full depth)."""
    cache = O.PdmCache(len(om.layers), om.pdm)
    P = t - 1 - a
    if P > 0:
        g = O.fuse_features(om.store, om.store_layers, list(range(P)), [om.n] * P,
                            om.fc_norm, om.w_fc, L=om.L, n=om.n, anchors=om.anchors,
                            mode=om.mode, eps=om.eps, norm_k0=om.norm_k0, schedule=om.schedule)
        O.pdm_step(g, 0, cache, om.layers, om.final_norm, om.pdm)
    return cache


def _f64(t):
    if t is None:
        return None
    return t.detach().float().cpu().numpy().astype(np.float64)


def model_from_inputs(ci, with_heads=True) -> OracleModel:
    """float64 OracleModel from a synth.CycleInputs (torch tensors on any device)."""
    s = ci.shape
    layers = [{k: _f64(v) for k, v in lw.items()} for lw in ci.layers]
    return OracleModel(
        L=s.L, n=s.n, anchors=tuple(s.anchors), mode=s.anchor_mode, norm_k0=bool(s.norm_k0),
        eps=s.eps, store_layers=list(ci.store_layers), store=_f64(ci.store),
        h_final=_f64(ci.h_final), fc_norm=_f64(ci.fc_norm), w_fc=_f64(ci.w_fc),
        layers=layers, final_norm=_f64(ci.final_norm),
        w_dlm=_f64(ci.w_dlm) if with_heads else None,
        w_tlm=_f64(ci.w_tlm) if with_heads else None,
        pdm=O.PdmConfig(d=s.d, Hq=s.Hq, Hkv=s.Hkv, hd=s.hd, dff=s.dff, eps=s.eps,
                        rope_theta=s.rope_theta),
        schedule=s.feature_schedule, top_k=s.top_k, top_p=s.top_p)
