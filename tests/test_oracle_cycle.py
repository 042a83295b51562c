"""Cycle-level pins of the oracle: the incremental cycle (cached keys/values,
truncation on rollback) equals the definitional draft of Eq. (1) -- the PDM
run over the whole current feature sequence -- on every cycle of a tiny
trajectory, and the state machine follows the rollback rule."""
import numpy as np

import synth
from oracle import cycle as C
from oracle import spd as O
from spd_testlib import make_inputs


def _full_recompute_draft(om, st_before):
    t, a, n = st_before.t, st_before.a, om.n
    dep = O.depths(t, a, n)
    G = O.fuse_features(om.store, om.store_layers, list(range(t)), dep, om.fc_norm, om.w_fc,
                        L=om.L, n=n, anchors=om.anchors, mode=om.mode, eps=om.eps,
                        norm_k0=om.norm_k0)
    h = O.pdm_forward(G, om.layers, om.final_norm, om.pdm)
    return O.argmax_first(O.lm_logits(om.w_dlm, h))


def test_tiny_trajectory_matches_full_recompute():
    s = synth.TINY
    ci = make_inputs(s, device="cpu", seed=0, T_cap=96)
    om = C.model_from_inputs(ci)
    t0 = s.ctx
    st = O.SeqState(t=t0, a=s.n, tokens=list(range(t0)))
    cache = C.prefill(om, st.t, st.a)
    ring = {}
    words = synth.cycle_words(40)
    rejects = 0
    for c in range(40):
        before = O.SeqState(t=st.t, a=st.a)
        want = _full_recompute_draft(om, before)
        out = C.run_cycle(om, st, cache, ring, 0.0, words[c])
        assert out.drafted == want, c
        if out.verified and out.n_accept == 0:
            rejects += 1
            assert st.t == before.t - s.n + 2 and st.a == 1
    assert rejects > 0            # random weights: greedy verify rejects often
    assert st.cycles == 40


def test_sampled_cycle_uses_ring_row():
    s = synth.TINY.with_(temperature=1.0)
    ci = make_inputs(s, device="cpu", seed=1, T_cap=96)
    om = C.model_from_inputs(ci)
    st = O.SeqState(t=s.ctx, a=1, tokens=list(range(s.ctx)))
    cache = C.prefill(om, st.t, st.a)
    ring = {}
    words = synth.cycle_words(30)
    for c in range(30):
        tb, ab = st.t, st.a
        out = C.run_cycle(om, st, cache, ring, 1.0, words[c])
        assert out.q is not None and abs(float(out.q.astype(np.float64).sum()) - 1) < 1e-5
        if out.verified:
            assert ab == s.n
            assert (tb - s.n + 1) in ring
