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


def _sampled_trajectory(seed_inputs, cycles, words_seed):
    """A T = 1 trajectory of the tiny workload from a saturated start, with the q
    row of every drafted position recorded by the test itself (positions that a
    rollback discards are drafted again and their record replaced)."""
    s = synth.TINY.with_(temperature=1.0)
    ci = make_inputs(s, device="cpu", seed=seed_inputs, T_cap=160)
    om = C.model_from_inputs(ci)
    t0 = s.ctx
    st = O.SeqState(t=t0, a=s.n, tokens=list(range(t0)))
    cache = C.prefill(om, st.t, st.a)
    # the n-1 tokens in flight at the start were drafted before the trajectory: their
    # q rows are seeded stand-ins, given to the oracle's ring and to the record alike
    seed_logits = np.random.default_rng(5).standard_normal((s.n, s.V)) * 3.0
    drafted_q, ring = {}, {}
    for i, pos in enumerate(range(t0 - s.n + 1, t0)):
        row = O.softmax(seed_logits[i], 1.0).astype(np.float32)
        drafted_q[pos] = ring[pos] = row
    words = synth.cycle_words(cycles, seed=words_seed)
    events = []
    for c in range(cycles):
        t, a, toks = st.t, st.a, list(st.tokens)
        out = C.run_cycle(om, st, cache, ring, 1.0, words[c])
        if out.verified:
            events.append(dict(t=t, tokens=toks, out=out, words=words[c],
                               record=dict(drafted_q), q_now=out.q))
        drafted_q[t] = out.q          # this cycle's draft fills position t
        cache.truncate(st.t - 1 - st.a)
    return s, events


def _decision(ev, q):
    x = ev["tokens"][ev["t"] - synth.TINY.n + 1]
    vw = np.asarray(ev["words"], dtype=np.uint64).reshape(2, 2)
    return O.verify([ev["out"].p], [q], [x], vw, temperature=1.0, bonus=False)


def test_sampled_verify_uses_the_row_its_token_was_drafted_from():
    """[SPD] 3.3-3.4: in a saturated cycle at length t the token x_{t-n+2} (0-based
    position t-n+1) is verified, and rejection sampling needs the draft
    distribution it was sampled from -- the q of the cycle that drafted it, n-1
    cycles earlier (not this cycle's q, not a neighbour's).  Every verification of
    a trajectory with rollbacks must use exactly that row, bit for bit, and its
    decision must be the verify rule applied to that row.  Mutations of the row
    choice (this cycle's q; the rows of positions cand-1 and cand+1) change at
    least one decision of the trajectory, so the check can tell them apart."""
    s, events = _sampled_trajectory(seed_inputs=4, cycles=60, words_seed=23)
    n = s.n
    assert len(events) >= 10
    rejected = sum(1 for ev in events if ev["out"].n_accept == 0)
    assert 1 <= rejected < len(events)
    differs = {"current": 0, "previous": 0, "next": 0}
    for ev in events:
        cand = ev["t"] - n + 1
        want = ev["record"][cand]
        assert ev["out"].q_verified is not None
        assert np.array_equal(ev["out"].q_verified.view(np.uint32), want.view(np.uint32))
        assert (ev["out"].n_accept, ev["out"].next_token) == _decision(ev, want)
        mut = {"current": ev["q_now"], "previous": ev["record"].get(cand - 1),
               "next": ev["record"].get(cand + 1)}
        for name, q in mut.items():
            if q is not None and _decision(ev, q) != _decision(ev, want):
                differs[name] += 1
    assert all(v >= 1 for v in differs.values()), differs


def test_sampled_verify_after_a_rollback_uses_the_redrafted_row():
    """After a rejection at length t the sequence is cut to t-n+1 positions plus the
    corrected token, and the next n-1 cycles draft positions t-n+2 .. again; the
    first verification after the refill checks the first of those new drafts
    against the q of its new draft, not the discarded draft that once held the
    same position."""
    s, events = _sampled_trajectory(seed_inputs=4, cycles=60, words_seed=23)
    n = s.n
    checked = 0
    for i, ev in enumerate(events[:-1]):
        if ev["out"].n_accept != 0:
            continue
        nxt = events[i + 1]
        cand = nxt["t"] - n + 1
        assert nxt["t"] == ev["t"] + 1          # n-1 verification-free refill cycles
        old = ev["record"].get(cand)            # what the position held before the cut
        new = nxt["record"][cand]
        assert np.array_equal(nxt["out"].q_verified.view(np.uint32), new.view(np.uint32))
        if old is not None and not np.array_equal(old, new):
            checked += 1
    assert checked >= 1
