"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and its host helpers agree with the oracle."""
import ctypes

import pytest

import synth
from oracle import spd as O
from spd_testlib import ensure_built, header_functions

spd = ensure_built()


def test_header_symbols_are_exported():
    names = header_functions()
    assert len(names) >= 11
    lib = spd.lib()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(spd.EXPORTED)
    for n in names:                      # the binding uses the C names
        if n not in ("spd_status_string", "spd_last_hip_error"):
            assert hasattr(spd, n), n
    assert spd.spd_version() == 3


def _cfg(s, **kw):
    base = dict(L=s.L, n=s.n, m=s.m, d=s.d, Ls=s.Ls, Hq=s.Hq, Hkv=s.Hkv, hd=s.hd, dff=s.dff,
                V=s.V, dtype=s.dtype, anchor_mode=s.anchor_mode, norm_k0=s.norm_k0)
    base.update(kw)
    return spd.make_config(**base)


@pytest.mark.parametrize("name", sorted(synth.SHAPES))
@pytest.mark.parametrize("mode", [O.ZERO_MASK, O.CLAMP_MIN])
def test_slot_table_matches_oracle(name, mode):
    s = synth.SHAPES[name].with_(anchor_mode=mode)
    tab, layers = spd.spd_slot_table(_cfg(s), s.anchors)
    assert layers == O.store_layers_for(s.L, s.n, s.anchors, mode)
    for k in range(s.n + 1):
        want = O.slot_layers(k, s.L, s.n, s.anchors, mode)
        got = [layers[x] if x >= 0 else -1 for x in tab[k * s.m:(k + 1) * s.m]]
        assert got == want, (k, got, want)


@pytest.mark.parametrize("name", ["tiny_fp32_n4", "qwen35_4b_n8_ls2_t1_mix", "qwen35_9b_n16_ls4_t1"])
@pytest.mark.parametrize("mode", [O.ZERO_MASK, O.CLAMP_MIN])
@pytest.mark.parametrize("schedule", [O.POST_STEP, O.FIRST_STAGE])
def test_slot_table_schedules_match_oracle(name, mode, schedule):
    s = synth.SHAPES[name].with_(anchor_mode=mode)
    tab, layers = spd.spd_slot_table(_cfg(s, feature_schedule=schedule), s.anchors)
    assert layers == O.store_layers_for(s.L, s.n, s.anchors, mode)   # same store for every schedule
    for k in range(s.n + 1):
        want = O.slot_layers(O.feature_depth(k, s.n, schedule), s.L, s.n, s.anchors, mode)
        got = [layers[x] if x >= 0 else -1 for x in tab[k * s.m:(k + 1) * s.m]]
        assert got == want, (k, got, want)


def test_config_rejects_unknown_schedule():
    s = synth.TINY
    with pytest.raises(spd.SpdError):
        spd.spd_slot_table(_cfg(s, feature_schedule=3), s.anchors)


@pytest.mark.parametrize("top_k,top_p", [(-1, 1.0), (spd.SPD_TOP_K_MAX + 1, 1.0), (50, 1.5),
                                         (50, -0.1), (50, float("nan"))])
def test_config_rejects_bad_sampling_filters(top_k, top_p):
    s = synth.TINY
    with pytest.raises(spd.SpdError):
        spd.spd_slot_table(_cfg(s, top_k=top_k, top_p=top_p), s.anchors)


def test_config_rejects_negative_head_workgroups():
    s = synth.TINY
    with pytest.raises(spd.SpdError):
        spd.spd_slot_table(_cfg(s, head_workgroups=-1), s.anchors)


def test_lm_head_workspace_holds_top_k_candidates():
    s = synth.HEADLINE
    base = spd.spd_workspace_size(spd.SPD_CALL_LM_HEAD, _cfg(s), 1)
    for k in (1, 50, spd.SPD_TOP_K_MAX):
        ws = spd.spd_workspace_size(spd.SPD_CALL_LM_HEAD, _cfg(s, top_k=k), 1)
        assert ws >= base + (-(-s.V // 2048)) * k * 8


def test_slot_table_rejects_bad_anchors():
    s = synth.TINY
    with pytest.raises(spd.SpdError):
        spd.spd_slot_table(_cfg(s), [1, 4, 7])
    with pytest.raises(spd.SpdError):
        spd.spd_slot_table(_cfg(s), [0, 7, 4])


@pytest.mark.parametrize("t,a,n", [(32, 4, 4), (32, 1, 4), (2048, 8, 8), (2048, 5, 8), (4096, 16, 16)])
def test_layout_matches_oracle(t, a, n):
    pos, dep = spd.spd_layout(t, a, n)
    pos0, opos, odep = O.cycle_rows(t, a, n)
    assert pos == opos and dep == odep and pos[0] == pos0


@pytest.mark.parametrize("n", [2, 4, 8, 16])
def test_cycle_plan_follows_the_pages(n):
    """The host's cycle plan against the oracle's layout and [SPD] 3.4: a cycle
    verifies iff the pipeline is saturated; then x_{t-n+1} (0-based t-n) exits and
    its successor, drafted n-1 cycles earlier at length t-n+1, is verified.  The
    ring row of a verified token is the row its own draft cycle wrote, and no draft
    in between (nor this cycle's) reuses it."""
    for t in range(n + 1, 3 * n + 4):
        for a in range(1, n + 1):
            p = spd.spd_cycle_plan(t, a, n)
            pos0, pos, _ = O.cycle_rows(t, a, n)
            assert (p.pos0, p.M) == (pos0, len(pos))
            assert p.draft_pos == t and p.ring_draft == t % n
            assert p.verifies == (1 if a == n else 0)
            if a == n:
                assert (p.exiting, p.cand) == (t - n, t - n + 1)
                # the candidate was drafted by the cycle at length cand; the drafts of
                # the n-1 cycles since (lengths cand+1 .. t) wrote other rows
                assert p.ring_cand == spd.spd_cycle_plan(p.cand, 1, n).ring_draft
                assert all(spd.spd_cycle_plan(L, 1, n).ring_draft != p.ring_cand
                           for L in range(p.cand + 1, t + 1))
            else:
                assert (p.exiting, p.cand, p.ring_cand) == (-1, -1, -1)


def test_cycle_plan_rejects_one_stage_and_bad_arguments():
    with pytest.raises(spd.SpdError) as e:
        spd.spd_cycle_plan(5, 1, 1)   # n = 1: the verified token would be this cycle's draft
    assert e.value.status == spd.SPD_E_UNSUPPORTED
    for args in ((5, 0, 4), (5, 5, 4), (4, 4, 4)):
        with pytest.raises(spd.SpdError) as e:
            spd.spd_cycle_plan(*args)
        assert e.value.status == spd.SPD_E_INVALID


def test_cycle_driver_refuses_one_stage():
    """SpdCycle asks the library's plan before it allocates anything: n = 1 is
    refused with a clear error instead of racing the draft against its own
    verification (features and PDM steps of an n = 1 model stay callable)."""
    from pipeline_draft_step_amd.cycle import SpdCycle
    model = type("M", (), {"cfg": _cfg(synth.TINY, n=1)})()
    with pytest.raises(spd.SpdError, match="spd_cycle_plan"):
        SpdCycle(model, 0.0, device="cpu")


def test_lm_head_refuses_nucleus_without_top_k():
    """A nucleus over the whole vocabulary (top_k = 0, 0 < top_p < 1, T > 0) is not
    offered: the call says so instead of sampling from the unfiltered softmax."""
    lib = spd.lib()
    s = synth.HEADLINE
    fake = 1 << 40
    c = _cfg(s, top_k=0, top_p=0.9)
    rc = lib.spd_lm_head(ctypes.byref(c), fake, fake, 1, ctypes.c_float(1.0), fake, fake, fake,
                         fake, fake, 16, None)
    assert rc == spd.SPD_E_UNSUPPORTED
    for kw, T in ((dict(top_k=50, top_p=0.9), 1.0), (dict(top_k=0, top_p=1.0), 1.0),
                  (dict(top_k=0, top_p=0.9), 0.0)):
        c = _cfg(s, **kw)
        rc = lib.spd_lm_head(ctypes.byref(c), fake, fake, 1, ctypes.c_float(T), fake, fake, fake,
                             fake, fake, 16, None)
        assert rc == spd.SPD_E_WORKSPACE, (kw, T)   # past the filter check, stopped by ws size


def test_prepared_feature_calls_check_their_arguments():
    """spd_fc_prepare is bf16 only and needs all three buffers; the prepared feature
    call needs its extra weights and otherwise checks what spd_fuse_features checks
    (every case returns on the host)."""
    lib = spd.lib()
    fake = 1 << 40
    c16 = _cfg(synth.HEADLINE)
    assert lib.spd_fc_prepare(ctypes.byref(c16), fake, None, fake, None) == spd.SPD_E_INVALID
    assert lib.spd_fc_prepare(ctypes.byref(c16), fake, fake, fake + 8, None) == spd.SPD_E_INVALID
    c32 = _cfg(synth.TINY)
    assert lib.spd_fc_prepare(ctypes.byref(c32), fake, fake, fake, None) == spd.SPD_E_UNSUPPORTED
    s = synth.TINY
    tab = (ctypes.c_int32 * ((s.n + 1) * s.m))(*([0] * ((s.n + 1) * s.m)))
    rc = lib.spd_fuse_features_scaled(ctypes.byref(c32), fake, 64, 3, tab, 0, 5, 4, fake, fake, None,
                                      fake, fake, 1 << 30, None)
    assert rc == spd.SPD_E_INVALID        # no prepared weights
    rc = lib.spd_fuse_features_scaled(ctypes.byref(c32), fake, 64, 3, tab, 0, 5, 4, fake, fake, fake,
                                      fake, fake, 16, None)
    assert rc == spd.SPD_E_WORKSPACE
    rc = lib.spd_fuse_features_scaled(ctypes.byref(c32), fake, 64, 3, tab, 62, 5, 4, fake, fake, fake,
                                      fake, fake, 1 << 30, None)
    assert rc == spd.SPD_E_INVALID        # pos0 + M > T_cap


def test_prepared_pdm_calls_check_their_arguments():
    """The prepared e4m3 weights exist for bf16, hd = 128, d and dff multiples of 128:
    their size (per layer: W_qkv, W_gate_up and W_down bytes plus one scale byte per
    row), and the host-side checks of spd_pdm_prepare and spd_pdm_step_prepared (every
    case returns before anything is enqueued)."""
    lib = spd.lib()
    fake = 1 << 40
    s = synth.HEADLINE
    c16 = _cfg(s)
    nq = (s.Hq + 2 * s.Hkv) * s.hd
    rows = nq + 2 * s.dff + s.d
    nbytes = spd.spd_pdm_prepared_bytes(c16)
    per_layer = nq * s.d + 2 * s.dff * s.d + s.d * s.dff + rows
    assert per_layer * s.Ls <= nbytes <= (per_layer + 6 * 256) * s.Ls
    c32 = _cfg(synth.TINY)
    assert spd.spd_pdm_prepared_bytes(c32) == 0
    lw = (spd.spd_layer_weights * s.Ls)()
    for i in range(s.Ls):
        for k, _ in spd.spd_layer_weights._fields_:
            setattr(lw[i], k, fake)
    assert lib.spd_pdm_prepare(ctypes.byref(c16), lw, None, nbytes, None) == spd.SPD_E_INVALID
    assert lib.spd_pdm_prepare(ctypes.byref(c16), lw, fake, nbytes - 1, None) == spd.SPD_E_WORKSPACE
    assert lib.spd_pdm_prepare(ctypes.byref(c16), lw, fake + 8, nbytes, None) == spd.SPD_E_INVALID
    assert lib.spd_pdm_prepare(ctypes.byref(c32), lw, fake, nbytes, None) == spd.SPD_E_UNSUPPORTED
    lw[0].w_down = None
    assert lib.spd_pdm_prepare(ctypes.byref(c16), lw, fake, nbytes, None) == spd.SPD_E_INVALID
    lw[0].w_down = fake
    T_cap = 2112
    ws = spd.spd_workspace_size(spd.SPD_CALL_PDM, c16, 2048, 0, T_cap)
    step = lib.spd_pdm_step_prepared
    assert step(ctypes.byref(c16), lw, fake, nbytes - 1, fake, fake, fake, T_cap, fake, 0, 2048, fake, fake, ws,
                None) == spd.SPD_E_WORKSPACE
    assert step(ctypes.byref(c16), lw, fake + 8, nbytes, fake, fake, fake, T_cap, fake, 0, 2048, fake, fake, ws,
                None) == spd.SPD_E_INVALID
    assert step(ctypes.byref(c16), lw, fake, nbytes, fake, fake, fake, T_cap, fake, 100, 2048, fake, fake, ws,
                None) == spd.SPD_E_INVALID  # pos0 + M > T_cap
    assert step(ctypes.byref(c16), lw, fake, nbytes, fake, fake, fake, T_cap, fake, 0, 2048, fake, fake, 16,
                None) == spd.SPD_E_WORKSPACE
    s32 = synth.TINY
    lw32 = (spd.spd_layer_weights * s32.Ls)()
    for i in range(s32.Ls):
        for k, _ in spd.spd_layer_weights._fields_:
            setattr(lw32[i], k, fake)
    ws32 = spd.spd_workspace_size(spd.SPD_CALL_PDM, c32, 5, 0, 64)
    assert step(ctypes.byref(c32), lw32, fake, 1 << 30, fake, fake, fake, 64, fake, 0, 5, fake, fake, ws32,
                None) == spd.SPD_E_INVALID  # fp32 takes no prepared weights


def test_layout_rejects_bad_arguments():
    for args in ((5, 0, 4), (5, 5, 4), (4, 4, 4)):
        with pytest.raises(spd.SpdError):
            spd.spd_layout(*args)


def test_workspace_sizes():
    s = synth.HEADLINE
    c = _cfg(s)
    for call in (spd.SPD_CALL_FUSE, spd.SPD_CALL_PDM, spd.SPD_CALL_LM_HEAD):
        a = spd.spd_workspace_size(call, c, 9, 0, 2112)
        b = spd.spd_workspace_size(call, c, 256, 0, 2112) if call != spd.SPD_CALL_LM_HEAD else a
        assert a >= 256 and b >= a
    assert spd.spd_workspace_size(spd.SPD_CALL_VERIFY, c, 64, 7) >= 64 * 75 * 64
    assert spd.spd_workspace_size(99, c, 1) == 0
    assert spd.spd_workspace_size(spd.SPD_CALL_FUSE, c, 0) == 0


def test_argument_errors_return_before_any_launch():
    """Invalid arguments are rejected on the host (no device needed)."""
    lib = spd.lib()
    s = synth.TINY
    c = _cfg(s)
    tab = (ctypes.c_int32 * ((s.n + 1) * s.m))(*([0] * ((s.n + 1) * s.m)))
    rc = lib.spd_fuse_features(ctypes.byref(c), None, 64, 3, tab, 0, 5, 4, None, None, None, None,
                               0, None)
    assert rc == spd.SPD_E_INVALID
    fake = 1 << 40   # never dereferenced: the size check fails first
    rc = lib.spd_fuse_features(ctypes.byref(c), fake, 64, 3, tab, 0, 5, 4, fake, fake, fake, fake,
                               16, None)
    assert rc == spd.SPD_E_WORKSPACE
    rc = lib.spd_fuse_features(ctypes.byref(c), fake, 64, 3, tab, 62, 5, 4, fake, fake, fake, fake,
                               1 << 30, None)
    assert rc == spd.SPD_E_INVALID        # pos0 + M > T_cap
    bad = _cfg(s, hd=48)
    lw = (spd.spd_layer_weights * 1)()
    for k, _ in spd.spd_layer_weights._fields_:
        setattr(lw[0], k, fake)
    rc = lib.spd_pdm_step(ctypes.byref(bad), lw, fake, fake, fake, 64, fake, 0, 5, fake, fake,
                          1 << 30, None)
    assert rc == spd.SPD_E_UNSUPPORTED
    rc = lib.spd_lm_head(ctypes.byref(c), fake, fake, 17, ctypes.c_float(0.0), None, fake, None,
                         fake, fake, 1 << 30, None)
    assert rc == spd.SPD_E_INVALID        # rows > 16
    rc = lib.spd_lm_head(ctypes.byref(c), fake, fake, 1, ctypes.c_float(1.0), None, fake, None,
                         fake, fake, 1 << 30, None)
    assert rc == spd.SPD_E_INVALID        # T > 0 needs probs and words
    rc = lib.spd_verify(0, 1, 10, ctypes.c_float(1.0), 0, fake, fake, fake, fake, fake, fake, fake,
                        1 << 30, None)
    assert rc == spd.SPD_E_INVALID
    rc = lib.spd_verify(1, 1, 10, ctypes.c_float(1.0), 0, fake, fake, fake, fake, fake, fake, fake,
                        16, None)
    assert rc == spd.SPD_E_WORKSPACE
    rc = lib.spd_rollback(None, 4, fake, fake, fake, fake, 64, None)
    assert rc == spd.SPD_E_INVALID
    assert spd.status_string(spd.SPD_E_WORKSPACE) == "workspace too small"


def test_tree_and_sibling_argument_errors():
    """The draft-tree calls reject bad masks pointers, node counts, output counts and
    candidate counts on the host."""
    lib = spd.lib()
    s = synth.TINY
    c = _cfg(s)
    tab = (ctypes.c_int32 * ((s.n + 1) * s.m))(*([0] * ((s.n + 1) * s.m)))
    fake = 1 << 40
    for anc, M, a in ((None, 5, 2), (fake + 4, 5, 2), (fake, spd.SPD_TREE_MAX_NODES + 1, 2),
                      (fake, 5, 0)):
        rc = lib.spd_fuse_features_tree(ctypes.byref(c), fake, 256, 3, tab, 0, M, a, anc, fake,
                                        fake, fake, fake, 1 << 30, None)
        assert rc == spd.SPD_E_INVALID, (anc, M, a)
    lw = (spd.spd_layer_weights * 1)()
    for k, _ in spd.spd_layer_weights._fields_:
        setattr(lw[0], k, fake)
    for anc, M, n_out in ((None, 5, 1), (fake + 2, 5, 1), (fake, 65, 1), (fake, 5, 0), (fake, 5, 6)):
        rc = lib.spd_pdm_step_tree(ctypes.byref(c), lw, fake, fake, fake, 256, fake, 0, M, anc,
                                   n_out, fake, fake, 1 << 30, None)
        assert rc == spd.SPD_E_INVALID, (anc, M, n_out)
    for B, W, T, q, words in ((0, 4, 0.0, None, None), (1, 0, 0.0, None, None),
                              (1, spd.SPD_TREE_MAX_NODES + 1, 0.0, None, None),
                              (1, 4, 1.0, None, fake), (1, 4, 1.0, fake, None),
                              (1, 4, -1.0, fake, fake)):
        rc = lib.spd_verify_siblings(B, W, 100, ctypes.c_float(T), fake, q, fake, words, fake,
                                     fake, fake, 1 << 30, None)
        assert rc == spd.SPD_E_INVALID, (B, W, T)
    rc = lib.spd_verify_siblings(1, 4, 100, ctypes.c_float(0.0), fake, None, fake, None, fake,
                                 fake, fake, 16, None)
    assert rc == spd.SPD_E_WORKSPACE


def test_missing_library_fails_loudly(monkeypatch):
    """No fallback: without libspd.so every binding raises instead of computing."""
    monkeypatch.setattr(spd, "_lib", None)
    monkeypatch.setattr(spd, "LIB_PATH", spd.LIB_PATH + ".absent")
    with pytest.raises(RuntimeError, match="missing"):
        spd.lib()
    with pytest.raises(RuntimeError, match="missing"):
        spd.spd_layout(32, 4, 4)
    with pytest.raises(RuntimeError, match="missing"):
        spd.spd_slot_table(_cfg(synth.TINY), synth.TINY.anchors)


def test_product_package_never_reaches_the_oracle():
    """The package and bench's timed path import nothing from oracle/ (only the
    tests, smoke() and the CPU-baseline leg may)."""
    import ast
    import os
    pkg = os.path.dirname(spd.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if not f.endswith(".py"):
                continue
            tree = ast.parse(open(os.path.join(root, f)).read())
            for node in ast.walk(tree):
                names = []
                if isinstance(node, ast.Import):
                    names = [a.name for a in node.names]
                elif isinstance(node, ast.ImportFrom):
                    names = [node.module or ""]
                for n in names:
                    assert not n.split(".")[0] == "oracle", (f, n)


# ---- property tests: the library's host helpers against the oracle on drawn configurations
from hypothesis import given, settings, strategies as st  # noqa: E402


@st.composite
def _eligibility_configs(draw):
    L = draw(st.integers(1, 96))
    n = draw(st.integers(1, min(32, 4 * L)))
    m = draw(st.integers(1, min(8, L + 1)))
    rest = sorted(draw(st.sets(st.integers(1, L), min_size=m - 1, max_size=m - 1))) if m > 1 else []
    anchors = [0] + rest
    mode = draw(st.sampled_from([O.ZERO_MASK, O.CLAMP_MIN]))
    schedule = draw(st.sampled_from([O.PRE_STEP, O.POST_STEP, O.FIRST_STAGE]))
    return L, n, anchors, mode, schedule


@settings(max_examples=300, deadline=None)
@given(_eligibility_configs())
def test_slot_table_matches_oracle_on_drawn_configs(c):
    L, n, anchors, mode, schedule = c
    cfg = spd.make_config(L=L, n=n, m=len(anchors), d=64, Ls=1, Hq=1, Hkv=1, hd=16, dff=64, V=64,
                          dtype=0, anchor_mode=mode, feature_schedule=schedule)
    tab, layers = spd.spd_slot_table(cfg, anchors)
    assert layers == O.store_layers_for(L, n, anchors, mode)
    m = len(anchors)
    for k in range(n + 1):
        want = O.slot_layers(O.feature_depth(k, n, schedule), L, n, anchors, mode)
        got = [layers[x] if x >= 0 else -1 for x in tab[k * m:(k + 1) * m]]
        assert got == want, (k, got, want)


@settings(max_examples=300, deadline=None)
@given(st.integers(1, 32).flatmap(lambda n: st.tuples(st.just(n), st.integers(1, n),
                                                      st.integers(0, 5000))))
def test_layout_matches_oracle_on_drawn_cycles(c):
    n, a, extra = c
    t = a + 1 + extra
    pos, dep = spd.spd_layout(t, a, n)
    pos0, opos, odep = O.cycle_rows(t, a, n)
    assert pos == opos and dep == odep and pos[0] == pos0
