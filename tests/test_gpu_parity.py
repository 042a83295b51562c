"""GPU parity: every C-ABI call against the CPU oracle on the same seeded inputs.

Floating-point outputs (features, PDM rows, logits, probabilities) must agree to
max|gpu - oracle| / rms(oracle) <= 1e-5 (fp32 path) or 2e-2 (bf16 path).  Token
decisions, accept counts and rollback state must be bit-exact whenever the
decision functions are given identical fp32 rows and random words: the oracle's
decision functions are applied to the rows the GPU produced.
"""
import sys

import numpy as np
import pytest
import torch

import synth
from oracle import cycle as OC
from oracle import spd as O
from spd_testlib import TOL_BF16, TOL_F32, ensure_built, f64, make_inputs, rel_err, tol_for

pytestmark = pytest.mark.gpu

spd = ensure_built()
from pipeline_draft_step_amd.cycle import DeviceWeights, SpdCycle, SpdModel  # noqa: E402

DEV = "cuda"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def device_model(ci):
    s = ci.shape
    w = DeviceWeights(store=ci.store, h_final=ci.h_final, fc_norm=ci.fc_norm, w_fc=ci.w_fc,
                      layers=ci.layers, final_norm=ci.final_norm, w_dlm=ci.w_dlm, w_tlm=ci.w_tlm)
    return SpdModel(L=s.L, n=s.n, anchors=s.anchors, d=s.d, Ls=s.Ls, Hq=s.Hq, Hkv=s.Hkv, hd=s.hd,
                    dff=s.dff, V=s.V, dtype=s.dtype, weights=w, anchor_mode=s.anchor_mode,
                    norm_k0=s.norm_k0, eps=s.eps, rope_theta=s.rope_theta,
                    feature_schedule=s.feature_schedule, top_k=s.top_k, top_p=s.top_p)


def row_depths(M, a, n):
    return [n if r < M - a else M - 1 - r for r in range(M)]


SMALL_BF16 = synth.SpdShape("small_bf16", L=32, n=8, anchors=(0, 8, 16, 24, 31), d=256, Ls=2,
                            Hq=4, Hkv=2, hd=128, dff=512, V=4096, dtype=synth.BF16, ctx=96,
                            temperature=1.0, lm_std=3.0 / 16)
SMALL_BF16_H64 = SMALL_BF16.with_(name="small_bf16_hd64", Hq=8, Hkv=2, hd=64, d=192, dff=384)


# ------------------------------------------------------------------ features

# (t, a) layouts; t = a + 1 is a sequence's first cycle (pos0 = 0), a = 0 a prefill of t rows
FUSE_CASES = [
    ("tiny", synth.TINY, [(32, 4), (32, 1), (32, 3), (28, 0), (5, 4), (2, 1), (1, 0)]),
    ("small_zero", SMALL_BF16, [(96, 8), (96, 3), (96, 1), (80, 0), (9, 8)]),
    ("small_clamp", SMALL_BF16.with_(anchor_mode=synth.CLAMP_MIN), [(96, 8), (96, 5)]),
    ("small_normk0", SMALL_BF16.with_(norm_k0=1), [(96, 8), (96, 2)]),
    # feature-schedule variants (slot-table switches, no kernel change)
    ("small_post_step", SMALL_BF16.with_(feature_schedule=1), [(96, 8), (96, 3), (96, 1)]),
    ("small_first_stage", SMALL_BF16.with_(feature_schedule=2), [(96, 8), (96, 3), (80, 0)]),
    ("small_first_stage_clamp", SMALL_BF16.with_(feature_schedule=2, anchor_mode=synth.CLAMP_MIN),
     [(96, 8), (96, 4)]),
    ("tiny_post_step", synth.TINY.with_(feature_schedule=1), [(32, 4), (32, 2)]),
    ("headline_post_step", synth.HEADLINE.with_(feature_schedule=1), [(2048, 8), (2048, 3)]),
    ("headline", synth.HEADLINE, [(2048, 8), (2048, 3), (2048, 1), (9, 8), (2, 1)]),
    ("4b_n4", synth.SHAPES["qwen35_4b_n4_ls1_greedy"], [(2048, 4), (2048, 3), (2048, 1), (5, 4)]),
    ("9b", synth.SHAPES["qwen35_9b_n16_ls4_t1"], [(4096, 16), (4096, 7), (4096, 1)]),
]


@pytest.mark.parametrize("name,shape,layouts", FUSE_CASES, ids=[c[0] for c in FUSE_CASES])
def test_fuse_features(name, shape, layouts):
    ci = make_inputs(shape, device=DEV, with_heads=False)
    model = device_model(ci)
    cyc = SpdCycle(model, shape.temperature)
    om = OC.model_from_inputs(ci, with_heads=False)
    for (t, a) in layouts:
        M = a + 1 if a > 0 else t
        pos0 = t - 1 - a if a > 0 else 0
        say(name, "fuse", t, a, M)
        out = torch.empty(M, shape.d, device=DEV)
        cyc.features(pos0, M, a, out=out)
        torch.cuda.synchronize()
        ref = O.fuse_features(om.store, om.store_layers, list(range(pos0, pos0 + M)),
                              row_depths(M, a, shape.n), om.fc_norm, om.w_fc, L=shape.L, n=shape.n,
                              anchors=shape.anchors, mode=shape.anchor_mode, eps=shape.eps,
                              norm_k0=bool(shape.norm_k0), schedule=shape.feature_schedule)
        err = rel_err(f64(out), ref)
        assert err < tol_for(shape.dtype), (t, a, err)


def test_fuse_features_drawn_configs():
    """20 drawn feature configurations (anchor sets, both anchor modes, the three
    schedules, norm_k0, fp32/bf16, widths, in-flight counts and prefixes, including
    a sequence's first cycle) against the oracle."""
    rng = np.random.default_rng(321)
    for case in range(20):
        L = int(rng.integers(2, 40))
        n = int(rng.integers(1, min(16, L) + 1))
        m = int(rng.integers(1, min(8, L + 1) + 1))
        anchors = tuple([0] + sorted(rng.choice(np.arange(1, L + 1), size=m - 1, replace=False).tolist()))
        mode = int(rng.integers(0, 2))
        sched = int(rng.integers(0, 3))
        dtype = int(rng.integers(0, 2))
        d = 64 * int(rng.integers(1, 5))
        a = int(rng.integers(0, n + 1))
        t = a + 1 + int(rng.integers(0, 60)) if a > 0 else int(rng.integers(1, 41))
        shape = synth.SpdShape(f"fdrawn{case}", L=L, n=n, anchors=anchors, d=d, Ls=1, Hq=1, Hkv=1,
                               hd=16, dff=64, V=64, dtype=dtype, ctx=t, temperature=0.0, lm_std=0.02,
                               anchor_mode=mode, norm_k0=int(rng.integers(0, 2)), feature_schedule=sched)
        M = a + 1 if a > 0 else t
        pos0 = t - 1 - a if a > 0 else 0
        say("fuse drawn", case, dict(L=L, n=n, anchors=anchors, mode=mode, sched=sched, dtype=dtype, d=d,
                                     t=t, a=a))
        ci = make_inputs(shape, device=DEV, with_heads=False, T_cap=(t + 15) // 8 * 8, seed=case)
        model = device_model(ci)
        om = OC.model_from_inputs(ci, with_heads=False)
        out = torch.empty(M, d, device=DEV)
        # the feature call alone (n = 1 is drawn too: a valid feature call, though the
        # cycle driver refuses it)
        ws = torch.zeros(spd.spd_workspace_size(spd.SPD_CALL_FUSE, model.cfg, M), dtype=torch.uint8,
                         device=DEV)
        spd.spd_fuse_features(model.cfg, ci.store, model.T_cap, len(model.store_layers), model.slot_tab,
                              pos0, M, a, ci.fc_norm, ci.w_fc, out, ws)
        torch.cuda.synchronize()
        ref = O.fuse_features(om.store, om.store_layers, list(range(pos0, pos0 + M)), row_depths(M, a, n),
                              om.fc_norm, om.w_fc, L=L, n=n, anchors=anchors, mode=mode, eps=shape.eps,
                              norm_k0=bool(shape.norm_k0), schedule=sched)
        assert rel_err(f64(out), ref) < tol_for(dtype), case


PREFILL_FUSE_CASES = [
    # (name, shape, M, rows checked: None = all)
    ("small_prefill", SMALL_BF16.with_(ctx=320), 300, None),
    ("small_prefill_h64", SMALL_BF16_H64.with_(ctx=600), 520, None),
    ("headline_prefill", synth.HEADLINE, 2048, 48),
    ("headline_prefill_ragged", synth.HEADLINE, 2039, 24),
]


@pytest.mark.parametrize("prepared", [False, True], ids=["gather", "prepared"])
@pytest.mark.parametrize("name,shape,M,nsample", PREFILL_FUSE_CASES,
                         ids=[c[0] for c in PREFILL_FUSE_CASES])
def test_fuse_features_prefill(name, shape, M, nsample, prepared):
    """Prefill-sized calls (every row at depth n) take the MFMA-tiled large-M GEMM:
    split-K partial tiles, ragged M and N tiles; either after the gather launch
    (spd_fuse_features) or, with the prepared weights (spd_fuse_features_scaled),
    straight from the anchor store with the row statistics formed in the product.
    The full headline product is checked on sampled rows (tile edges included),
    which the oracle computes one by one."""
    ci = make_inputs(shape, device=DEV, with_heads=False)
    model = device_model(ci)
    cyc = SpdCycle(model, shape.temperature)
    om = OC.model_from_inputs(ci, with_heads=False)
    say(name, "prefill fuse", M, "prepared" if prepared else "gather")
    out = torch.full((M, shape.d), float("nan"), device=DEV)
    pos0 = 3 if M < 2048 else 0   # the store rows from pos0 (ctx leaves room for it)
    for rep in range(2):  # the second call reuses the arrival counters the first left at zero
        if prepared:
            cyc.features(pos0, M, 0, out=out)
        else:
            spd.spd_fuse_features(model.cfg, model.w.store, model.T_cap, len(model.store_layers),
                                  model.slot_tab, pos0, M, 0, model.w.fc_norm, model.w.w_fc, out, cyc.ws)
    torch.cuda.synchronize()
    if nsample is None:
        rows = list(range(M))
    else:
        rng = np.random.default_rng(5)
        edges = [0, 1, 255, 256, 511, 512, M // 2, M - 2, M - 1]
        rows = sorted(set(edges) | set(int(x) for x in rng.choice(M, nsample, replace=False)))
    ref = O.fuse_features(om.store, om.store_layers, [pos0 + r for r in rows], [shape.n] * len(rows),
                          om.fc_norm, om.w_fc, L=shape.L, n=shape.n, anchors=shape.anchors,
                          mode=shape.anchor_mode, eps=shape.eps, norm_k0=bool(shape.norm_k0))
    got = f64(out)[rows]
    assert np.isfinite(got).all()
    err = rel_err(got, ref)
    assert err < tol_for(shape.dtype), (M, err)


def test_fc_prepare_folds_the_norm_into_the_weights():
    """spd_fc_prepare: every weight times its column's norm weight, rounded to bf16
    once (the fp32 product of two bf16 values is exact), bit for bit."""
    s = synth.HEADLINE
    ci = make_inputs(s, device=DEV, with_heads=False)
    model = device_model(ci)
    say("fc_prepare", tuple(ci.w_fc.shape))
    out = torch.empty_like(ci.w_fc)
    spd.spd_fc_prepare(model.cfg, ci.fc_norm, ci.w_fc, out)
    ref = (ci.w_fc.float() * ci.fc_norm.float()[None, :]).to(torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_prepared_features_fall_back_where_rows_are_not_all_full_depth():
    """With prepared weights, calls that do not qualify for the one-launch form
    (rows in flight, decode sizes) are the gather path exactly."""
    s = synth.HEADLINE
    ci = make_inputs(s, device=DEV, with_heads=False)
    model = device_model(ci)
    cyc = SpdCycle(model, s.temperature)
    for pos0, M, a in ((100, 300, 8), (s.ctx - 9, 9, 8), (s.ctx - 4, 4, 3)):
        say("prepared fallback", pos0, M, a)
        x = torch.empty(M, s.d, device=DEV)
        y = torch.empty(M, s.d, device=DEV)
        cyc.features(pos0, M, a, out=x)
        spd.spd_fuse_features(model.cfg, model.w.store, model.T_cap, len(model.store_layers), model.slot_tab,
                              pos0, M, a, model.w.fc_norm, model.w.w_fc, y, cyc.ws)
        torch.cuda.synchronize()
        assert torch.equal(x, y), (pos0, M, a)


# ------------------------------------------------------------------ PDM step

def _oracle_cache_from(k, v, pos0, shape):
    c = O.PdmCache(shape.Ls, O.PdmConfig(d=shape.d, Hq=shape.Hq, Hkv=shape.Hkv, hd=shape.hd,
                                         dff=shape.dff))
    kk = f64(k)  # [Ls][Hkv][T][hd]
    vv = f64(v)  # [Ls][Hkv][hd][T]
    c.k = [kk[l].transpose(1, 0, 2)[:pos0].copy() for l in range(shape.Ls)]
    c.v = [vv[l].transpose(2, 0, 1)[:pos0].copy() for l in range(shape.Ls)]
    return c


def _check_cache_rows(cyc, cache, lo, hi, tol):
    for l in range(len(cache.k)):
        gk = f64(cyc.k_cache[l]).transpose(1, 0, 2)[lo:hi]
        gv = f64(cyc.v_cache[l]).transpose(2, 0, 1)[lo:hi]
        assert rel_err(gk, cache.k[l][lo:hi]) < tol
        assert rel_err(gv, cache.v[l][lo:hi]) < tol


@pytest.mark.parametrize("shape", [synth.TINY, SMALL_BF16, SMALL_BF16_H64, SMALL_BF16.with_(ctx=320),
                                   synth.HEADLINE],
                         ids=["tiny", "small_bf16", "small_bf16_hd64", "small_bf16_large_m",
                              "headline_large_m"])
def test_pdm_prefill_then_cycle(shape):
    """Prefill through the library, then one saturated and one partial cycle; the
    oracle runs the same rows incrementally (pinned equal to full recompute).
    Prefills of 256 rows or more in bf16 with head size 128 take the large-M
    path (MFMA-tiled GEMMs with bf16 activations, row kernels for the
    epilogues): 311 rows at d = 256 and the headline's 2039 rows at d = 2560,
    every cache row and the final row checked.  bf16 models with d and dff
    multiples of 128 run it with prepared e4m3 weights (the activation residuals'
    products on the fp8 MFMA)."""
    _prefill_then_cycle(shape, prepared=True)


def _excess_over_bf16(dev, ref):
    """max |dev - ref| beyond half a bf16 unit in the last place of ref, over rms(ref):
    the error a computation adds on top of storing its result in bf16."""
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    return float(np.maximum(np.abs(dev - ref) - ulp / 2, 0).max() / np.sqrt((ref ** 2).mean()))


@pytest.mark.parametrize("prepared", [True, False], ids=["prepared", "plain"])
def test_pdm_prefill_9b_shape(prepared):
    """A 2048-row prefill of the 9B-shaped PDM (d = 4096, 4 layers, GQA 32/8): the
    output row within 2e-2; every cache row within 3e-2 beyond its own bf16 storage
    rounding (half a unit in the last place of the exact value; the largest keys sit
    near 6.5 rms, where storage alone costs 0.015 of rms).  The cache is bf16 by
    design and the fp64 oracle's is exact: each layer's attention reads the earlier
    rows' rounded keys and values (every score moves by about 2^-9 of its size), so
    the deeper layers' entries drift further from the exact ones (measured 0.012,
    0.015 and 0.021 beyond storage in layers 1-3, both forms), while the output row
    stays near 0.002."""
    shape = synth.SHAPES["qwen35_9b_n16_ls4_t1"]
    ci = make_inputs(shape, device=DEV, with_heads=False)
    model = device_model(ci)
    model.use_pdm_prep = prepared
    cyc = SpdCycle(model, shape.temperature)
    om = OC.model_from_inputs(ci, with_heads=False)
    P = 2048
    G = synth.normal((P, shape.d), 1.0, device=DEV, seed=9, name="pdm_rows")
    say("9b prefill", prepared)
    cyc.pdm(0, P, g=G)
    torch.cuda.synchronize()
    cache = O.PdmCache(shape.Ls, om.pdm)
    last, _ = O.pdm_step(f64(G), 0, cache, om.layers, om.final_norm, om.pdm)
    assert rel_err(f64(cyc.h_last), last) < TOL_BF16
    for l in range(shape.Ls):
        gk = f64(cyc.k_cache[l]).transpose(1, 0, 2)[:P]
        gv = f64(cyc.v_cache[l]).transpose(2, 0, 1)[:P]
        ek, ev = _excess_over_bf16(gk, cache.k[l][:P]), _excess_over_bf16(gv, cache.v[l][:P])
        say("layer", l, "excess", round(ek, 4), round(ev, 4))
        assert ek < 3e-2 and ev < 3e-2, (l, ek, ev)


@pytest.mark.parametrize("shape", [SMALL_BF16.with_(ctx=320), synth.HEADLINE],
                         ids=["small_bf16_large_m", "headline_large_m"])
def test_pdm_prefill_then_cycle_plain_form(shape):
    """The same prefill and cycles without prepared weights (the residuals' products
    as a second bf16 pass)."""
    _prefill_then_cycle(shape, prepared=False)


def _prefill_then_cycle(shape, prepared):
    ci = make_inputs(shape, device=DEV, with_heads=False)
    model = device_model(ci)
    model.use_pdm_prep = prepared
    cyc = SpdCycle(model, shape.temperature)
    om = OC.model_from_inputs(ci, with_heads=False)
    tol = tol_for(shape.dtype)
    t, n = shape.ctx, shape.n
    G = synth.normal((t + 2, shape.d), 1.0, device=DEV, seed=9, name="pdm_rows")
    Gh = f64(G)
    cache = O.PdmCache(shape.Ls, om.pdm)
    P = t - 1 - n
    say(shape.name, "prefill", P)
    cyc.pdm(0, P, g=G[:P].contiguous())
    torch.cuda.synchronize()
    last, _ = O.pdm_step(Gh[:P], 0, cache, om.layers, om.final_norm, om.pdm)
    assert rel_err(f64(cyc.h_last), last) < tol
    _check_cache_rows(cyc, cache, 0, P, tol)
    for (pos0, M) in ((P, n + 1), (P + 1, 3)):
        say(shape.name, "step", pos0, M)
        rows = G[pos0:pos0 + M].contiguous()
        cyc.pdm(pos0, M, g=rows)
        torch.cuda.synchronize()
        cache.truncate(pos0)
        last, _ = O.pdm_step(Gh[pos0:pos0 + M], pos0, cache, om.layers, om.final_norm, om.pdm)
        assert rel_err(f64(cyc.h_last), last) < tol, (pos0, M)
        _check_cache_rows(cyc, cache, pos0, pos0 + M, tol)


@pytest.mark.parametrize("shape", [synth.HEADLINE, synth.SHAPES["qwen35_4b_n4_ls1_greedy"],
                                   synth.SHAPES["qwen35_9b_n16_ls4_t1"]],
                         ids=["headline", "4b_n4", "9b_n16"])
def test_pdm_full_size_on_synthetic_cache(shape):
    """Full-size PDM step at context t: the committed cache holds seeded values
    (an input of the call), the M new rows are checked against the oracle."""
    ci = make_inputs(shape, device=DEV, with_heads=False)
    model = device_model(ci)
    cyc = SpdCycle(model, shape.temperature)
    om = OC.model_from_inputs(ci, with_heads=False)
    k, v = synth.kv_cache(shape, model.T_cap, device=DEV)
    t, n = shape.ctx, shape.n
    for a in (n, 1):
        cyc.k_cache.copy_(k)       # every step starts from the seeded committed cache
        cyc.v_cache.copy_(v)
        pos0, M = t - 1 - a, a + 1
        say(shape.name, "pdm full", pos0, M)
        g = synth.normal((M, shape.d), 1.0, device=DEV, seed=10 + a, name="rows")
        cyc.pdm(pos0, M, g=g)
        torch.cuda.synchronize()
        cache = _oracle_cache_from(k, v, pos0, shape)
        last, _ = O.pdm_step(f64(g), pos0, cache, om.layers, om.final_norm, om.pdm)
        err = rel_err(f64(cyc.h_last), last)
        assert err < TOL_BF16, (a, err)
        _check_cache_rows(cyc, cache, pos0, pos0 + M, TOL_BF16)


@pytest.mark.parametrize("shape", [synth.TINY, SMALL_BF16, synth.HEADLINE],
                         ids=["tiny", "small_bf16", "headline"])
def test_pdm_step_with_empty_committed_prefix(shape):
    """The first cycle of a sequence: pos0 = 0, so nothing is committed and the M
    rows attend only to each other (M = 1: a row attending to itself alone)."""
    ci = make_inputs(shape, device=DEV, with_heads=False)
    model = device_model(ci)
    cyc = SpdCycle(model, shape.temperature)
    om = OC.model_from_inputs(ci, with_heads=False)
    tol = tol_for(shape.dtype)
    for M in (1, shape.n + 1):
        say(shape.name, "pdm empty prefix", M)
        g = synth.normal((M, shape.d), 1.0, device=DEV, seed=20 + M, name="rows0")
        cyc.pdm(0, M, g=g)
        torch.cuda.synchronize()
        cache = O.PdmCache(shape.Ls, om.pdm)
        last, _ = O.pdm_step(f64(g), 0, cache, om.layers, om.final_norm, om.pdm)
        assert rel_err(f64(cyc.h_last), last) < tol, M
        _check_cache_rows(cyc, cache, 0, M, tol)


def test_pdm_drawn_shapes():
    """16 drawn decoder configurations (fp32 and bf16; head sizes 16..128, GQA ratios
    1..4, widths, 1-2 layers, 1-40 rows over one or two row tiles, committed prefixes
    0..300) on a seeded committed cache: last row and the new cache rows within
    tolerance of the oracle."""
    rng = np.random.default_rng(123)
    for case in range(16):
        dtype = int(rng.integers(0, 2))
        hd = int(rng.choice([32, 64, 128] if dtype == synth.BF16 else [16, 32, 64, 128]))
        Hkv = int(rng.integers(1, 4))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        while (Hq * hd) % 32:
            Hq += Hkv
        d = 64 * int(rng.integers(1, 5))
        dff = 64 * int(rng.integers(1, 9))
        Ls = int(rng.integers(1, 3))
        M = int(rng.integers(1, 41))
        pos0 = int(rng.integers(0, 301))
        T_cap = (pos0 + M + 15) // 8 * 8
        shape = synth.SpdShape(f"drawn{case}", L=8, n=4, anchors=(0, 4, 7), d=d, Ls=Ls, Hq=Hq, Hkv=Hkv,
                               hd=hd, dff=dff, V=64, dtype=dtype, ctx=pos0 + M, temperature=0.0,
                               lm_std=0.02)
        say("pdm drawn", case, dict(dtype=dtype, d=d, Ls=Ls, Hq=Hq, Hkv=Hkv, hd=hd, dff=dff, M=M,
                                    pos0=pos0))
        ci = make_inputs(shape, device=DEV, with_heads=False, T_cap=T_cap, seed=case)
        model = device_model(ci)
        cyc = SpdCycle(model, 0.0)
        om = OC.model_from_inputs(ci, with_heads=False)
        k, v = synth.kv_cache(shape, model.T_cap, device=DEV, seed=50 + case)
        cyc.k_cache.copy_(k)
        cyc.v_cache.copy_(v)
        g = synth.normal((M, d), 1.0, device=DEV, seed=60 + case, name="rows")
        cyc.pdm(pos0, M, g=g)
        torch.cuda.synchronize()
        cache = _oracle_cache_from(k, v, pos0, shape)
        last, _ = O.pdm_step(f64(g), pos0, cache, om.layers, om.final_norm, om.pdm)
        tol = tol_for(dtype)
        assert rel_err(f64(cyc.h_last), last) < tol, case
        _check_cache_rows(cyc, cache, pos0, pos0 + M, tol)


def _prep_layout(s):
    """Byte offsets of the prepared weights of one layer (spd_pdm_prepare's layout:
    W_qkv, W_gate_up, W_down e4m3 rows, then their scale bytes, each 256-aligned)."""
    nq = (s.Hq + 2 * s.Hkv) * s.hd
    off, out = 0, {}
    for key, n in (("qkv8", nq * s.d), ("gu8", 2 * s.dff * s.d), ("dn8", s.d * s.dff), ("qkv_s", nq),
                   ("gu_s", 2 * s.dff), ("dn_s", s.d)):
        out[key] = off
        off = (off + n + 255) // 256 * 256
    out["layer"] = off
    return out


@pytest.mark.parametrize("shape", [synth.HEADLINE, synth.SHAPES["qwen35_9b_n16_ls4_t1"]],
                         ids=["headline", "9b_n16"])
def test_pdm_prepare_writes_scaled_e4m3_rows(shape):
    """spd_pdm_prepare: row n of W_qkv, W_gate_up and W_down becomes the e4m3 value
    (round to nearest even: torch's float8_e4m3fn) of W_n 2^e_n, e_n = 8 - E_n for the
    row's largest magnitude f 2^E_n (0.5 <= f < 1), and its scale byte is 127 - e_n;
    checked bit for bit on every row of every layer."""
    ci = make_inputs(shape, device=DEV, with_heads=False)
    model = device_model(ci)
    prep = model.pdm_prep().cpu()
    L = _prep_layout(shape)
    assert prep.numel() >= L["layer"] * shape.Ls
    for l, lw in enumerate(ci.layers):
        base = l * L["layer"]
        for wkey, k8, ks in (("wqkv", "qkv8", "qkv_s"), ("w_gate_up", "gu8", "gu_s"), ("w_down", "dn8", "dn_s")):
            W = lw[wkey].float().cpu()
            N, K = W.shape
            say("prepare", shape.name, l, wkey)
            m = W.abs().amax(dim=1)
            e = torch.where(m > 0, 8 - torch.frexp(m)[1], torch.zeros_like(m, dtype=torch.int32))
            want = torch.ldexp(W, e[:, None].float()).to(torch.float8_e4m3fn).view(torch.uint8)
            got = prep[base + L[k8]: base + L[k8] + N * K].view(N, K)
            assert torch.equal(got, want), (l, wkey, int((got != want).sum()))
            assert torch.equal(prep[base + L[ks]: base + L[ks] + N].to(torch.int32), (127 - e).to(torch.int32))


def test_large_m_drawn_shapes():
    """Prefill-sized calls on the large-M MFMA path at drawn, ragged sizes: 4 feature
    calls (256..700 rows, anchor counts 2..5, widths 64..256) checked on every row,
    and 4 decoder steps (256..600 rows after a committed prefix of 0..200, head size
    128, GQA 1..4, 1-2 layers) checked on the last row and every new cache row."""
    rng = np.random.default_rng(808)
    for case in range(4):
        m = int(rng.integers(2, 6))
        anchors = tuple([0] + sorted(rng.choice(np.arange(1, 33), size=m - 1, replace=False).tolist()))
        d = 64 * int(rng.integers(1, 5))
        M = int(rng.integers(256, 701))
        shape = synth.SpdShape(f"bigf{case}", L=32, n=8, anchors=anchors, d=d, Ls=1, Hq=1, Hkv=1, hd=16,
                               dff=64, V=64, dtype=synth.BF16, ctx=M, temperature=0.0, lm_std=0.02)
        say("large-M fuse drawn", case, dict(m=m, d=d, M=M))
        ci = make_inputs(shape, device=DEV, with_heads=False, T_cap=(M + 15) // 8 * 8, seed=case)
        model = device_model(ci)
        cyc = SpdCycle(model, 0.0)
        om = OC.model_from_inputs(ci, with_heads=False)
        out = torch.empty(M, d, device=DEV)
        cyc.features(0, M, 0, out=out)
        torch.cuda.synchronize()
        ref = O.fuse_features(om.store, om.store_layers, list(range(M)), [shape.n] * M, om.fc_norm,
                              om.w_fc, L=shape.L, n=shape.n, anchors=anchors, mode=0, eps=shape.eps,
                              norm_k0=False, schedule=0)
        assert rel_err(f64(out), ref) < TOL_BF16, case
    for case in range(4):
        Hkv = int(rng.integers(1, 3))
        Hq = Hkv * int(rng.choice([1, 2, 4]))
        d = 128 * int(rng.integers(1, 4))
        dff = 128 * int(rng.integers(1, 5))
        Ls = int(rng.integers(1, 3))
        M = int(rng.integers(256, 601))
        pos0 = int(rng.integers(0, 201))
        T_cap = (pos0 + M + 15) // 8 * 8
        shape = synth.SpdShape(f"bigp{case}", L=8, n=4, anchors=(0, 4, 7), d=d, Ls=Ls, Hq=Hq, Hkv=Hkv,
                               hd=128, dff=dff, V=64, dtype=synth.BF16, ctx=pos0 + M, temperature=0.0,
                               lm_std=0.02)
        say("large-M pdm drawn", case, dict(Hq=Hq, Hkv=Hkv, d=d, dff=dff, Ls=Ls, M=M, pos0=pos0))
        ci = make_inputs(shape, device=DEV, with_heads=False, T_cap=T_cap, seed=10 + case)
        model = device_model(ci)
        cyc = SpdCycle(model, 0.0)
        om = OC.model_from_inputs(ci, with_heads=False)
        k, v = synth.kv_cache(shape, model.T_cap, device=DEV, seed=20 + case)
        cyc.k_cache.copy_(k)
        cyc.v_cache.copy_(v)
        g = synth.normal((M, d), 1.0, device=DEV, seed=30 + case, name="big_rows")
        cyc.pdm(pos0, M, g=g)
        torch.cuda.synchronize()
        cache = _oracle_cache_from(k, v, pos0, shape)
        last, _ = O.pdm_step(f64(g), pos0, cache, om.layers, om.final_norm, om.pdm)
        assert rel_err(f64(cyc.h_last), last) < TOL_BF16, case
        _check_cache_rows(cyc, cache, pos0, pos0 + M, TOL_BF16)


def test_cycle_calls_are_deterministic():
    """The same feature call and PDM step twice (same inputs, same cache) give the
    same rows, cache entries and last row bit for bit: every cross-block sum runs
    in a fixed order whichever block arrives last."""
    s = synth.HEADLINE
    ci = make_inputs(s, device=DEV, with_heads=False)
    model = device_model(ci)
    cyc = SpdCycle(model, s.temperature)
    k, v = synth.kv_cache(s, model.T_cap, device=DEV)
    a = s.n
    pos0, M = s.ctx - 1 - a, a + 1
    outs = []
    for _ in range(2):
        cyc.k_cache.copy_(k)
        cyc.v_cache.copy_(v)
        g = cyc.features(pos0, M, a).clone()
        cyc.pdm(pos0, M)
        torch.cuda.synchronize()
        outs.append((g, cyc.h_last.clone(), cyc.k_cache.clone(), cyc.v_cache.clone()))
    for x, y in zip(*outs):
        assert torch.equal(x, y)


def test_pdm_step_prepared_contract():
    """spd_pdm_step_prepared: a decode-sized step (M < 256) does not read the prepared
    weights, and prep == NULL is spd_pdm_step, on a prefill-sized step too -- rows,
    cache entries and last row bit for bit."""
    s = synth.HEADLINE
    ci = make_inputs(s, device=DEV, with_heads=False)
    model = device_model(ci)
    cyc = SpdCycle(model, s.temperature)
    prep = model.pdm_prep()
    assert prep is not None
    k, v = synth.kv_cache(s, model.T_cap, device=DEV)
    m = model
    for pos0, M in ((s.ctx - 1 - s.n, s.n + 1), (0, 300)):
        g = synth.normal((M, s.d), 1.0, device=DEV, seed=40 + M, name="rows")
        outs = []
        for mode in ("plain", "prepared" if M < 256 else "null"):
            cyc.k_cache.copy_(k)
            cyc.v_cache.copy_(v)
            say("prepared contract", M, mode)
            if mode == "plain":
                spd.spd_pdm_step(m.cfg, m.layer_arr, m.w.final_norm, cyc.k_cache, cyc.v_cache, m.T_cap, g,
                                 pos0, M, cyc.h_last, cyc.ws)
            else:
                spd.spd_pdm_step_prepared(m.cfg, m.layer_arr, prep if mode == "prepared" else None,
                                          m.w.final_norm, cyc.k_cache, cyc.v_cache, m.T_cap, g, pos0, M,
                                          cyc.h_last, cyc.ws)
            torch.cuda.synchronize()
            outs.append((cyc.h_last.clone(), cyc.k_cache.clone(), cyc.v_cache.clone()))
        for x, y in zip(*outs):
            assert torch.equal(x, y), (pos0, M)


# ------------------------------------------------------------------ LM head

def _lm_case(V, d, dtype, std, rows, T, seed):
    wdt = synth.storage_dtype(dtype)
    W = synth.normal((V, d), std, device=DEV, seed=seed, name="w_lm", dtype=wdt)
    h = synth.normal((rows, d), 1.0, device=DEV, seed=seed, name="h")
    cfg = spd.make_config(L=1, n=1, m=1, d=d, Ls=1, Hq=1, Hkv=1, hd=16, dff=64, V=V, dtype=dtype)
    words = synth.rand_words(seed, 5, rows)
    wt = synth.words_tensor(words, DEV)
    logits = torch.empty(rows, V, device=DEV)
    probs = torch.empty(rows, V, device=DEV)
    tok = torch.zeros(rows, dtype=torch.int32, device=DEV)
    ws = torch.zeros(spd.spd_workspace_size(spd.SPD_CALL_LM_HEAD, cfg, rows), dtype=torch.uint8,
                     device=DEV)
    spd.spd_lm_head(cfg, W, h, rows, T, wt, logits, probs, tok, ws)
    torch.cuda.synchronize()
    return W, h, words, logits, probs, tok, cfg, ws, wt


LM_CASES = [
    ("tiny_t0", 512, 64, 0, 0.02, 1, 0.0),
    ("tiny_t1", 512, 64, 0, 1.0, 1, 1.0),
    ("tiny_rows", 512, 64, 0, 1.0, 5, 0.7),
    ("full_t1", 151936, 2560, 1, 3.0 / np.sqrt(2560), 1, 1.0),
    ("full_t0", 151936, 2560, 1, 0.02, 1, 0.0),
    ("full_rows3", 151936, 2560, 1, 3.0 / np.sqrt(2560), 3, 1.0),
    ("9b_t1", 151936, 4096, 1, 3.0 / np.sqrt(4096), 1, 1.0),
    ("ragged_v", 151936 - 37, 2560, 1, 3.0 / np.sqrt(2560), 1, 1.0),
    # several hidden rows share one pass over the head (skinny MFMA GEMM path)
    ("full_rows2", 151936, 2560, 1, 3.0 / np.sqrt(2560), 2, 1.0),
    ("full_rows4_t0", 151936, 2560, 1, 0.02, 4, 0.0),
    ("9b_rows3", 151936, 4096, 1, 3.0 / np.sqrt(4096), 3, 0.8),
    ("9b_rows4", 151936, 4096, 1, 3.0 / np.sqrt(4096), 4, 1.0),
    ("ragged_rows4", 151936 - 37, 2560, 1, 3.0 / np.sqrt(2560), 4, 1.0),
    # the most rows one call takes (16: one full MFMA row tile)
    ("tiny_rows16_t0", 512, 64, 0, 0.02, 16, 0.0),
    ("full_rows16_t1", 151936, 2560, 1, 3.0 / np.sqrt(2560), 16, 1.0),
    # near one-hot and near flat distributions
    ("full_t_low", 151936, 2560, 1, 3.0 / np.sqrt(2560), 1, 0.05),
    ("full_t_high", 151936, 2560, 1, 3.0 / np.sqrt(2560), 2, 20.0),
]


@pytest.mark.parametrize("name,V,d,dtype,std,rows,T", LM_CASES, ids=[c[0] for c in LM_CASES])
def test_lm_head(name, V, d, dtype, std, rows, T):
    say("lm_head", name)
    W, h, words, logits, probs, tok, *_ = _lm_case(V, d, dtype, std, rows, T, seed=11)
    Wh, hh = f64(W), f64(h)
    gl = f64(logits)
    toks = tok.cpu().numpy()
    for r in range(rows):
        ref = O.lm_logits(Wh, hh[r])
        assert rel_err(gl[r], ref) < tol_for(dtype), r
        if T == 0:
            assert toks[r] == O.argmax_first(logits[r].cpu().numpy())
        else:
            gp = probs[r].cpu().numpy()
            pref = O.softmax(logits[r].cpu().numpy().astype(np.float64), T)
            assert np.max(np.abs(gp - pref)) <= 1e-5 * pref.max()
            assert toks[r] == O.sample_probs(gp, int(words[r]) >> 32)


def test_lm_head_is_deterministic():
    say("lm_head determinism")
    W, h, words, logits, probs, tok, cfg, ws, wt = _lm_case(151936, 2560, 1, 3.0 / np.sqrt(2560),
                                                            1, 1.0, 12)
    l2 = torch.empty_like(logits)
    p2 = torch.empty_like(probs)
    t2 = torch.zeros_like(tok)
    spd.spd_lm_head(cfg, W, h, 1, 1.0, wt, l2, p2, t2, ws)
    torch.cuda.synchronize()
    assert torch.equal(l2, logits) and torch.equal(p2, probs) and torch.equal(t2, tok)


@pytest.mark.parametrize("workgroups", [1, 7, 256, 5000])
def test_lm_head_workgroup_cap_is_bitwise_neutral(workgroups):
    """A capped vocabulary GEMV (each workgroup loops over row groups) gives the
    same logits, probabilities and token, bit for bit."""
    say("lm_head workgroups", workgroups)
    W, h, words, logits, probs, tok, cfg, ws, wt = _lm_case(151936, 2560, 1, 3.0 / np.sqrt(2560),
                                                            1, 1.0, 13)
    cfg.head_workgroups = workgroups
    l2 = torch.empty_like(logits)
    p2 = torch.empty_like(probs)
    t2 = torch.zeros_like(tok)
    spd.spd_lm_head(cfg, W, h, 1, 1.0, wt, l2, p2, t2, ws)
    torch.cuda.synchronize()
    assert torch.equal(l2, logits) and torch.equal(p2, probs) and torch.equal(t2, tok)


@pytest.mark.parametrize("V,T", [(3000, 1.0), (3000, 0.0), (300000, 1.0), (530000, 0.0)])
def test_lm_head_vocabulary_sizes(V, T):
    """The one-row GEMV finishes the head in its own launch: a ragged second chunk,
    more chunks than the finish uses workers (300000 entries: 147 chunks), and a
    greedy vocabulary past the finish's chunk counters (530000: a separate argmax
    launch).  Logits are checked on sampled rows, the probabilities and the token
    on the whole row."""
    say("lm_head vocabulary", V, T)
    d = 512
    W, h, words, logits, probs, tok, *_ = _lm_case(V, d, 1, 3.0 / np.sqrt(d), 1, T, seed=14)
    rng = np.random.default_rng(14)
    rows = np.unique(np.concatenate([rng.integers(0, V, 2048), [0, V - 1, 2047, 2048]]))
    ref = O.lm_logits(f64(W[torch.as_tensor(rows, device=DEV)]), f64(h)[0])
    lg = logits[0].cpu().numpy()
    assert rel_err(lg[rows].astype(np.float64), ref) < tol_for(1)
    if T == 0:
        assert int(tok.item()) == O.argmax_first(lg)
    else:
        gp = probs[0].cpu().numpy()
        pref = O.softmax(lg.astype(np.float64), T)
        assert np.max(np.abs(gp - pref)) <= 1e-5 * pref.max()
        assert int(tok.item()) == O.sample_probs(gp, int(words[0]) >> 32)


# ------------------------------------------------------------------ top-k / top-p sampling

def _run_lm(W, h, V, d, dtype, rows, T, seed, top_k, top_p):
    cfg = spd.make_config(L=1, n=1, m=1, d=d, Ls=1, Hq=1, Hkv=1, hd=16, dff=64, V=V, dtype=dtype,
                          top_k=top_k, top_p=top_p)
    words = synth.rand_words(seed, 5, rows)
    wt = synth.words_tensor(words, DEV)
    logits = torch.empty(rows, V, device=DEV)
    probs = torch.full((rows, V), -1.0, device=DEV)     # every entry must be written
    tok = torch.full((rows,), -7, dtype=torch.int32, device=DEV)
    ws = torch.zeros(spd.spd_workspace_size(spd.SPD_CALL_LM_HEAD, cfg, rows), dtype=torch.uint8,
                     device=DEV)
    spd.spd_lm_head(cfg, W, h, rows, T, wt, logits, probs, tok, ws)
    torch.cuda.synchronize()
    return words, logits, probs, tok


def _check_filtered(words, logits, probs, tok, T, top_k, top_p):
    """The kept set is exact (the oracle's filters applied to the device's fp32
    logits), the probabilities are within fp32 rounding of the oracle's, and the
    token is the oracle's draw from the device's probability row."""
    toks = tok.cpu().numpy()
    for r in range(logits.shape[0]):
        lg = logits[r].cpu().numpy().astype(np.float64)
        gp = probs[r].cpu().numpy()
        ref = O.filtered_softmax(lg, T, top_k, top_p)
        assert np.array_equal(np.flatnonzero(gp), np.flatnonzero(ref)), r
        assert np.max(np.abs(gp - ref)) <= 2e-6 * ref.max(), r
        assert abs(float(gp.astype(np.float64).sum()) - 1.0) < 1e-5
        assert toks[r] == O.sample_probs(gp, int(words[r]) >> 32), r


TOPK_CASES = [
    # name, V, d, dtype, std, rows, T, top_k, top_p
    ("full_k50", 151936, 2560, 1, 3.0 / np.sqrt(2560), 1, 1.0, 50, 1.0),
    ("full_k50_p09", 151936, 2560, 1, 3.0 / np.sqrt(2560), 1, 1.0, 50, 0.9),
    ("full_k256", 151936, 2560, 1, 3.0 / np.sqrt(2560), 1, 1.0, 256, 1.0),
    ("full_k256_p05", 151936, 2560, 1, 3.0 / np.sqrt(2560), 1, 0.7, 256, 0.5),
    ("full_k1", 151936, 2560, 1, 3.0 / np.sqrt(2560), 1, 1.0, 1, 1.0),
    ("ragged_k50", 151936 - 37, 2560, 1, 3.0 / np.sqrt(2560), 1, 1.0, 50, 1.0),
    ("rows3_k50", 151936, 2560, 1, 3.0 / np.sqrt(2560), 3, 1.0, 50, 0.95),
    ("9b_k50", 151936, 4096, 1, 3.0 / np.sqrt(4096), 1, 1.0, 50, 1.0),
    ("small_three_chunks", 5000, 64, 0, 1.0, 2, 0.7, 100, 0.8),
    ("k_above_v", 200, 64, 0, 1.0, 1, 1.0, 256, 1.0),
    ("k_equals_v", 256, 64, 0, 1.0, 1, 1.0, 256, 0.3),
    ("k_in_last_chunk_only", 2049, 64, 0, 1.0, 1, 1.0, 2, 1.0),
]


@pytest.mark.parametrize("name,V,d,dtype,std,rows,T,top_k,top_p", TOPK_CASES,
                         ids=[c[0] for c in TOPK_CASES])
def test_lm_head_top_k_top_p(name, V, d, dtype, std, rows, T, top_k, top_p):
    say("lm_head filters", name)
    wdt = synth.storage_dtype(dtype)
    W = synth.normal((V, d), std, device=DEV, seed=31, name="w_lm", dtype=wdt)
    h = synth.normal((rows, d), 1.0, device=DEV, seed=31, name="h")
    words, logits, probs, tok = _run_lm(W, h, V, d, dtype, rows, T, 31, top_k, top_p)
    Wh, hh = f64(W), f64(h)
    for r in range(rows):
        assert rel_err(f64(logits[r]), O.lm_logits(Wh, hh[r])) < tol_for(dtype), r
    _check_filtered(words, logits, probs, tok, T, top_k, top_p)


@pytest.mark.parametrize("V,top_k", [(5000, 50), (151936, 50), (151936, 256)])
def test_lm_head_top_k_ties_break_by_index(V, top_k):
    """Integer-valued logits (small integer weights, 0/1 hidden rows: every sum is
    exact in any order) with thousands of equal values: the kept set takes the
    lowest indices among the equal logits at the cut; the result is repeatable."""
    say("lm_head ties", V, top_k)
    d = 64
    gen = torch.Generator().manual_seed(41)
    W = torch.randint(-2, 3, (V, d), generator=gen).float().to(DEV)
    h = torch.randint(0, 2, (1, d), generator=gen).float().to(DEV)
    words, logits, probs, tok = _run_lm(W, h, V, d, 0, 1, 1.0, 41, top_k, 1.0)
    lg = logits[0].cpu().numpy().astype(np.float64)
    assert np.array_equal(lg, np.round(lg))
    cut = np.sort(lg)[::-1][top_k - 1]
    assert np.count_nonzero(lg == cut) > 1            # the cut falls inside a run of ties
    _check_filtered(words, logits, probs, tok, 1.0, top_k, 1.0)
    _, l2, p2, t2 = _run_lm(W, h, V, d, 0, 1, 1.0, 41, top_k, 1.0)
    assert torch.equal(p2, probs) and torch.equal(t2, tok)


def test_lm_head_drawn_shapes():
    """60 drawn head calls: vocabulary sizes that are ragged against the GEMV's row
    groups and the 2048-entry sampling chunks, several widths, row counts,
    temperatures and filters; logits within tolerance, every decision exact."""
    rng = np.random.default_rng(91)
    say("lm_head drawn shapes")
    for case in range(60):
        V = int(rng.integers(1, 9000))
        d = int(rng.choice([64, 128, 192]))
        dtype = int(rng.integers(0, 2))
        rows = int(rng.integers(1, 7))
        T = float(rng.choice([0.0, 0.3, 1.0, 3.0]))
        top_k = int(rng.integers(1, 257)) if (T > 0 and rng.random() < 0.5) else (1 if rng.random() < 0.2 else 0)
        top_p = float(rng.uniform(0.3, 0.99)) if (top_k > 0 and T > 0 and rng.random() < 0.5) else 1.0
        W = synth.normal((V, d), 2.0 / np.sqrt(d), device=DEV, seed=100 + case, name="w_lm",
                         dtype=synth.storage_dtype(dtype))
        h = synth.normal((rows, d), 1.0, device=DEV, seed=100 + case, name="h")
        words, logits, probs, tok = _run_lm(W, h, V, d, dtype, rows, T, 100 + case, top_k, top_p)
        Wh, hh = f64(W), f64(h)
        for r in range(rows):
            assert rel_err(f64(logits[r]), O.lm_logits(Wh, hh[r])) < tol_for(dtype), (case, r)
        if T == 0:
            toks = tok.cpu().numpy()
            for r in range(rows):
                assert toks[r] == O.argmax_first(logits[r].cpu().numpy()), (case, r)
        elif top_k > 0:
            _check_filtered(words, logits, probs, tok, T, top_k, top_p)
        else:
            toks = tok.cpu().numpy()
            for r in range(rows):
                gp = probs[r].cpu().numpy()
                pref = O.softmax(logits[r].cpu().numpy().astype(np.float64), T)
                assert np.max(np.abs(gp - pref)) <= 1e-5 * pref.max(), (case, r)
                assert toks[r] == O.sample_probs(gp, int(words[r]) >> 32), (case, r)


# ------------------------------------------------------------------ draft trees

def _width_tree(W, a):
    """Parents of a width-W tree with a levels below the root: level 1 holds W
    children of the root, every deeper level W nodes whose parents are the first
    nodes of the level above (two children each), as a top-W expansion keeps the
    likeliest paths."""
    parents, prev = [-1], [0]
    for lvl in range(a):
        cur = []
        for i in range(W):
            parents.append(0 if lvl == 0 else prev[min(i // 2, len(prev) - 1)])
            cur.append(len(parents) - 1)
        prev = cur
    return parents


def _masks(parents):
    anc = []
    for i, p in enumerate(parents):
        anc.append((1 << i) | (anc[p] if p >= 0 else 0))
    return anc


def _anc_tensor(anc):
    return torch.from_numpy(np.array(anc, dtype=np.uint64).view(np.int64)).to(DEV)


TREE_CASES = [
    # name, shape, W, a, pos0 (None: the cycle's, ctx - 1 - n)
    ("small_w4_a3", SMALL_BF16, 4, 3, None),
    ("small_w4_a3_short_prefix", SMALL_BF16, 4, 3, 3),
    ("small_w2_a8", SMALL_BF16, 2, 8, None),
    ("tiny_w3_a3", synth.TINY, 3, 3, None),
    ("tiny_w4_a4_no_prefix", synth.TINY, 4, 4, 0),
    ("headline_w4_a7", synth.HEADLINE, 4, 7, None),
    ("headline_w4_a8_two_row_tiles", synth.HEADLINE, 4, 8, None),
    ("small_w9_a7_max_nodes", SMALL_BF16, 9, 7, None),          # 64 nodes: the mask limit
]


@pytest.mark.parametrize("name,shape,W,a,pos0", TREE_CASES, ids=[c[0] for c in TREE_CASES])
def test_tree_features_and_pdm_step(name, shape, W, a, pos0):
    """Features of every tree node (depth n at the root, a - level below) and the
    tree-masked PDM step on a seeded committed cache: the deepest level's final
    rows and every node's cache slot against the oracle.  The short-prefix cases
    make the tree's own keys dominate attention, so a wrong mask or position
    cannot hide inside the tolerance."""
    ci = make_inputs(shape, device=DEV, with_heads=False)
    model = device_model(ci)
    cyc = SpdCycle(model, shape.temperature)
    om = OC.model_from_inputs(ci, with_heads=False)
    anc = _width_tree(W, a)
    anc = _masks(anc)
    M = len(anc)
    if pos0 is None:
        pos0 = shape.ctx - 1 - shape.n
    assert pos0 + M <= model.T_cap
    say(name, "tree", M, pos0)
    dev_anc = _anc_tensor(anc)
    ws = torch.zeros(max(spd.spd_workspace_size(spd.SPD_CALL_FUSE, model.cfg, M),
                         spd.spd_workspace_size(spd.SPD_CALL_PDM, model.cfg, M, 0, model.T_cap)),
                     dtype=torch.uint8, device=DEV)
    g = torch.empty(M, shape.d, device=DEV)
    spd.spd_fuse_features_tree(model.cfg, model.w.store, model.T_cap, len(model.store_layers),
                               model.slot_tab, pos0, M, a, dev_anc, model.w.fc_norm, model.w.w_fc, g,
                               ws)
    torch.cuda.synchronize()
    rows, depth, _ = O.tree_rows(anc, a, shape.n, pos0)
    ref = O.fuse_features(om.store, om.store_layers, rows, depth, om.fc_norm, om.w_fc, L=shape.L,
                          n=shape.n, anchors=shape.anchors, mode=shape.anchor_mode, eps=shape.eps,
                          norm_k0=bool(shape.norm_k0), schedule=shape.feature_schedule)
    assert rel_err(f64(g), ref) < tol_for(shape.dtype)

    k, v = synth.kv_cache(shape, model.T_cap, device=DEV)
    cyc.k_cache.copy_(k)
    cyc.v_cache.copy_(v)
    gin = synth.normal((M, shape.d), 1.0, device=DEV, seed=77, name="tree_rows")
    n_out = W
    h_out = torch.empty(n_out, shape.d, device=DEV)
    spd.spd_pdm_step_tree(model.cfg, model.layer_arr, model.w.final_norm, cyc.k_cache, cyc.v_cache,
                          model.T_cap, gin, pos0, M, dev_anc, n_out, h_out, ws)
    torch.cuda.synchronize()
    cache = _oracle_cache_from(k, v, pos0, shape)
    ref_rows, _ = O.pdm_step_tree(f64(gin), pos0, cache, om.layers, om.final_norm, om.pdm, anc)
    tol = tol_for(shape.dtype)
    for o in range(n_out):
        assert rel_err(f64(h_out[o]), ref_rows[M - n_out + o]) < tol, o
    _check_cache_rows(cyc, cache, pos0, pos0 + M, tol)


def _random_tree(rng, M, a):
    """Parents of a random tree of M nodes (topological order, root 0) whose levels
    stay within a."""
    parents, level = [-1], [0]
    for i in range(1, M):
        cand = [j for j in range(i) if level[j] < a]
        p = int(rng.choice(cand))
        parents.append(p)
        level.append(level[p] + 1)
    return parents


def test_tree_drawn_shapes():
    """12 random trees (arbitrary branching, 2..64 nodes, levels up to a, committed
    prefixes from empty upward) on three small workloads: features of every node,
    the last n_out final rows and every node's cache slot against the oracle."""
    rng = np.random.default_rng(555)
    shapes = [synth.TINY, SMALL_BF16, SMALL_BF16_H64]
    for case in range(12):
        shape = shapes[case % 3]
        ci = make_inputs(shape, device=DEV, with_heads=False, T_cap=shape.ctx + 64, seed=case)
        model = device_model(ci)
        cyc = SpdCycle(model, shape.temperature)
        om = OC.model_from_inputs(ci, with_heads=False)
        a = int(rng.integers(1, shape.n + 1))
        M = int(rng.integers(2, min(64, model.T_cap) + 1))
        anc = _masks(_random_tree(rng, M, a))
        pos0 = int(rng.integers(0, model.T_cap - M + 1))
        n_out = int(rng.integers(1, min(M, 8) + 1))
        say("tree drawn", case, shape.name, dict(M=M, a=a, pos0=pos0, n_out=n_out))
        dev_anc = _anc_tensor(anc)
        ws = torch.zeros(max(spd.spd_workspace_size(spd.SPD_CALL_FUSE, model.cfg, M),
                             spd.spd_workspace_size(spd.SPD_CALL_PDM, model.cfg, M, 0, model.T_cap)),
                         dtype=torch.uint8, device=DEV)
        g = torch.empty(M, shape.d, device=DEV)
        spd.spd_fuse_features_tree(model.cfg, model.w.store, model.T_cap, len(model.store_layers),
                                   model.slot_tab, pos0, M, a, dev_anc, model.w.fc_norm, model.w.w_fc, g,
                                   ws)
        torch.cuda.synchronize()
        rows, depth, _ = O.tree_rows(anc, a, shape.n, pos0)
        ref = O.fuse_features(om.store, om.store_layers, rows, depth, om.fc_norm, om.w_fc, L=shape.L,
                              n=shape.n, anchors=shape.anchors, mode=shape.anchor_mode, eps=shape.eps,
                              norm_k0=bool(shape.norm_k0), schedule=shape.feature_schedule)
        tol = tol_for(shape.dtype)
        assert rel_err(f64(g), ref) < tol, case
        k, v = synth.kv_cache(shape, model.T_cap, device=DEV, seed=80 + case)
        cyc.k_cache.copy_(k)
        cyc.v_cache.copy_(v)
        gin = synth.normal((M, shape.d), 1.0, device=DEV, seed=90 + case, name="tree_rows")
        h_out = torch.empty(n_out, shape.d, device=DEV)
        spd.spd_pdm_step_tree(model.cfg, model.layer_arr, model.w.final_norm, cyc.k_cache, cyc.v_cache,
                              model.T_cap, gin, pos0, M, dev_anc, n_out, h_out, ws)
        torch.cuda.synchronize()
        cache = _oracle_cache_from(k, v, pos0, shape)
        ref_rows, _ = O.pdm_step_tree(f64(gin), pos0, cache, om.layers, om.final_norm, om.pdm, anc)
        for o in range(n_out):
            assert rel_err(f64(h_out[o]), ref_rows[M - n_out + o]) < tol, (case, o)
        _check_cache_rows(cyc, cache, pos0, pos0 + M, tol)


def test_tree_pdm_chain_matches_causal_step():
    """A chain given as tree masks is the ordinary step, bit for bit."""
    shape = SMALL_BF16
    ci = make_inputs(shape, device=DEV, with_heads=False)
    model = device_model(ci)
    cyc = SpdCycle(model, shape.temperature)
    k, v = synth.kv_cache(shape, model.T_cap, device=DEV)
    M, pos0 = 9, shape.ctx - 9
    g = synth.normal((M, shape.d), 1.0, device=DEV, seed=78, name="chain_rows")
    anc = _anc_tensor(_masks([-1] + list(range(M - 1))))
    ws = torch.zeros(spd.spd_workspace_size(spd.SPD_CALL_PDM, model.cfg, M, 0, model.T_cap),
                     dtype=torch.uint8, device=DEV)
    outs = []
    for tree in (False, True):
        cyc.k_cache.copy_(k)
        cyc.v_cache.copy_(v)
        h = torch.empty(1, shape.d, device=DEV)
        if tree:
            spd.spd_pdm_step_tree(model.cfg, model.layer_arr, model.w.final_norm, cyc.k_cache,
                                  cyc.v_cache, model.T_cap, g, pos0, M, anc, 1, h, ws)
        else:
            spd.spd_pdm_step(model.cfg, model.layer_arr, model.w.final_norm, cyc.k_cache,
                             cyc.v_cache, model.T_cap, g, pos0, M, h, ws)
        torch.cuda.synchronize()
        outs.append((h.clone(), cyc.k_cache.clone(), cyc.v_cache.clone()))
    for x, y in zip(*outs):
        assert torch.equal(x, y)


@pytest.mark.parametrize("rows,V,d,dtype,W", [(1, 151936, 2560, 1, 4), (4, 151936, 2560, 1, 4),
                                              (1, 5000, 64, 0, 8), (2, 300, 64, 0, 256)])
def test_lm_head_top_w_children(rows, V, d, dtype, W):
    """T = 0 with top_k = W: the ordered W largest logits of each row (the
    children of a greedy tree node), -1 past the vocabulary."""
    say("lm_head top-W", rows, V, W)
    wdt = synth.storage_dtype(dtype)
    Wt = synth.normal((V, d), 0.02 if dtype else 1.0, device=DEV, seed=51, name="w_lm", dtype=wdt)
    h = synth.normal((rows, d), 1.0, device=DEV, seed=51, name="h")
    cfg = spd.make_config(L=1, n=1, m=1, d=d, Ls=1, Hq=1, Hkv=1, hd=16, dff=64, V=V, dtype=dtype,
                          top_k=W)
    logits = torch.empty(rows, V, device=DEV)
    tok = torch.full((rows, W), -7, dtype=torch.int32, device=DEV)
    ws = torch.zeros(spd.spd_workspace_size(spd.SPD_CALL_LM_HEAD, cfg, rows), dtype=torch.uint8,
                     device=DEV)
    spd.spd_lm_head(cfg, Wt, h, rows, 0.0, None, logits, None, tok, ws)
    torch.cuda.synchronize()
    got = tok.cpu().numpy()
    for r in range(rows):
        want = O.top_k_list(logits[r].cpu().numpy().astype(np.float64), min(W, V))
        want += [-1] * (W - len(want))
        assert got[r].tolist() == want, r


def test_verify_siblings_greedy():
    B, W, V = 40, 4, 151936
    say("verify siblings", B, W)
    logits = synth.normal((B, V), 3.0, device=DEV, seed=61, name="sib_logits")
    best = logits.argmax(-1).to(torch.int32).cpu().numpy()
    gen = np.random.default_rng(61)
    cand = gen.integers(0, V, size=(B, W)).astype(np.int32)
    for b in range(B):
        j = b % (W + 1)                 # W: no sibling matches
        cand[b][cand[b] == best[b]] = (best[b] + 1) % V
        if j < W:
            cand[b][j] = best[b]
    cand_d = torch.from_numpy(cand).to(DEV)
    cfg = spd.make_config(L=1, n=1, m=1, d=64, Ls=1, Hq=1, Hkv=1, hd=16, dff=64, V=V, dtype=0)
    ws = torch.zeros(spd.spd_workspace_size(spd.SPD_CALL_VERIFY, cfg, B, 0), dtype=torch.uint8,
                     device=DEV)
    acc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nxt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    spd.spd_verify_siblings(B, W, V, 0.0, logits, None, cand_d, None, acc, nxt, ws)
    torch.cuda.synchronize()
    lc = logits.cpu().numpy()
    for b in range(B):
        ref = O.verify_siblings(lc[b], cand[b])
        assert (int(acc[b]), int(nxt[b])) == ref, b
        assert ref[0] == (b % (W + 1) if b % (W + 1) < W else -1)


@pytest.mark.parametrize("B,W,V,top_k", [(6, 4, 151936, 0), (4, 4, 151936, 50), (48, 3, 5000, 0),
                                         (24, 8, 700, 20), (80, 3, 2100, 0), (1, 1, 151936, 0)])
def test_verify_siblings_sampled(B, W, V, top_k):
    """T = 1: W independent draws from q per sequence, multi-round rejection; the
    accepted index or the replacement token equal the oracle's on the device's rows
    and words, bit for bit.  Half the sequences get R words that force the early
    rounds to reject, so the residual rounds and the final draw are exercised."""
    say("verify siblings sampled", B, W, V, top_k)
    lp = synth.normal((B, V), 3.0, device=DEV, seed=62, name="sib_p")
    lq = lp + synth.normal((B, V), 1.0, device=DEV, seed=63, name="sib_q")
    if top_k:
        def filt(x):
            th = torch.topk(x, top_k, dim=-1).values[:, -1:]
            return torch.where(x >= th, x, torch.full_like(x, -float("inf")))
        lp, lq = filt(lp), filt(lq)
    p = torch.softmax(lp, -1).contiguous()
    q = torch.softmax(lq, -1).contiguous()
    gen = torch.Generator(device=DEV)
    gen.manual_seed(64)
    cand = torch.multinomial(q, W, replacement=True, generator=gen).to(torch.int32).contiguous()
    words = synth.rand_words(65, 5, B * (W + 1) * 2).reshape(B, W + 1, 2)
    for b in range(0, B, 2):
        for i in range(min(W - 1, 2)):
            words[b, i, 0] = np.uint64(((1 << 24) - 1) << 40)
    cfg = spd.make_config(L=1, n=1, m=1, d=64, Ls=1, Hq=1, Hkv=1, hd=16, dff=64, V=V, dtype=0)
    ws = torch.zeros(spd.spd_workspace_size(spd.SPD_CALL_VERIFY, cfg, B, 0), dtype=torch.uint8,
                     device=DEV)
    acc = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nxt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    spd.spd_verify_siblings(B, W, V, 1.0, p, q, cand, synth.words_tensor(words, DEV), acc, nxt, ws)
    torch.cuda.synchronize()
    pc, qc, cc = p.cpu().numpy(), q.cpu().numpy(), cand.cpu().numpy()
    hist = {"accepted": 0, "replaced": 0}
    for b in range(B):
        ref = O.verify_siblings_sampled(pc[b], qc[b], cc[b], words[b])
        assert (int(acc[b]), int(nxt[b])) == ref, b
        hist["accepted" if ref[0] >= 0 else "replaced"] += 1
    assert hist["replaced"] > 0 or B < 8


def test_verify_siblings_sampled_drawn_rows():
    """80 drawn sequences of small vocabularies (smooth, sparse, tied and
    wide-range rows from _drawn_row), W = 1..8 candidates, some outside q's
    support, random and forced-reject words: bit-exact against the oracle."""
    rng = np.random.default_rng(606)
    say("verify siblings drawn rows")
    for case in range(80):
        V = int(rng.integers(1, 3000))
        W = int(rng.integers(1, 9))
        p, q = _drawn_row(rng, V), _drawn_row(rng, V)
        cand = rng.integers(0, V, size=W).astype(np.int32)
        words = rng.integers(0, 2 ** 64, size=(1, W + 1, 2), dtype=np.uint64)
        if rng.random() < 0.5:
            words[0, :, 0] = np.uint64(((1 << 24) - 1) << 40)   # every round's test at its hardest
        cfg = spd.make_config(L=1, n=1, m=1, d=64, Ls=1, Hq=1, Hkv=1, hd=16, dff=64, V=V, dtype=0)
        ws = torch.zeros(spd.spd_workspace_size(spd.SPD_CALL_VERIFY, cfg, 1, 0), dtype=torch.uint8,
                         device=DEV)
        acc = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        nxt = torch.full((1,), -7, dtype=torch.int32, device=DEV)
        spd.spd_verify_siblings(1, W, V, 1.0, torch.tensor(p, device=DEV).reshape(1, V),
                                torch.tensor(q, device=DEV).reshape(1, V),
                                torch.tensor(cand, device=DEV).reshape(1, W),
                                synth.words_tensor(words, DEV), acc, nxt, ws)
        torch.cuda.synchronize()
        ref = O.verify_siblings_sampled(p, q, cand, words[0])
        assert (int(acc[0]), int(nxt[0])) == ref, (case, V, W)


# ------------------------------------------------------------------ verify

def _verify_gpu(p, q, draft, words, T, bonus):
    B, G = draft.shape
    V = p.shape[-1]
    cfg = spd.make_config(L=1, n=1, m=1, d=64, Ls=1, Hq=1, Hkv=1, hd=16, dff=64, V=V, dtype=0)
    ws = torch.zeros(spd.spd_workspace_size(spd.SPD_CALL_VERIFY, cfg, B, G), dtype=torch.uint8,
                     device=DEV)
    na = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    nt = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    spd.spd_verify(B, G, V, T, bonus, p, q, draft, synth.words_tensor(words, DEV), na, nt, ws)
    torch.cuda.synchronize()
    return na.cpu().numpy(), nt.cpu().numpy()


def test_verify_batched_stress_bitexact():
    v = synth.VERIFY_STRESS
    say("verify stress", v.B, v.gamma, v.V)
    p, q, draft, words = synth.verify_stress_inputs(v, device=DEV)
    na, nt = _verify_gpu(p, q, draft, words, v.temperature, v.bonus)
    pc, qc, dc = p.cpu().numpy(), q.cpu().numpy(), draft.cpu().numpy()
    hist = np.zeros(v.gamma + 1, int)
    for b in range(v.B):
        ref = O.verify(pc[b], qc[b], list(dc[b]), words[b], temperature=v.temperature,
                       bonus=bool(v.bonus))
        assert (int(na[b]), int(nt[b])) == ref, b
        hist[ref[0]] += 1
    assert hist[0] < v.B      # the correlated drafts are accepted at times


def test_verify_sampled_large_batch():
    """16400 sampled sequences (gamma = 2, bonus) in one call: every checked
    sequence's outcome is the oracle's."""
    B, G, V = 16400, 2, 256
    say("verify two-launch", B, G, V)
    pl = synth.normal((B, G + 1, V), 2.0, device=DEV, seed=41, name="big_p")
    p = torch.softmax(pl, -1)
    q = torch.softmax(pl[:, :G] + synth.normal((B, G, V), 1.0, device=DEV, seed=42, name="big_q"), -1)
    draft = torch.multinomial(q.reshape(-1, V), 1, generator=torch.Generator(device=DEV).manual_seed(43))
    draft = draft.reshape(B, G).to(torch.int32).contiguous()
    words = synth.rand_words(44, 3, B * (G + 1) * 2).reshape(B, G + 1, 2)
    na, nt = _verify_gpu(p, q.contiguous(), draft, words, 1.0, 1)
    pc, qc, dc = p.cpu().numpy(), q.cpu().numpy(), draft.cpu().numpy()
    for b in range(0, B, 7):
        ref = O.verify(pc[b], qc[b], list(dc[b]), words[b], temperature=1.0, bonus=True)
        assert (int(na[b]), int(nt[b])) == ref, b
    for b in range(B - 40, B):
        ref = O.verify(pc[b], qc[b], list(dc[b]), words[b], temperature=1.0, bonus=True)
        assert (int(na[b]), int(nt[b])) == ref, b


def test_verify_greedy_gamma_form():
    say("verify greedy")
    B, G, V = 16, 7, 151936
    logits = synth.normal((B, G + 1, V), 3.0, device=DEV, seed=21, name="vg_logits")
    am = logits.argmax(-1).to(torch.int32)
    draft = am[:, :G].clone()
    # sequence b keeps its first b % (G+1) drafts right, then goes wrong
    for b in range(B):
        j = b % (G + 1)
        if j < G:
            draft[b, j] = (draft[b, j] + 1) % V
    words = np.zeros((B, G + 1, 2), np.uint64)
    na, nt = _verify_gpu(logits, None, draft.contiguous(), words, 0.0, 1)
    lc, dc = logits.cpu().numpy(), draft.cpu().numpy()
    for b in range(B):
        ref = O.verify(lc[b], None, list(dc[b]), words[b], temperature=0, bonus=True)
        assert (int(na[b]), int(nt[b])) == ref
        assert ref[0] == b % (G + 1)


def test_verify_streaming_edge_cases():
    """B = 1, gamma = 1 as in the SPD cycle: forced accept (p(x) >= q(x)), forced
    reject (p(x) = 0), empty residual (fallback to p), a ragged vocabulary."""
    V = 151936 - 5
    say("verify streaming edge", V)
    base = torch.softmax(synth.normal((V,), 3.0, device=DEV, seed=30, name="e_p"), 0)
    qrow = torch.softmax(synth.normal((V,), 3.0, device=DEV, seed=31, name="e_q"), 0)
    cases = []
    x = int(torch.argmax(base).item())
    cases.append((base, qrow, x))                                   # p(x) large: accept likely
    p0 = base.clone(); p0[17] = 0.0
    cases.append((p0, qrow, 17))                                    # p(x) = 0: reject
    cases.append((base * 0.5, base.clone(), x))                     # residual empty at reject
    rng = np.random.default_rng(5)
    for (p, q, xx) in cases:
        for _ in range(3):
            words = rng.integers(0, 2 ** 64, size=(1, 2, 2), dtype=np.uint64)
            d = torch.tensor([[xx]], dtype=torch.int32, device=DEV)
            na, nt = _verify_gpu(p.reshape(1, 1, V).contiguous(), q.reshape(1, 1, V).contiguous(),
                                 d, words, 1.0, 0)
            ref = O.verify([p.cpu().numpy()], [q.cpu().numpy()], [xx], words[0], temperature=1.0,
                           bonus=False)
            assert (int(na[0]), int(nt[0])) == ref


def _drawn_row(rng, V):
    """A float32 probability row of one of several shapes: smooth, sparse (exact
    zeros), tied (few distinct values), or spanning tiny values."""
    kind = int(rng.integers(0, 4))
    if kind == 0:
        x = rng.normal(0, 3, V)
    elif kind == 1:
        x = np.where(rng.random(V) < 0.8, -np.inf, rng.normal(0, 2, V))
        x[int(rng.integers(0, V))] = 0.0
    elif kind == 2:
        x = rng.integers(0, 3, V).astype(np.float64)
    else:
        x = rng.normal(0, 30, V)
    e = np.exp(x - x.max())
    return (e / e.sum()).astype(np.float32)


def test_verify_streaming_drawn_rows_bitexact():
    """Streaming verify (B = 1, gamma = 1) on 200 drawn small-vocabulary cases: the
    device's (accepted, next token) equals the oracle's decision on the same fp32 rows
    and words, bit for bit; the draft token is sometimes one q gives zero mass."""
    rng = np.random.default_rng(77)
    say("verify drawn rows")
    for case in range(200):
        V = int(rng.integers(1, 3000))
        p, q = _drawn_row(rng, V), _drawn_row(rng, V)
        x = int(rng.integers(0, V))
        words = rng.integers(0, 2 ** 64, size=(1, 2, 2), dtype=np.uint64)
        na, nt = _verify_gpu(torch.tensor(p, device=DEV).reshape(1, 1, V),
                             torch.tensor(q, device=DEV).reshape(1, 1, V),
                             torch.tensor([[x]], dtype=torch.int32, device=DEV), words, 1.0, 0)
        ref = O.verify([p], [q], [x], words[0], temperature=1.0, bonus=False)
        assert (int(na[0]), int(nt[0])) == ref, (case, V, x)


def test_verify_greedy_drawn_rows_bitexact():
    """Greedy verify (T = 0) on 100 drawn logit rows with many ties: accepted iff the
    draft is the lowest-index argmax, the correction that argmax."""
    rng = np.random.default_rng(78)
    say("verify greedy drawn rows")
    for case in range(100):
        V = int(rng.integers(1, 5000))
        logits = rng.integers(-3, 3, V).astype(np.float32)
        am = O.argmax_first(logits)
        x = am if rng.random() < 0.5 else int(rng.integers(0, V))
        words = rng.integers(0, 2 ** 64, size=(1, 2, 2), dtype=np.uint64)
        na, nt = _verify_gpu(torch.tensor(logits, device=DEV).reshape(1, 1, V), None,
                             torch.tensor([[x]], dtype=torch.int32, device=DEV), words, 0.0, 0)
        ref = O.verify([logits], None, [x], words[0], temperature=0.0, bonus=False)
        assert (int(na[0]), int(nt[0])) == ref, (case, V, x)


def test_verify_gamma_form_drawn_bitexact():
    """40 drawn batched verifications (B = 1..12 sequences of gamma = 1..8 drafts,
    with and without the bonus row, T = 1 on drawn probability rows and T = 0 on
    tied integer logits): every (accepted count, next token) equals the oracle's."""
    rng = np.random.default_rng(707)
    say("verify gamma drawn")
    for case in range(40):
        B, G, V = int(rng.integers(1, 13)), int(rng.integers(1, 9)), int(rng.integers(1, 2000))
        bonus = int(rng.integers(0, 2))
        T = float(rng.choice([0.0, 1.0]))
        if T > 0:
            p = np.stack([np.stack([_drawn_row(rng, V) for _ in range(G + bonus)]) for _ in range(B)])
            q = np.stack([np.stack([_drawn_row(rng, V) for _ in range(G)]) for _ in range(B)])
            qd = torch.tensor(q, device=DEV)
        else:
            p = rng.integers(-2, 3, size=(B, G + bonus, V)).astype(np.float32)
            q, qd = None, None
        draft = rng.integers(0, V, size=(B, G)).astype(np.int32)
        if T == 0:
            for b in range(B):                      # long accepted runs as well
                k = int(rng.integers(0, G + 1))
                for j in range(k):
                    draft[b, j] = O.argmax_first(p[b, j])
        words = rng.integers(0, 2 ** 64, size=(B, G + 1, 2), dtype=np.uint64)
        na, nt = _verify_gpu(torch.tensor(p, device=DEV), qd, torch.tensor(draft, device=DEV), words, T,
                             bonus)
        for b in range(B):
            ref = O.verify(p[b], None if q is None else q[b], draft[b], words[b], temperature=T,
                           bonus=bool(bonus))
            assert (int(na[b]), int(nt[b])) == ref, (case, b)


# ------------------------------------------------------------------ rollback

def test_rollback_state_machine():
    n, T_cap = 4, 64
    say("rollback")
    st = torch.zeros(4, dtype=torch.int32, device=DEV)
    tokens = torch.zeros(T_cap, dtype=torch.int32, device=DEV)
    d = torch.zeros(1, dtype=torch.int32, device=DEV)
    na = torch.zeros(1, dtype=torch.int32, device=DEV)
    nx = torch.zeros(1, dtype=torch.int32, device=DEV)
    ost = O.SeqState(t=10, a=n, tokens=list(range(100, 110)))
    st.copy_(torch.tensor([10, n, 0, 0], dtype=torch.int32))
    tokens[:10] = torch.arange(100, 110, dtype=torch.int32)
    rng = np.random.default_rng(3)
    for step in range(60):
        dv, av, xv = int(rng.integers(0, 1000)), int(rng.random() < 0.5), int(rng.integers(0, 1000))
        d.fill_(dv); na.fill_(av); nx.fill_(xv)
        spd.spd_rollback(st, n, d, na, nx, tokens, T_cap)
        O.transition(ost, n, dv, ost.a == n, av, xv)
        torch.cuda.synchronize()
        assert st.tolist() == [ost.t, ost.a, ost.commits, ost.cycles], step
        assert tokens[:ost.t].tolist() == ost.tokens


# ------------------------------------------------------------------ whole cycles

@pytest.mark.parametrize("schedule", [0, 1, 2], ids=["pre_step", "post_step", "first_stage"])
def test_cycle_trajectory_tiny(schedule):
    """A device-state trajectory (greedy) against the oracle: each cycle's
    features, last hidden row and logits within fp32 tolerance; the decisions the
    device takes equal the oracle decision functions on the device's rows; the
    state after every cycle matches the oracle state machine.  Run under each
    feature schedule (the prefill and every cycle's features follow it)."""
    _greedy_trajectory(synth.TINY.with_(feature_schedule=schedule), 48)


def test_cycle_trajectory_most_stages_and_anchors():
    """The same greedy trajectory at the most stages and anchors the library takes
    (n = 32, m = 8): saturated cycles recompute 33 rows, two row tiles of 32 in every
    product, and each rejection is followed by 31 refill cycles."""
    s = synth.SpdShape("max_stages_anchors", L=32, n=32, anchors=(0, 4, 8, 12, 16, 20, 24, 31), d=64,
                       Ls=1, Hq=4, Hkv=2, hd=16, dff=256, V=512, dtype=synth.F32, ctx=48,
                       temperature=0.0, lm_std=0.02)
    assert s.n == spd.SPD_MAX_STAGES and s.m == spd.SPD_MAX_ANCHORS
    _greedy_trajectory(s, 72)


def _greedy_trajectory(s, ncycles):
    ci = make_inputs(s, device=DEV, T_cap=128)
    model = device_model(ci)
    cyc = SpdCycle(model, 0.0)
    om = OC.model_from_inputs(ci)
    t0 = s.ctx
    ost = O.SeqState(t=t0, a=s.n, tokens=list(range(t0)))
    cyc.set_state(t0, s.n, ost.tokens)
    cyc.prefill(t0 - 1 - s.n)
    cache = OC.prefill(om, t0, s.n)
    wb = synth.cycle_words(ncycles)
    wdev = synth.words_tensor(wb, DEV)
    saturated = 0
    for c in range(ncycles):
        t, a = ost.t, ost.a
        saturated += a == s.n
        say("trajectory cycle", s.name, c, t, a)
        assert cyc.read_state()[:2] == (t, a)
        cyc.cycle(t, a, wdev[c])
        torch.cuda.synchronize()
        out = OC.run_cycle(om, O.SeqState(t=t, a=a, tokens=list(ost.tokens)), cache, {}, 0.0, wb[c])
        assert rel_err(f64(cyc.h_last), out.h_last) < TOL_F32
        gl = cyc.dlogits.cpu().numpy()
        assert rel_err(gl, out.draft_logits) < TOL_F32
        drafted = O.argmax_first(gl)
        assert int(cyc.dtoken.item()) == drafted
        na, nt = -1, -1
        if a == s.n:
            tl = cyc.tlogits.cpu().numpy()
            assert rel_err(tl, out.target_logits) < TOL_F32
            na, nt = O.verify([tl], None, [ost.tokens[t - s.n + 1]], np.zeros((2, 2), np.uint64),
                              temperature=0, bonus=False)
            assert (int(cyc.n_accept.item()), int(cyc.next_token.item())) == (na, nt)
        O.transition(ost, s.n, drafted, a == s.n, na, nt)
        tt, aa, cm, cy = cyc.read_state()
        assert (tt, aa, cm, cy) == (ost.t, ost.a, ost.commits, ost.cycles)
        assert cyc.tokens[:ost.t].tolist() == ost.tokens
        cache.truncate(ost.t - 1 - ost.a)
    assert saturated >= 2


@pytest.mark.parametrize("top_k,top_p", [(0, 1.0), (50, 1.0), (20, 0.8)],
                         ids=["full_softmax", "top_k50", "top_k20_p08"])
def test_cycle_trajectory_tiny_sampled(top_k, top_p):
    """A T = 1 device-state trajectory with rejections and rollbacks: every draft is
    the oracle's draw from the device's (filtered) q row, every verification the
    oracle's decision with the oracle's own ring of q rows (fed with the device's
    rows as they are drafted), the kept sets are the oracle's filters of the
    device's logits, and the state matches the oracle state machine after every
    cycle.  The q row the device verifies against is, bit for bit, the row it
    wrote when that token was drafted n-1 cycles earlier ([SPD] 3.3-3.4)."""
    s = synth.TINY.with_(top_k=top_k, top_p=top_p)
    n = s.n
    ci = make_inputs(s, device=DEV, T_cap=128)
    model = device_model(ci)
    cyc = SpdCycle(model, 1.0)
    om = OC.model_from_inputs(ci)
    t0 = s.ctx
    ost = O.SeqState(t=t0, a=n, tokens=list(range(t0)))
    cyc.set_state(t0, n, ost.tokens)
    cyc.prefill(t0 - 1 - n)
    cache = OC.prefill(om, t0, n)
    # q rows of the n-1 tokens in flight at the start (drafted before the trajectory):
    # the device ring row of position P is P mod n (the library's plan), the oracle's
    # ring is keyed by position
    seed_logits = synth.normal((n, s.V), 3.0, device="cpu", seed=91, name="ring_seed")
    oring, drafted_q = {}, {}
    for i, P in enumerate(range(t0 - n + 1, t0)):
        row = O.filtered_softmax(seed_logits[i].double().numpy(), 1.0, top_k, top_p).astype(np.float32)
        cyc.ring[P % n].copy_(torch.from_numpy(row))
        oring[P] = drafted_q[P] = row
    wb = synth.cycle_words(40, seed=17)
    wdev = synth.words_tensor(wb, DEV)
    verified = rejected = 0
    for c in range(40):
        t, a = ost.t, ost.a
        say("sampled trajectory cycle", c, t, a)
        plan = cyc.plan(t, a)
        assert (plan.verifies == 1) == (a == n) and plan.draft_pos == t
        if plan.verifies:
            assert plan.cand == t - n + 1
            q_dev = cyc.ring[plan.ring_cand].cpu().numpy().copy()
            assert np.array_equal(q_dev.view(np.uint32), drafted_q[plan.cand].view(np.uint32))
        cyc.cycle(t, a, wdev[c])
        torch.cuda.synchronize()
        gq = cyc.ring[plan.ring_draft].cpu().numpy().copy()
        gp = cyc.p.cpu().numpy() if plan.verifies else None
        probs_from = {"q": gq} if gp is None else {"q": gq, "p": gp}
        out = OC.run_cycle(om, O.SeqState(t=t, a=a, tokens=list(ost.tokens)), cache, oring, 1.0,
                           wb[c], probs_from=probs_from)
        drafted_q[t] = gq
        assert rel_err(f64(cyc.h_last), out.h_last) < TOL_F32
        dl = cyc.dlogits.cpu().numpy()
        assert rel_err(dl, out.draft_logits) < TOL_F32
        dref = O.filtered_softmax(dl.astype(np.float64), 1.0, top_k, top_p)
        assert np.array_equal(np.flatnonzero(gq), np.flatnonzero(dref))
        assert int(cyc.dtoken.item()) == out.drafted
        if plan.verifies:
            verified += 1
            rejected += out.n_accept == 0
            assert np.array_equal(out.q_verified.view(np.uint32), q_dev.view(np.uint32))
            tl = cyc.tlogits.cpu().numpy()
            assert rel_err(tl, out.target_logits) < TOL_F32
            tref = O.filtered_softmax(tl.astype(np.float64), 1.0, top_k, top_p)
            assert np.array_equal(np.flatnonzero(gp), np.flatnonzero(tref))
            assert (int(cyc.n_accept.item()), int(cyc.next_token.item())) == (out.n_accept,
                                                                             out.next_token)
        O.transition(ost, n, out.drafted, a == n, out.n_accept, out.next_token)
        assert cyc.read_state() == (ost.t, ost.a, ost.commits, ost.cycles)
        assert cyc.tokens[:ost.t].tolist() == ost.tokens
        cache.truncate(ost.t - 1 - ost.a)
    assert verified >= 5 and rejected >= 1      # rollbacks are exercised


@pytest.mark.parametrize("top_k,top_p", [(0, 1.0), (50, 1.0), (50, 0.9)],
                         ids=["full_softmax", "top_k50", "top_k50_p09"])
def test_cycle_full_headline_sampled(top_k, top_p):
    """One saturated and one partial cycle of the headline workload (T = 1) on a
    seeded committed cache: features, last row, draft/target logits and
    probabilities within bf16 tolerance; the sampled draft, the verify outcome
    and the state update bit-exact on the device's rows.  With the sampling
    filters on, the draft and target rows keep exactly the oracle's sets."""
    s = synth.HEADLINE.with_(top_k=top_k, top_p=top_p)
    ci = make_inputs(s, device=DEV)
    model = device_model(ci)
    cyc = SpdCycle(model, 1.0)
    om = OC.model_from_inputs(ci)
    k, v = synth.kv_cache(s, model.T_cap, device=DEV)
    t = s.ctx
    wb = synth.cycle_words(2, seed=7)
    wdev = synth.words_tensor(wb, DEV)
    qstand = torch.softmax(synth.draft_row_logits(s.V, 3.0, device=DEV, seed=8, name="q_standin"), 0)
    xg = torch.Generator(device=DEV)
    xg.manual_seed(99)
    x = int(torch.multinomial(qstand, 1, generator=xg).item())
    for c, a in enumerate((s.n, 3)):
        say("headline cycle", a)
        tokens = list(range(t))
        tokens[t - s.n + 1] = x
        cyc.k_cache.copy_(k)       # each cycle starts from the seeded committed cache
        cyc.v_cache.copy_(v)
        cyc.set_state(t, a, tokens)
        cyc.cycle(t, a, wdev[c], q_row=qstand)
        torch.cuda.synchronize()
        pos0 = t - 1 - a
        cache = _oracle_cache_from(k, v, pos0, s)
        st = O.SeqState(t=t, a=a, tokens=list(tokens))
        gq = cyc.ring[t % s.n].cpu().numpy()
        gp = cyc.p.cpu().numpy()
        out = OC.run_cycle(om, st, cache, {}, 1.0, wb[c], q_override=qstand.cpu().numpy(),
                           probs_from={"q": gq, "p": gp})
        assert rel_err(f64(cyc.h_last), out.h_last) < TOL_BF16
        assert rel_err(cyc.dlogits.cpu().numpy(), out.draft_logits) < TOL_BF16
        assert int(cyc.dtoken.item()) == out.drafted
        dl = cyc.dlogits.cpu().numpy().astype(np.float64)
        dref = O.filtered_softmax(dl, 1.0, top_k, top_p)
        assert np.array_equal(np.flatnonzero(gq), np.flatnonzero(dref))
        assert np.max(np.abs(gq - dref)) <= 2e-6 * dref.max()
        if a == s.n:
            assert rel_err(cyc.tlogits.cpu().numpy(), out.target_logits) < TOL_BF16
            tl = cyc.tlogits.cpu().numpy().astype(np.float64)
            tref = O.filtered_softmax(tl, 1.0, top_k, top_p)
            assert np.array_equal(np.flatnonzero(gp), np.flatnonzero(tref))
            assert np.max(np.abs(gp - tref)) <= 2e-6 * tref.max()
            assert (int(cyc.n_accept.item()), int(cyc.next_token.item())) == (out.n_accept,
                                                                             out.next_token)
        assert cyc.read_state() == (st.t, st.a, st.commits, st.cycles)


# ------------------------------------------------------------------ whole cycles at full size

def _full_cycle(cyc, om, s, k, v, t, a, tokens, wblock, wdev, qstand):
    """One independent cycle from the seeded committed cache: device and oracle,
    with the oracle's decisions taken on the device's fp32 rows."""
    cyc.k_cache.copy_(k)
    cyc.v_cache.copy_(v)
    cyc.set_state(t, a, tokens)
    cyc.cycle(t, a, wdev, q_row=qstand)
    torch.cuda.synchronize()
    plan = cyc.plan(t, a)
    cache = _oracle_cache_from(k, v, plan.pos0, s)
    st = O.SeqState(t=t, a=a, tokens=list(tokens))
    pf = None
    if s.temperature > 0:
        pf = {"q": cyc.ring[plan.ring_draft].cpu().numpy()}
        if plan.verifies:
            pf["p"] = cyc.p.cpu().numpy()
    out = OC.run_cycle(om, st, cache, {}, s.temperature, wblock,
                       q_override=None if qstand is None else qstand.cpu().numpy(), probs_from=pf)
    assert rel_err(f64(cyc.g[:plan.M]), out.g) < TOL_BF16
    assert rel_err(f64(cyc.h_last), out.h_last) < TOL_BF16
    dl = cyc.dlogits.cpu().numpy()
    assert rel_err(dl, out.draft_logits) < TOL_BF16
    if s.temperature == 0:
        assert int(cyc.dtoken.item()) == O.argmax_first(dl)
    assert int(cyc.dtoken.item()) == out.drafted
    if plan.verifies:
        assert rel_err(cyc.tlogits.cpu().numpy(), out.target_logits) < TOL_BF16
        assert (int(cyc.n_accept.item()), int(cyc.next_token.item())) == (out.n_accept,
                                                                         out.next_token)
    assert cyc.read_state() == (st.t, st.a, st.commits, st.cycles)
    assert cyc.tokens[:st.t].tolist() == st.tokens
    return out


@pytest.mark.parametrize("key", ["qwen35_4b_n4_ls1_greedy", "qwen35_9b_n16_ls4_t1"],
                         ids=["4b_n4_greedy", "9b_n16_sampled"])
def test_cycle_full_size(key):
    """Whole cycles (features -> PDM -> draft head -> target head + verify ->
    rollback) at the Qwen3.5-4B-shaped n = 4 greedy workload and the 9B-shaped
    n = 16, L_s = 4, T = 1 workload at context 4096, on a seeded committed cache:
    a saturated cycle whose verification accepts, one forced to reject (the state
    rolls back to t-n+1 plus the corrected token), and a partial cycle.  Rows within
    the bf16 tolerance, decisions and state bit-exact on the device's rows."""
    s = synth.SHAPES[key]
    say("full cycle", key)
    ci = make_inputs(s, device=DEV)
    model = device_model(ci)
    cyc = SpdCycle(model, s.temperature)
    om = OC.model_from_inputs(ci)
    k, v = synth.kv_cache(s, model.T_cap, device=DEV)
    t, n = s.ctx, s.n
    cand = t - n + 1
    wb = synth.cycle_words(4, seed=29)
    qstand = None
    if s.temperature > 0:
        qstand = torch.softmax(synth.draft_row_logits(s.V, 3.0, device=DEV, seed=8, name="q_standin"), 0)
        wb[:2, 0] = np.uint64(((1 << 24) - 1) << 40)   # R = 2^24 - 1: accept iff q(x) <= p(x)
    wdev = synth.words_tensor(wb, DEV)
    tokens = list(range(t))
    # probe: the target row of the exiting token does not depend on the token under
    # verification, so one saturated cycle gives the row the forced cases choose from
    say("full cycle probe", key)
    _full_cycle(cyc, om, s, k, v, t, n, tokens, wb[0], wdev[0], qstand)
    if s.temperature == 0:
        best = O.argmax_first(cyc.tlogits.cpu().numpy())
        x_acc, x_rej = best, (best + 1) % s.V
    else:
        p = cyc.p.cpu().numpy().astype(np.float64)
        q = qstand.cpu().numpy().astype(np.float64)
        x_acc, x_rej = int(np.argmax(p - q)), int(np.argmax(q - p))
        assert p[x_acc] >= q[x_acc] and q[x_rej] > p[x_rej]
    for c, (x, want) in enumerate(((x_acc, 1), (x_rej, 0))):
        say("full cycle", key, "forced", want)
        toks = list(tokens)
        toks[cand] = x
        out = _full_cycle(cyc, om, s, k, v, t, n, toks, wb[c], wdev[c], qstand)
        assert out.n_accept == want
        if want == 0:
            assert cyc.read_state()[:2] == (t - n + 2, 1)
            assert out.next_token >= 0 and cyc.tokens[cand].item() == out.next_token
    say("full cycle", key, "partial")
    _full_cycle(cyc, om, s, k, v, t, 3, tokens, wb[3], wdev[3], qstand)


# ------------------------------------------------------------------ graph capture

def test_cycle_graph_replay_matches_eager():
    """A saturated and a partial headline cycle captured into one HIP graph (two
    streams, the side head joined by events) and replayed several times, with
    eager work and synchronisations between the replays: every replay's rows,
    draft, target decision and q row equal the eager run bit for bit (the
    library records no memset; its arrival counters return to zero)."""
    s = synth.HEADLINE
    ci = make_inputs(s, device=DEV)
    model = device_model(ci)
    cyc = SpdCycle(model, s.temperature)
    k, v = synth.kv_cache(s, model.T_cap, device=DEV)
    t = s.ctx
    wdev = synth.words_tensor(synth.cycle_words(2, seed=31), DEV)
    qstand = torch.softmax(synth.draft_row_logits(s.V, 3.0, device=DEV, seed=8, name="q_standin"), 0)
    x = torch.full((1,), 17, dtype=torch.int32, device=DEV)

    def run():
        cyc.k_cache.copy_(k)
        cyc.v_cache.copy_(v)
        for c, a in enumerate((s.n, 3)):
            cyc.cycle(t, a, wdev[c], q_row=qstand, x_ptr=x.data_ptr())
        return [cyc.g[:4].clone(), cyc.h_last.clone(), cyc.dlogits.clone(), cyc.dtoken.clone(),
                cyc.tlogits.clone(), cyc.p.clone(), cyc.n_accept.clone(), cyc.next_token.clone(),
                cyc.ring.clone(), cyc.k_cache.clone()]

    say("graph eager")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ref = run()
        ref = run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    keep = {}
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = run()
    torch.cuda.synchronize()
    for r in range(4):
        say("graph replay", r)
        g.replay()
        torch.cuda.synchronize()
        for a_, b_ in zip(outs, ref):
            assert torch.equal(a_, b_), r
        cyc.features(t - 4, 4, 3)        # eager work between replays
        torch.cuda.synchronize()


# ------------------------------------------------------------------ guard regions

GUARD = 4096  # bytes of sentinel on each side of a buffer


class Guarded:
    """A device buffer with sentinel bytes before and after it: a write outside
    the buffer changes the sentinel."""

    def __init__(self, shape, dtype, fill=None):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        self.raw = torch.empty(n + 2 * GUARD, dtype=torch.uint8, device=DEV)
        self.pattern = torch.tensor([0xA5, 0x5A, 0xC3, 0x3C], dtype=torch.uint8, device=DEV)
        self.raw.copy_(self.pattern.repeat((n + 2 * GUARD) // 4 + 1)[:n + 2 * GUARD])
        self.t = self.raw[GUARD:GUARD + n].view(dtype).view(*shape)
        if fill is not None:
            self.t.copy_(fill)
        self.n = n

    def intact(self):
        rep = self.pattern.repeat(GUARD // 4)
        return bool(torch.equal(self.raw[:GUARD], rep) and torch.equal(self.raw[GUARD + self.n:], rep))


@pytest.mark.parametrize("shape,M,a,rows", [(synth.HEADLINE, 9, 8, 1), (synth.HEADLINE, 4, 3, 3),
                                            (synth.HEADLINE, 2048, 0, 1),
                                            (SMALL_BF16.with_(V=4097), 7, 6, 2),
                                            (synth.TINY.with_(V=517), 3, 2, 5)],
                         ids=["headline_sat", "headline_partial", "headline_prefill",
                              "small_ragged", "tiny_ragged"])
def test_calls_write_only_their_buffers(shape, M, a, rows):
    """Every output and the workspace of each call sit between sentinel regions:
    after the feature call, the PDM step, the LM head (T = 0 and T = 1, top-k on
    and off), the verify and the rollback, no sentinel byte has changed, at full
    and ragged sizes."""
    s = shape
    say("guard", s.name, M, a, rows)
    ci = make_inputs(s, device=DEV)
    model = device_model(ci)
    c = model.cfg
    T_cap = model.T_cap
    pos0 = s.ctx - 1 - a if a > 0 else 0
    wdt = torch.bfloat16 if s.dtype == synth.BF16 else torch.float32
    ws = Guarded((max(spd.spd_workspace_size(spd.SPD_CALL_FUSE, c, M),
                      spd.spd_workspace_size(spd.SPD_CALL_PDM, c, M, 0, T_cap)),), torch.uint8,
                 fill=torch.zeros(1, dtype=torch.uint8, device=DEV))
    g = Guarded((M, s.d), torch.float32)
    spd.spd_fuse_features(c, ci.store, T_cap, len(model.store_layers), model.slot_tab, pos0, M, a,
                          ci.fc_norm, ci.w_fc, g.t, ws.t)
    kc = Guarded((s.Ls, s.Hkv, T_cap, s.hd), wdt, fill=torch.zeros(1, dtype=wdt, device=DEV))
    vc = Guarded((s.Ls, s.Hkv, s.hd, T_cap), wdt, fill=torch.zeros(1, dtype=wdt, device=DEV))
    h = Guarded((s.d,), torch.float32)
    spd.spd_pdm_step(c, model.layer_arr, ci.final_norm, kc.t, vc.t, T_cap, g.t, pos0, M, h.t, ws.t)
    torch.cuda.synchronize()
    for b in (ws, g, kc, vc, h):
        assert b.intact()
    hr = synth.normal((rows, s.d), 1.0, device=DEV, seed=5, name="guard_h")
    words = synth.words_tensor(synth.cycle_words(rows, seed=6)[:, :1].copy(), DEV)
    for T, top_k in ((0.0, 0), (1.0, 0), (1.0, min(50, s.V))):
        cfg = spd.spd_config.from_buffer_copy(c)
        cfg.top_k = top_k
        wsh = Guarded((spd.spd_workspace_size(spd.SPD_CALL_LM_HEAD, cfg, rows),), torch.uint8,
                      fill=torch.zeros(1, dtype=torch.uint8, device=DEV))
        lg = Guarded((rows, s.V), torch.float32)
        pr = Guarded((rows, s.V), torch.float32)
        tok = Guarded((rows,), torch.int32)
        spd.spd_lm_head(cfg, ci.w_dlm, hr, rows, T, words if T > 0 else None, lg.t,
                        pr.t if T > 0 else None, tok.t, wsh.t)
        torch.cuda.synchronize()
        for b in (wsh, lg, pr, tok):
            assert b.intact(), (T, top_k)
    # verify (streaming, T = 1, forced rejection so the residual path runs) and rollback
    p = torch.softmax(synth.normal((s.V,), 3.0, device=DEV, seed=7, name="gp"), 0).contiguous()
    q = torch.softmax(synth.normal((s.V,), 3.0, device=DEV, seed=8, name="gq"), 0).contiguous()
    x = int(torch.argmax(q - p).item())
    xd = torch.tensor([x], dtype=torch.int32, device=DEV)
    vw = np.zeros((2, 2), np.uint64)
    vw[0, 0] = np.uint64(((1 << 24) - 1) << 40)
    vwd = synth.words_tensor(vw, DEV)
    wsv = Guarded((spd.spd_workspace_size(spd.SPD_CALL_VERIFY, c, 1, 1),), torch.uint8,
                  fill=torch.zeros(1, dtype=torch.uint8, device=DEV))
    na = Guarded((1,), torch.int32)
    nt = Guarded((1,), torch.int32)
    spd.spd_verify(1, 1, s.V, 1.0, 0, p, q, xd, vwd, na.t, nt.t, wsv.t)
    st = Guarded((4,), torch.int32, fill=torch.tensor([s.ctx, s.n, 0, 0], dtype=torch.int32, device=DEV))
    toks = Guarded((T_cap,), torch.int32, fill=torch.zeros(1, dtype=torch.int32, device=DEV))
    spd.spd_rollback(st.t, s.n, xd, na.t, nt.t, toks.t, T_cap)
    torch.cuda.synchronize()
    assert int(na.t.item()) == 0
    for b in (wsv, na, nt, st, toks):
        assert b.intact()
