"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formula: each checks it against a printed
value (tests/golden), a closed form, a library routine (torch, transformers,
numpy), an invariant, or exact counting on a small lattice.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import spd as O


def _golden(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


# ------------------------------------------------------------------ P1, P2

@pytest.mark.parametrize("n", [4, 8, 16])
def test_eligible_sets_L32(golden_dir, n):
    g = _golden(golden_dir, "eligibility_L32.json")
    want = g["zero_mask_eligible"][str(n)]
    for k in range(n + 1):
        got = [l for l in O.slot_layers(k, 32, n, g["anchors"], O.ZERO_MASK) if l >= 0]
        assert got == want[k], (n, k)


def test_eligible_sets_tiny(golden_dir):
    g = _golden(golden_dir, "eligibility_L32.json")["tiny"]
    for k in range(g["n"] + 1):
        got = [l for l in O.slot_layers(k, g["L"], g["n"], g["anchors"]) if l >= 0]
        assert got == g["zero_mask_eligible"][k]


def test_clamp_min_slots(golden_dir):
    g = _golden(golden_dir, "eligibility_L32.json")
    for k, want in enumerate(g["clamp_min_slots_n8"]):
        assert O.slot_layers(k, 32, 8, g["anchors"], O.CLAMP_MIN) == want


def test_eligibility_invariants():
    B = [0, 8, 16, 24, 31]
    for n in (2, 4, 8, 16, 32):
        prev = None
        for k in range(n + 1):
            s = {l for l in O.slot_layers(k, 32, n, B) if l >= 0}
            assert 0 in s                           # the embedding is always there
            if n <= 16:                             # stage depth >= 2: layer 31 needs all stages
                assert (31 in s) == (k == n)
            if prev is not None:
                assert prev <= s                    # features only get richer with depth
            prev = s
    assert O.l_max(0, 32, 8) == 0 and O.l_max(8, 32, 8) == 32
    assert O.l_max(1, 32, 3) == 10                  # floor of 32/3


@pytest.mark.parametrize("n", [4, 8])
def test_post_step_eligible_sets(golden_dir, n):
    g = _golden(golden_dir, "feature_schedules_L32.json")
    want = g["post_step_zero_mask"][str(n)]
    for k in range(n + 1):
        e = O.feature_depth(k, n, O.POST_STEP)
        got = [l for l in O.slot_layers(e, 32, n, g["anchors"], O.ZERO_MASK) if l >= 0]
        assert got == want[k], (n, k)


@pytest.mark.parametrize("n", [4, 8, 16])
def test_first_stage_eligible_sets(golden_dir, n):
    g = _golden(golden_dir, "feature_schedules_L32.json")
    want = g["first_stage_zero_mask"][str(n)]
    for k in range(n + 1):
        e = O.feature_depth(k, n, O.FIRST_STAGE)
        got = [l for l in O.slot_layers(e, 32, n, g["anchors"], O.ZERO_MASK) if l >= 0]
        assert got == want[k], (n, k)
        assert max(got) <= 32 // n            # nothing deeper than the first stage


def test_first_stage_clamp_min_slots(golden_dir):
    g = _golden(golden_dir, "feature_schedules_L32.json")
    for k, want in enumerate(g["first_stage_clamp_min_slots_n8"]):
        assert O.slot_layers(O.feature_depth(k, 8, O.FIRST_STAGE), 32, 8, g["anchors"],
                             O.CLAMP_MIN) == want


def test_schedule_invariants():
    for n in (2, 4, 8, 16):
        for k in range(n + 1):
            assert O.feature_depth(k, n, O.PRE_STEP) == k
            post = O.feature_depth(k, n, O.POST_STEP)
            assert post == (k + 1 if k < n else n)     # one stage deeper, prefix unchanged
            assert O.feature_depth(k, n, O.FIRST_STAGE) <= 1
    with pytest.raises(ValueError):
        O.feature_depth(0, 8, 7)


def test_post_step_newest_row_is_normalised_depth1_feature():
    """[SPD] 3.3's example: post-step gives the newest token g^1, not g^0.  The
    staircase row at depth 0 must then equal the pre-step feature of a depth-1
    row (RMSNorm over the eligible concat, then FC) and differ from FC(H^0)."""
    rng = np.random.default_rng(11)
    d, L, n, B = 16, 8, 4, (0, 4, 7)
    sl, store, gamma, w = _fuse_setup(rng, d, L, n, B)
    g_post = O.fuse_features(store, sl, [6], [0], gamma, w, L=L, n=n, anchors=B,
                             schedule=O.POST_STEP)
    # depth 1 at L = 8, n = 4 reaches layer 2: only the embedding anchor is eligible
    x = torch.tensor(store[6, sl.index(0)])
    ref = F.linear(F.rms_norm(x, (d,), torch.tensor(gamma[:d]), eps=1e-6), torch.tensor(w[:, :d]))
    assert np.allclose(g_post[0], ref.numpy(), rtol=1e-12, atol=1e-12)
    g_pre = O.fuse_features(store, sl, [6], [0], gamma, w, L=L, n=n, anchors=B)
    assert not np.allclose(g_pre[0], g_post[0])
    # the depth-1 row under post-step reads depth 2 (layers 0 and 4)
    g1 = O.fuse_features(store, sl, [6], [1], gamma, w, L=L, n=n, anchors=B, schedule=O.POST_STEP)
    x2 = torch.tensor(np.concatenate([store[6, sl.index(0)], store[6, sl.index(4)]]))
    ref2 = F.linear(F.rms_norm(x2, (2 * d,), torch.tensor(gamma[:2 * d]), eps=1e-6),
                    torch.tensor(w[:, :2 * d]))
    assert np.allclose(g1[0], ref2.numpy(), rtol=1e-12, atol=1e-12)


def test_first_stage_prefix_row_uses_first_stage_only():
    """PPSD's features: a fully processed row (k = n) reads nothing deeper than
    layer L/n, and deeper layers of the store do not change it."""
    rng = np.random.default_rng(12)
    d, L, n, B = 16, 8, 2, (0, 4, 7)
    sl, store, gamma, w = _fuse_setup(rng, d, L, n, B)
    g = O.fuse_features(store, sl, [3], [n], gamma, w, L=L, n=n, anchors=B, schedule=O.FIRST_STAGE)
    x = torch.tensor(np.concatenate([store[3, sl.index(0)], store[3, sl.index(4)]]))   # L/n = 4
    ref = F.linear(F.rms_norm(x, (2 * d,), torch.tensor(gamma[:2 * d]), eps=1e-6),
                   torch.tensor(w[:, :2 * d]))
    assert np.allclose(g[0], ref.numpy(), rtol=1e-12, atol=1e-12)
    store2 = store.copy()
    store2[3, sl.index(7)] += 1.0
    g2 = O.fuse_features(store2, sl, [3], [n], gamma, w, L=L, n=n, anchors=B, schedule=O.FIRST_STAGE)
    assert np.array_equal(g, g2)


def test_layouts(golden_dir):
    g = _golden(golden_dir, "layouts.json")
    for c in g["cases"]:
        want = eval(c["depths"], {})  # literal list expressions from the fixture
        assert O.depths(c["t"], c["a"], c["n"]) == want
    # the partial-fill layout at a = n is Eq. (2)
    assert O.depths(40, 8, 8) == [8] * 32 + list(range(7, -1, -1))
    pos0, pos, dep = O.cycle_rows(2048, 8, 8)
    assert pos0 == 2039 and len(pos) == 9 and dep == [8, 7, 6, 5, 4, 3, 2, 1, 0]
    pos0, pos, dep = O.cycle_rows(2048, 3, 8)
    assert pos0 == 2044 and dep == [8, 2, 1, 0]


# ------------------------------------------------------------------ P3, P4

def _fuse_setup(rng, d=16, L=8, n=4, anchors=(0, 4, 7), T=12, mode=O.ZERO_MASK):
    sl = O.store_layers_for(L, n, anchors, mode)
    store = rng.standard_normal((T, len(sl), d))
    m = len(anchors)
    gamma = rng.uniform(0.5, 1.5, m * d)
    w = rng.standard_normal((d, m * d)) * 0.1
    return sl, store, gamma, w


def test_k0_is_projection_of_embedding():
    rng = np.random.default_rng(1)
    d, L, n, B = 16, 8, 4, (0, 4, 7)
    sl, store, gamma, w = _fuse_setup(rng, d, L, n, B)
    g = O.fuse_features(store, sl, [5], [0], gamma, w, L=L, n=n, anchors=B)
    direct = w[:, :d] @ store[5, sl.index(0)]
    assert np.allclose(g[0], direct, rtol=0, atol=1e-12)
    store2 = store.copy()
    store2[5, 1:] += rng.standard_normal(store2[5, 1:].shape)   # deeper layers change
    g2 = O.fuse_features(store2, sl, [5], [0], gamma, w, L=L, n=n, anchors=B)
    assert np.array_equal(g, g2)
    # clamped mode has the same k = 0 rule
    sl_c, store_c, _, _ = _fuse_setup(np.random.default_rng(1), d, L, n, B, mode=O.CLAMP_MIN)
    gc = O.fuse_features(store_c, sl_c, [5], [0], gamma, w, L=L, n=n, anchors=B, mode=O.CLAMP_MIN)
    assert np.allclose(gc[0], w[:, :d] @ store_c[5, sl_c.index(0)], atol=1e-12)


def test_full_depth_feature_is_rmsnorm_then_linear():
    rng = np.random.default_rng(2)
    d, L, n, B = 16, 8, 4, (0, 4, 7)
    sl, store, gamma, w = _fuse_setup(rng, d, L, n, B)
    g = O.fuse_features(store, sl, [3], [n], gamma, w, L=L, n=n, anchors=B)
    x = torch.tensor(np.concatenate([store[3, sl.index(b)] for b in B]))
    ref = F.linear(F.rms_norm(x, (x.numel(),), torch.tensor(gamma), eps=1e-6), torch.tensor(w))
    assert np.allclose(g[0], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_partial_depth_feature_uses_eligible_anchors_only():
    """Zero-mask reading: the norm runs over the concatenation of the eligible
    anchors and the FC sees zeros in the other slots, i.e. only its columns of
    the eligible slots act."""
    rng = np.random.default_rng(3)
    d, L, n, B = 16, 8, 4, (0, 4, 7)
    sl, store, gamma, w = _fuse_setup(rng, d, L, n, B)
    g = O.fuse_features(store, sl, [7], [2], gamma, w, L=L, n=n, anchors=B)   # anchors 0, 4
    x = torch.tensor(np.concatenate([store[7, sl.index(0)], store[7, sl.index(4)]]))
    ref = F.linear(F.rms_norm(x, (2 * d,), torch.tensor(gamma[:2 * d]), eps=1e-6),
                   torch.tensor(w[:, :2 * d]))
    assert np.allclose(g[0], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_clamped_feature_is_rmsnorm_of_all_slots():
    rng = np.random.default_rng(4)
    d, L, n, B = 16, 32, 8, (0, 8, 16, 24, 31)
    sl, store, gamma, w = _fuse_setup(rng, d, L, n, B, T=4, mode=O.CLAMP_MIN)
    g = O.fuse_features(store, sl, [1], [3], gamma, w, L=L, n=n, anchors=B, mode=O.CLAMP_MIN)
    layers = [0, 8, 12, 12, 12]
    x = torch.tensor(np.concatenate([store[1, sl.index(l)] for l in layers]))
    ref = F.linear(F.rms_norm(x, (x.numel(),), torch.tensor(gamma), eps=1e-6), torch.tensor(w))
    assert np.allclose(g[0], ref.numpy(), rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ P5-P7, P9

def _qwen3_layer(d, Hq, Hkv, hd, dff, seed):
    from transformers import Qwen3Config
    from transformers.models.qwen3 import modeling_qwen3 as mq
    torch.manual_seed(seed)
    c = Qwen3Config(hidden_size=d, intermediate_size=dff, num_attention_heads=Hq,
                    num_key_value_heads=Hkv, head_dim=hd, rms_norm_eps=1e-6, rope_theta=1e6,
                    attention_bias=False)
    c._attn_implementation = "eager"
    layer = mq.Qwen3DecoderLayer(c, 0).double().requires_grad_(False)
    for p in layer.parameters():
        p.normal_(0, 0.05)
    for nm in ("input_layernorm", "post_attention_layernorm"):
        getattr(layer, nm).weight.uniform_(0.5, 1.5)
    layer.self_attn.q_norm.weight.uniform_(0.5, 1.5)
    layer.self_attn.k_norm.weight.uniform_(0.5, 1.5)
    a, m = layer.self_attn, layer.mlp
    lw = dict(attn_norm=layer.input_layernorm.weight.numpy(),
              wqkv=torch.cat([a.q_proj.weight, a.k_proj.weight, a.v_proj.weight]).numpy(),
              q_norm=a.q_norm.weight.numpy(), k_norm=a.k_norm.weight.numpy(),
              wo=a.o_proj.weight.numpy(), mlp_norm=layer.post_attention_layernorm.weight.numpy(),
              w_gate_up=torch.cat([m.gate_proj.weight, m.up_proj.weight]).numpy(),
              w_down=m.down_proj.weight.numpy())
    return c, layer, mq.Qwen3RotaryEmbedding(c), lw


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (6, 2)])
def test_decoder_layer_matches_transformers_qwen3(Hq, Hkv):
    d, hd, dff, T, p0 = 64, 16, 256, 9, 11
    c, layer, rot, lw = _qwen3_layer(d, Hq, Hkv, hd, dff, seed=Hq * 10 + Hkv)
    x = torch.randn(1, T, d, dtype=torch.float64)
    pos = torch.arange(p0, p0 + T)[None]
    cos, sin = rot(x, pos)
    mask = torch.full((T, T), float("-inf"), dtype=torch.float64).triu(1)[None, None]
    y = layer(x, attention_mask=mask, position_ids=pos, position_embeddings=(cos, sin))
    y = y[0] if isinstance(y, tuple) else y
    h, _, _ = O.decoder_layer(x[0].numpy(), list(range(p0, p0 + T)), lw,
                              O.PdmConfig(d=d, Hq=Hq, Hkv=Hkv, hd=hd, dff=dff))
    # transformers builds its rotary tables in float32, hence ~1e-7 agreement
    assert np.abs(h - y[0].numpy()).max() < 1e-6


def test_attention_matches_torch_sdpa():
    rng = np.random.default_rng(5)
    c = O.PdmConfig(d=0, Hq=6, Hkv=2, hd=8, dff=0)
    Tq, P = 5, 7
    q = rng.standard_normal((Tq, 6, 8))
    k = rng.standard_normal((P + Tq, 2, 8))
    v = rng.standard_normal((P + Tq, 2, 8))
    qpos = list(range(P, P + Tq))
    out = O._attend(q, k, v, qpos, list(range(P + Tq)), c)
    kk = torch.tensor(k).repeat_interleave(3, dim=1).permute(1, 0, 2)
    vv = torch.tensor(v).repeat_interleave(3, dim=1).permute(1, 0, 2)
    qq = torch.tensor(q).permute(1, 0, 2)
    mask = torch.arange(P + Tq)[None, :] <= torch.tensor(qpos)[:, None]
    ref = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask).permute(1, 0, 2)
    assert np.allclose(out, ref.numpy(), atol=1e-12)


def test_rope_is_a_rotation_with_relative_phase():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((3, 2, 16))
    y = rng.standard_normal((3, 2, 16))
    for pos in ([0, 5, 900], [3, 1000, 4095]):
        r = O.rope(x, pos, 1e6)
        assert np.allclose(np.linalg.norm(r, axis=-1), np.linalg.norm(x, axis=-1), atol=1e-12)
    # <R_m x, R_n y> depends on m - n only
    a = np.sum(O.rope(x, [10, 10, 10], 1e6) * O.rope(y, [4, 4, 4], 1e6), axis=-1)
    b = np.sum(O.rope(x, [106, 106, 106], 1e6) * O.rope(y, [100, 100, 100], 1e6), axis=-1)
    assert np.allclose(a, b, atol=1e-10)
    assert np.allclose(O.rope(x, [0, 0, 0], 1e6), x)
    assert not np.allclose(O.rope(x, [1, 1, 1], 1e6), x)


def test_silu_and_rmsnorm_match_torch():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((4, 32)) * 3
    assert np.allclose(O.silu(x), F.silu(torch.tensor(x)).numpy(), atol=1e-14)
    w = rng.uniform(0.5, 1.5, 32)
    assert np.allclose(O.rms_norm(x, w, 1e-6),
                       F.rms_norm(torch.tensor(x), (32,), torch.tensor(w), eps=1e-6).numpy(),
                       atol=1e-13)


def _random_pdm(rng, c, Ls):
    def lw():
        return dict(attn_norm=rng.uniform(0.5, 1.5, c.d),
                    wqkv=rng.standard_normal(((c.Hq + 2 * c.Hkv) * c.hd, c.d)) * 0.1,
                    q_norm=rng.uniform(0.5, 1.5, c.hd), k_norm=rng.uniform(0.5, 1.5, c.hd),
                    wo=rng.standard_normal((c.d, c.Hq * c.hd)) * 0.1,
                    mlp_norm=rng.uniform(0.5, 1.5, c.d),
                    w_gate_up=rng.standard_normal((2 * c.dff, c.d)) * 0.1,
                    w_down=rng.standard_normal((c.d, c.dff)) * 0.1)
    return [lw() for _ in range(Ls)], rng.uniform(0.5, 1.5, c.d)


def test_incremental_pdm_equals_full_recompute():
    rng = np.random.default_rng(8)
    c = O.PdmConfig(d=32, Hq=4, Hkv=2, hd=8, dff=64)
    layers, fnorm = _random_pdm(rng, c, 2)
    G = rng.standard_normal((20, 32))
    cache = O.PdmCache(2, c)
    last, _ = O.pdm_step(G[:14], 0, cache, layers, fnorm, c)        # prefill
    assert np.allclose(last, O.pdm_forward(G[:14], layers, fnorm, c), atol=1e-12)
    # cycle: rows 13..19 recomputed with new features (13 reached full depth)
    G2 = G.copy()
    G2[13:] = rng.standard_normal((7, 32))
    last, _ = O.pdm_step(G2[13:], 13, cache, layers, fnorm, c)
    assert np.allclose(last, O.pdm_forward(G2, layers, fnorm, c), atol=1e-12)
    assert cache.length() == 20
    # a stale row in the cache must change the answer (the cache is really read)
    cache.k[0][5] += 1.0
    last2, _ = O.pdm_step(G2[13:], 13, cache, layers, fnorm, c)
    assert not np.allclose(last2, last)


# ------------------------------------------------------------------ draft trees

def _tree_masks(parents):
    """Ancestor masks from a parent list (parents[0] = -1)."""
    anc = []
    for i, p in enumerate(parents):
        anc.append((1 << i) | (anc[p] if p >= 0 else 0))
    return anc


def test_tree_levels_and_rejects_bad_masks():
    anc = _tree_masks([-1, 0, 0, 1, 2, 2, 3])
    assert anc == [1, 3, 5, 11, 21, 37, 75]
    assert O.tree_levels(anc) == [0, 1, 1, 2, 2, 2, 3]
    chain = _tree_masks([-1, 0, 1, 2])
    assert O.tree_levels(chain) == [0, 1, 2, 3]
    for bad in ([3], [1, 2], [1, 3, 7 | 16], [1, 3, 6], [1, 3, 5, 14]):
        with pytest.raises(ValueError):
            O.tree_levels(bad)


def test_tree_rows_of_a_chain_are_the_cycle_layout():
    for n, a in ((8, 8), (8, 3), (4, 1)):
        t = 40
        pos0, pos, dep = O.cycle_rows(t, a, n)
        rows, depth, tpos = O.tree_rows(_tree_masks([-1] + list(range(a))), a, n, pos0)
        assert rows == pos and tpos == pos and depth == dep


def test_tree_rows_branches_share_positions():
    anc = _tree_masks([-1, 0, 0, 0, 0, 1, 1, 2])
    rows, depth, pos = O.tree_rows(anc, 3, 8, 100)
    assert rows == list(range(100, 108))
    assert pos == [100, 101, 101, 101, 101, 102, 102, 102]
    assert depth == [8, 2, 2, 2, 2, 1, 1, 1]


def test_tree_pdm_rows_equal_the_full_forward_of_their_root_paths():
    """Every node's final-normed row equals the definitional causal forward over
    the committed prefix followed by the node's own root path; siblings do not
    see each other."""
    rng = np.random.default_rng(25)
    c = O.PdmConfig(d=32, Hq=4, Hkv=2, hd=8, dff=64)
    layers, fnorm = _random_pdm(rng, c, 2)
    P = 9
    prefix = rng.standard_normal((P, 32))
    cache = O.PdmCache(2, c)
    O.pdm_step(prefix, 0, cache, layers, fnorm, c)
    parents = [-1, 0, 0, 0, 1, 1, 2, 4]
    anc = _tree_masks(parents)
    G = rng.standard_normal((len(parents), 32))
    rows, _ = O.pdm_step_tree(G, P, cache, layers, fnorm, c, anc)
    assert cache.length() == P + len(parents)
    for i in range(len(parents)):
        path = [j for j in range(len(parents)) if (anc[i] >> j) & 1]
        ref = O.pdm_forward(np.concatenate([prefix, G[path]]), layers, fnorm, c)
        assert np.allclose(rows[i], ref, atol=1e-12), i


def test_tree_pdm_of_a_chain_is_the_causal_step():
    rng = np.random.default_rng(26)
    c = O.PdmConfig(d=32, Hq=4, Hkv=4, hd=8, dff=64)
    layers, fnorm = _random_pdm(rng, c, 1)
    prefix = rng.standard_normal((6, 32))
    G = rng.standard_normal((5, 32))
    c1, c2 = O.PdmCache(1, c), O.PdmCache(1, c)
    O.pdm_step(prefix, 0, c1, layers, fnorm, c)
    O.pdm_step(prefix, 0, c2, layers, fnorm, c)
    last, _ = O.pdm_step(G, 6, c1, layers, fnorm, c)
    rows, _ = O.pdm_step_tree(G, 6, c2, layers, fnorm, c, _tree_masks([-1, 0, 1, 2, 3]))
    assert np.allclose(rows[-1], last, atol=1e-13)
    assert np.allclose(c1.k[0], c2.k[0], atol=1e-13) and np.allclose(c1.v[0], c2.v[0], atol=1e-13)


def test_top_k_list_order():
    x = np.random.default_rng(27).standard_normal(3000) * 3
    for k in (1, 4, 50):
        assert O.top_k_list(x, k) == torch.topk(torch.tensor(x), k, sorted=True).indices.tolist()
    ties = np.array([2.0, 5.0, 5.0, np.nan, 1.0, 5.0, 2.0])
    assert O.top_k_list(ties, 5) == [1, 2, 5, 0, 6]
    assert O.top_k_list(ties, 7) == [1, 2, 5, 0, 6, 4, 3]
    assert O.top_k_list(ties, 1) == [O.argmax_first(ties)]


def test_verify_siblings_greedy():
    p = np.array([0.1, 3.0, 2.0, 3.0, -1.0])
    assert O.verify_siblings(p, [2, 1, 3]) == (1, -1)     # argmax is index 1 (first of the ties)
    assert O.verify_siblings(p, [3, 2]) == (-1, 1)        # an equal value is not the argmax
    assert O.verify_siblings(p, [1]) == (0, -1)
    rng = np.random.default_rng(28)
    for _ in range(50):        # one sibling: the streaming greedy verify
        row = rng.standard_normal(64)
        x = int(rng.integers(0, 64)) if rng.random() < 0.5 else O.argmax_first(row)
        na, nt = O.verify([row], None, [x], np.zeros((2, 2), np.uint64), temperature=0,
                          bonus=False)
        acc, nxt = O.verify_siblings(row, [x])
        assert (acc == 0) == (na == 1) and (nxt if acc < 0 else -1) == nt


def _accept_threshold(run, lo=0, hi=1 << 24):
    """Number of R values in [lo, hi) for which run(R) accepts, acceptance being
    monotone (accepts exactly for R below a threshold): binary search."""
    if not run(lo):
        return 0
    while hi - lo > 1:
        mid = (lo + hi) // 2
        if run(mid):
            lo = mid
        else:
            hi = mid
    return hi


def _sibling_law(p, q, W):
    """Exact output law of verify_siblings_sampled with W candidates drawn
    independently from the integer q, computed by calling the oracle as a black
    box: per candidate tuple and round, the accepted share of the 2^24 R lattice
    (binary search on the monotone accept region); after W rejections, the share of
    the 2^32 u lattice each token takes (binary search on the monotone inverse CDF)."""
    V = len(p)
    B = O.sibling_weights(q)
    SB = sum(B)
    law = [Fraction(0)] * V
    rej_all = 1 << 24                   # R that rejects whenever rejection is possible
    for tup in itertools.product(range(V), repeat=W):
        wq = Fraction(1)
        for x in tup:
            wq *= Fraction(B[x], SB)
        if wq == 0:
            continue
        reach = Fraction(1)
        for i in range(W):
            def run(R, i=i):
                words = np.zeros((W + 1, 2), np.uint64)
                for k in range(i):
                    words[k][0] = np.uint64((rej_all - 1) << 40)
                words[i][0] = np.uint64(R << 40)
                acc, _ = O.verify_siblings_sampled(p, q, tup, words)
                return acc == i
            n_acc = _accept_threshold(run)
            law[tup[i]] += wq * reach * Fraction(n_acc, 1 << 24)
            reach *= Fraction((1 << 24) - n_acc, 1 << 24)
            if reach == 0:
                break
        if reach == 0:
            continue

        def draw(u):
            words = np.zeros((W + 1, 2), np.uint64)
            for k in range(W):
                words[k][0] = np.uint64((rej_all - 1) << 40)
            words[W][1] = np.uint64(u << 32)
            return O.verify_siblings_sampled(p, q, tup, words)[1]
        start = 0
        while start < (1 << 32):
            tok = draw(start)
            lo, hi = start, 1 << 32         # last u with the same token: binary search
            while hi - lo > 1:
                mid = (lo + hi) // 2
                if draw(mid) == tok:
                    lo = mid
                else:
                    hi = mid
            law[tok] += wq * reach * Fraction(hi - start, 1 << 32)
            start = hi
    return law


@pytest.mark.parametrize("V,W", [(4, 1), (4, 2), (5, 3)])
def test_sampled_sibling_verify_output_law_is_exactly_p(V, W):
    """Multi-candidate speculative sampling with W independent draws from q
    outputs exactly p (up to the 2^-24 / 2^-32 lattices): checked on small
    vocabularies, including rows with zeros (filtered p and q of different
    supports)."""
    rng = np.random.default_rng(29 + V * 10 + W)
    cases = [(rng.dirichlet(np.ones(V) * 0.7).astype(np.float32),
              rng.dirichlet(np.ones(V) * 0.7).astype(np.float32))]
    lp = rng.standard_normal(V) * 2
    cases.append((O.filtered_softmax(lp, 1.0, V - 1).astype(np.float32),
                  O.filtered_softmax(lp + rng.standard_normal(V), 1.0, V - 1).astype(np.float32)))
    for p, q in cases:
        law = _sibling_law(p, q, W)
        A = O.sibling_weights(p)
        assert abs(float(sum(law)) - 1.0) < 1e-12
        for j in range(V):
            assert abs(float(law[j]) - A[j] / sum(A)) < (W + 1) * V * 2.0 ** -22, (j, W)


def test_sampled_sibling_verify_cases():
    p = np.array([0.5, 0.25, 0.25, 0.0], np.float32)
    q = np.array([0.25, 0.25, 0.25, 0.25], np.float32)
    w = np.zeros((3, 2), np.uint64)
    # p >= q at a token always accepts; p = 0 never does
    assert O.verify_siblings_sampled(p, q, [0, 1], w) == (0, -1)
    w[0][0] = np.uint64(((1 << 24) - 1) << 40)
    assert O.verify_siblings_sampled(p, q, [3, 0], w) == (1, -1)
    # two rejections at token 3: the residual after round 1 is max(0, p - q) = (1/4, 0, 0, 0)
    w[1][0] = np.uint64(((1 << 24) - 1) << 40)
    assert O.verify_siblings_sampled(p, q, [3, 3], w) == (-1, 0)
    # out-of-vocabulary candidates are rejected
    assert O.verify_siblings_sampled(p, q, [7, -1], w)[0] == -1


# ------------------------------------------------------------------ P8

def test_argmax_first_and_nan():
    assert O.argmax_first([1.0, 3.0, 3.0, 2.0]) == 1
    assert O.argmax_first([np.nan, 1.0, 1.0]) == 1
    assert O.argmax_first([-np.inf, -np.inf]) == 0
    x = np.random.default_rng(9).standard_normal(1000)
    assert O.argmax_first(x) == int(np.argmax(x))


def test_softmax_matches_torch():
    x = np.random.default_rng(10).standard_normal(513) * 3
    for T in (1.0, 0.7):
        p = O.softmax(x, T)
        assert abs(p.sum() - 1) < 1e-12
        assert np.allclose(p, torch.softmax(torch.tensor(x) / T, 0).numpy(), atol=1e-15)


# ------------------------------------------------------------------ top-k / top-p filters

def _brute_top_k(x, k):
    """i is kept iff fewer than k entries precede it in the order value descending,
    equal values by ascending index, NaN after every number (rank counting)."""
    V = len(x)

    def precedes(j, i):
        a, b = x[j], x[i]
        if math.isnan(a):
            return math.isnan(b) and j < i
        if math.isnan(b):
            return True
        return a > b or (a == b and j < i)

    return [i for i in range(V) if sum(precedes(j, i) for j in range(V)) < k]


def test_top_k_set_brute_force_with_ties():
    rng = np.random.default_rng(20)
    for trial in range(60):
        V = int(rng.integers(1, 20))
        x = rng.integers(-3, 4, size=V).astype(np.float64)     # many equal values
        if trial % 4 == 0:
            x[rng.integers(0, V)] = np.nan
        if trial % 5 == 0:
            x[rng.integers(0, V)] = -0.0
        for k in range(-1, V + 2):
            want = list(range(V)) if k <= 0 or k >= V else _brute_top_k(list(x), k)
            assert list(O.top_k_set(x, k)) == want, (x, k)


def test_top_k_set_matches_torch_topk_on_distinct_values():
    x = np.random.default_rng(21).standard_normal(4096) * 3
    for k in (1, 50, 257, 4095):
        ref = np.sort(torch.topk(torch.tensor(x), k).indices.numpy())
        assert np.array_equal(O.top_k_set(x, k), ref)


def test_top_k_softmax_is_masked_torch_softmax():
    """top-k alone: softmax of the logits with every other entry set to -inf."""
    x = np.random.default_rng(22).standard_normal(1000) * 3
    for T in (1.0, 0.6):
        for k in (0, 1, 50, 999, 1000):
            xt = torch.tensor(x)
            if 0 < k < len(x):
                idx = torch.topk(xt, k).indices
                masked = torch.full_like(xt, -math.inf)
                masked[idx] = xt[idx]
            else:
                masked = xt
            ref = torch.softmax(masked / T, 0).numpy()
            got = O.filtered_softmax(x, T, k)
            assert np.allclose(got, ref, rtol=0, atol=1e-15)
            assert np.count_nonzero(got) == (k if 0 < k < len(x) else len(x))
    one = O.filtered_softmax(x, 1.0, 1)
    assert one[O.argmax_first(x)] == 1.0 and one.sum() == 1.0


def test_top_p_worked_example():
    """p = (0.4, 0.3, 0.2, 0.1): the nucleus for 0.65 is the first two tokens (0.7
    >= 0.65 > 0.4), for 0.75 the first three; top_p = 1 keeps everything."""
    x = np.log([0.1, 0.4, 0.2, 0.3])
    got = O.filtered_softmax(x, 1.0, 4, 0.65)
    assert np.allclose(got, [0, 4 / 7, 0, 3 / 7], atol=1e-15)
    got = O.filtered_softmax(x, 1.0, 4, 0.75)
    assert np.allclose(got, [0, 4 / 9, 2 / 9, 3 / 9], atol=1e-15)
    assert np.allclose(O.filtered_softmax(x, 1.0, 4, 1.0), [0.1, 0.4, 0.2, 0.3], atol=1e-15)
    assert np.allclose(O.filtered_softmax(x, 1.0, 3, 1e-9), [0, 1, 0, 0], atol=0)
    # top_k = 0: the nucleus over the whole vocabulary (0.4 < 0.5 <= 0.7)
    assert np.allclose(O.filtered_softmax(x, 1.0, 0, 0.5), [0, 4 / 7, 0, 3 / 7], atol=1e-15)
    assert np.allclose(O.filtered_softmax(x, 1.0, 0, 0.95), [0.1, 0.4, 0.2, 0.3], atol=1e-15)
    assert np.allclose(O.filtered_softmax(x, 1.0, 0, 0.85), [0, 4 / 9, 2 / 9, 3 / 9], atol=1e-15)


def test_top_p_matches_ascending_cumulative_removal():
    """A second formulation of the nucleus: sort ascending, drop the tokens whose
    cumulative mass is <= 1 - top_p, always keep the most probable one."""
    rng = np.random.default_rng(23)
    for trial in range(30):
        V = 600
        x = rng.standard_normal(V) * 2.5
        k = int(rng.choice([0, 5, 50, 200, 600]))
        top_p = float(rng.choice([0.2, 0.5, 0.9, 0.97]))
        T = float(rng.choice([1.0, 0.7]))
        xt = torch.tensor(x) / T
        if 0 < k < V:
            idx = torch.topk(xt, k).indices
            masked = torch.full_like(xt, -math.inf)
            masked[idx] = xt[idx]
        else:
            masked = xt
        probs = torch.softmax(masked, 0)
        sp, si = torch.sort(probs)
        remove = torch.cumsum(sp, 0) <= 1 - top_p
        remove[-1] = False
        masked2 = masked.clone()
        masked2[si[remove]] = -math.inf
        ref = torch.softmax(masked2, 0).numpy()
        got = O.filtered_softmax(x, T, k, top_p)
        assert np.allclose(got, ref, rtol=0, atol=1e-14), (trial, k, top_p)


def test_verify_law_is_exactly_filtered_p():
    """Verification with top-k/top-p filtered p and q (zeros outside their sets,
    supports that differ) still outputs exactly p."""
    rng = np.random.default_rng(24)
    for V, k, tp in ((6, 3, 1.0), (8, 4, 0.8), (7, 7, 0.6)):
        for _ in range(3):
            lp = rng.standard_normal(V) * 2
            lq = lp + rng.standard_normal(V)
            p = O.filtered_softmax(lp, 1.0, k, tp).astype(np.float32)
            q = O.filtered_softmax(lq, 1.0, k, tp).astype(np.float32)
            law = _exact_output_distribution(p, q, O.residual_weights)
            ps = sum(Fraction(float(v)) for v in p)
            for j in range(V):
                want = Fraction(float(p[j])) / ps
                assert abs(float(law[j]) - float(want)) < V * 2.0 ** -22
                if p[j] == 0:
                    assert law[j] == 0


# ------------------------------------------------------------------ P11

def test_sampler_interval_boundaries():
    """Each j owns exactly the u in [ceil(C_{j-1} 2^32 / S), ceil(C_j 2^32 / S)),
    C_j the inclusive prefix sums: a reading of 'smallest j with prefix > tau'
    that is off by one in either direction fails at a boundary."""
    rng = np.random.default_rng(11)
    for trial in range(20):
        w = rng.integers(0, 1 << 40, size=7, dtype=np.uint64)
        w[rng.integers(0, 7)] = 0
        S = int(w.sum())
        C = list(itertools.accumulate(int(v) for v in w))
        prev = 0
        for j in range(7):
            lo = prev
            hi = -((-C[j] << 32) // S)     # ceil(C_j 2^32 / S)
            if hi > lo:
                assert O.sample_weights(w, lo) == j
                assert O.sample_weights(w, hi - 1) == j
                assert abs((hi - lo) - int(w[j]) * 2 ** 32 / S) <= 1
            else:
                assert int(w[j]) == 0 or (hi - lo) == 0
            prev = max(prev, hi)
        assert prev == 2 ** 32
    assert O.sample_weights(np.zeros(4, np.uint64), 123) is None


def test_accept_test_counting():
    """#{R in [0, 2^24): accept} = min(2^24, floor(2^24 p / q)) for r = (R+1)/2^24,
    checked at the exact boundary (p, q fp32): P(accept) = min(1, p/q) up to the
    2^-24 lattice, never above it."""
    rng = np.random.default_rng(12)
    for _ in range(200):
        p = float(np.float32(rng.uniform(0, 1)))
        q = float(np.float32(rng.uniform(1e-3, 1)))
        cnt = min(2 ** 24, math.floor(Fraction(p) * 2 ** 24 / Fraction(q)))
        if 0 < cnt < 2 ** 24:
            assert O.accept_test(p, q, cnt - 1)
            assert not O.accept_test(p, q, cnt)
        elif cnt == 2 ** 24:
            assert O.accept_test(p, q, 2 ** 24 - 1)
        else:
            assert not O.accept_test(p, q, 0)
    assert O.accept_test(0.0, 0.0, 2 ** 24 - 1)      # q(x) = 0 accepts
    assert not O.accept_test(0.0, 0.5, 0)            # p(x) = 0 never accepts
    assert O.accept_test(0.5, 0.5, 2 ** 24 - 1)      # p >= q always accepts


# ------------------------------------------------------------------ P12, P13

def _exact_output_distribution(p32, q32, residual_fn):
    """Exact output law of one verify step when x ~ q: sum over drafts x of
    q(x)[acc(x) 1{x} + (1-acc(x)) res], with acc counted on the 24-bit R lattice
    and res counted on the 32-bit U lattice through the sampler's intervals."""
    V = len(p32)
    out = [Fraction(0)] * V
    qf = [Fraction(float(v)) for v in q32]
    qs = sum(qf)
    res_w = residual_fn(p32, q32)
    S = int(res_w.sum())
    if S == 0:
        res_w = O.prob_weights(p32)
        S = int(res_w.sum())
    C = list(itertools.accumulate(int(v) for v in res_w))
    res = []
    prev = 0
    for j in range(V):
        hi = -((-C[j] << 32) // S)
        res.append(Fraction(hi - prev, 2 ** 32))
        prev = hi
    for x in range(V):
        if qf[x] == 0:
            continue
        px, qx = float(p32[x]), float(q32[x])
        cnt = min(2 ** 24, math.floor(Fraction(px) * 2 ** 24 / Fraction(qx)))
        acc = Fraction(cnt, 2 ** 24)
        w = qf[x] / qs
        out[x] += w * acc
        for j in range(V):
            out[j] += w * (1 - acc) * res[j]
    return out


def _pq(rng, V):
    p = rng.dirichlet(np.ones(V) * 0.7).astype(np.float32)
    q = rng.dirichlet(np.ones(V) * 0.7).astype(np.float32)
    return p, q


def test_verify_output_law_is_exactly_p():
    rng = np.random.default_rng(13)
    for V in (2, 5, 8):
        for _ in range(4):
            p, q = _pq(rng, V)
            law = _exact_output_distribution(p, q, O.residual_weights)
            ps = sum(Fraction(float(v)) for v in p)
            for j in range(V):
                assert abs(float(law[j]) - float(Fraction(float(p[j])) / ps)) < V * 2.0 ** -22


def test_resampling_from_p_instead_of_residual_is_biased():
    rng = np.random.default_rng(14)
    p, q = _pq(rng, 6)
    law = _exact_output_distribution(p, q, lambda a, b: O.prob_weights(a))
    assert max(abs(float(law[j]) - float(p[j])) for j in range(6)) > 1e-3


def test_verify_monte_carlo_law_and_acceptance():
    """Monte Carlo through oracle.verify itself: chi-square of the output token
    against p, and the acceptance rate against sum_x min(p, q) = 1 - TVD."""
    from scipy import stats
    rng = np.random.default_rng(15)
    V, N = 6, 60000
    p, q = _pq(rng, V)
    bit = np.random.Philox(key=77)
    words = bit.random_raw(2 * N).astype(np.uint64).reshape(N, 1, 2)
    words = np.concatenate([words, np.zeros((N, 1, 2), np.uint64)], axis=1)
    drafts = rng.choice(V, size=N, p=q.astype(np.float64) / q.sum())
    counts = np.zeros(V)
    acc = 0
    for i in range(N):
        na, nt = O.verify([p], [q], [int(drafts[i])], words[i], temperature=1.0, bonus=False)
        tok = int(drafts[i]) if na == 1 else nt
        acc += na
        counts[tok] += 1
    pe = p.astype(np.float64) / p.sum()
    chi = ((counts - N * pe) ** 2 / (N * pe)).sum()
    assert chi < stats.chi2.ppf(0.999, V - 1)
    alpha = np.minimum(pe, q / q.sum()).sum()
    assert abs(acc / N - alpha) < 4 * math.sqrt(alpha * (1 - alpha) / N)


def test_all_accept_probability_example(golden_dir):
    """alpha^K with K = 5, alpha = 0.8 rounds to the 33% printed on the SSD page.
    Built from five positions whose sum_x min(p, q) is exactly 0.8 and counted
    exactly through the accept test."""
    g = _golden(golden_dir, "acceptance_examples.json")["all_accept"]
    p = np.array([0.5, 0.5, 0.0, 0.0], np.float32)
    q = np.array([0.5, 0.3, 0.2, 0.0], np.float32)   # sum min = 0.8
    alpha = Fraction(0)
    for x in range(4):
        if q[x] > 0:
            cnt = min(2 ** 24, math.floor(Fraction(float(p[x])) * 2 ** 24 / Fraction(float(q[x]))))
            alpha += Fraction(float(q[x])) * Fraction(cnt, 2 ** 24)
    assert abs(float(alpha) - g["alpha"]) < 1e-6
    assert round(100 * float(alpha) ** g["K"]) == g["probability_rounded_percent"]
    # and through the oracle's gamma-form verify (Monte Carlo on 5 i.i.d. positions)
    rng = np.random.default_rng(16)
    N, K = 20000, g["K"]
    words = np.random.Philox(key=5).random_raw(N * (K + 1) * 2).astype(np.uint64).reshape(N, K + 1, 2)
    drafts = rng.choice(4, size=(N, K), p=q.astype(np.float64))
    P = [p] * (K + 1)
    Q = [q] * K
    full = sum(O.verify(P, Q, list(drafts[i]), words[i], temperature=1.0, bonus=True)[0] == K
               for i in range(N))
    a5 = g["alpha"] ** K
    assert abs(full / N - a5) < 4 * math.sqrt(a5 * (1 - a5) / N)


def test_expected_tokens_per_iteration_matches_speedup_formula():
    """At c = 0 the explainer's speedup is the expected tokens per iteration,
    sum_{j<=gamma} alpha^j, bounded by gamma + 1."""
    p = np.array([0.5, 0.5, 0.0, 0.0], np.float32)
    q = np.array([0.5, 0.3, 0.2, 0.0], np.float32)
    gamma, N = 4, 20000
    rng = np.random.default_rng(17)
    words = np.random.Philox(key=9).random_raw(N * (gamma + 1) * 2).astype(np.uint64)
    words = words.reshape(N, gamma + 1, 2)
    drafts = rng.choice(4, size=(N, gamma), p=q.astype(np.float64))
    tok = [O.verify([p] * (gamma + 1), [q] * gamma, list(drafts[i]), words[i],
                    temperature=1.0, bonus=True)[0] + 1 for i in range(N)]
    e = O.expected_speedup(0.8, gamma, 0.0)
    assert abs(e - sum(0.8 ** j for j in range(gamma + 1))) < 1e-12
    assert abs(np.mean(tok) - e) < 4 * np.std(tok) / math.sqrt(N)
    assert O.expected_speedup(0.999999, gamma, 0.0) < gamma + 1


def test_greedy_verify():
    p = np.array([[0.1, 2.0, 2.0, -1.0], [5.0, 0.0, 0.0, 0.0], [0.0, 0.0, 0.0, 9.0]])
    w = np.zeros((3, 2), np.uint64)
    assert O.verify(p, None, [1, 0], w, temperature=0, bonus=True) == (2, 3)
    assert O.verify(p, None, [2, 0], w, temperature=0, bonus=True) == (0, 1)
    assert O.verify(p, None, [1, 3], w, temperature=0, bonus=False) == (1, 0)
    assert O.verify(p[:2], None, [1, 0], w, temperature=0, bonus=False) == (2, -1)


def test_degenerate_residual_falls_back_to_p():
    """Rows need not be normalised: with p = 0.3, q = 0.6 everywhere the residual
    max(0, P - Q) is empty, a high R rejects, and the next token is drawn from p."""
    p = np.array([0.3, 0.3], np.float32)
    q = np.array([0.6, 0.6], np.float32)
    assert O.sample_weights(O.residual_weights(p, q), 5) is None
    hi_r = np.uint64(0xFFFFFF) << np.uint64(40)
    for u, want in ((0, 0), ((1 << 31) - 1, 0), (1 << 31, 1), ((1 << 32) - 1, 1)):
        w = np.array([[hi_r, np.uint64(u) << np.uint64(32)], [0, 0]], np.uint64)
        assert O.verify([p], [q], [0], w, temperature=1.0, bonus=False) == (0, want)
    lo_r = np.array([[0, 0], [0, 0]], np.uint64)                  # R = 0 accepts (1*0.6 <= 0.3*2^24)
    assert O.verify([p], [q], [0], lo_r, temperature=1.0, bonus=False) == (1, -1)


# ------------------------------------------------------------------ P14, rollback

def _simulate(n, beta, cycles, seed):
    rng = np.random.default_rng(seed)
    st = O.SeqState(t=n + 1, a=1, tokens=list(range(n + 1)))
    for _ in range(cycles):
        if st.a == n:
            ok = rng.random() < beta
            O.transition(st, n, 0, True, 1 if ok else 0, 1)
        else:
            O.transition(st, n, 0, False, 0, -1)
    return st


@pytest.mark.parametrize("n,beta", [(8, 0.8), (16, 0.5), (4, 1.0), (4, 0.0)])
def test_step_acceptance_closed_form(n, beta):
    """Each rejection costs n-1 commit-free refill cycles, so under a Bernoulli(beta)
    verifier N/K -> 1 / (1 + (1-beta)(n-1)); L_acc' = (N/K) n."""
    st = _simulate(n, beta, 200000, seed=n)
    want = 1.0 / (1.0 + (1.0 - beta) * (n - 1))
    assert abs(O.step_acceptance(st) - want) < 0.01
    assert abs(O.acceptance_length(st, n) - want * n) < 0.01 * n


def test_rollback_truncates_to_t_minus_n_plus_1():
    n = 4
    st = O.SeqState(t=32, a=4, tokens=list(range(100, 132)))
    O.transition(st, n, drafted=999, verified=True, n_accept=0, next_token=7)
    assert st.t == 30 and st.a == 1                         # kept t-n+1 = 29, + corrected
    assert st.tokens == list(range(100, 129)) + [7]
    assert st.commits == 1 and st.cycles == 1
    verified = []
    for _ in range(n - 1):                                  # refill: no verification
        verified.append(st.a == n)
        O.transition(st, n, drafted=5, verified=False, n_accept=0, next_token=-1)
    assert verified == [False] * (n - 1) and st.a == n
    O.transition(st, n, drafted=6, verified=True, n_accept=1, next_token=-1)
    assert st.a == n and st.t == 34 and st.tokens[-1] == 6 and st.commits == 2
