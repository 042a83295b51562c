"""The allocation-free LM head (spd_lm_head_noalloc, for callers that cannot
allocate) against spd_lm_head with a caller workspace: the same kernels on the
library's own per-GPU scratch array give the same logits, probabilities and
tokens bit for bit, on two calls in a row (the second with a smaller input, so it
runs on what the first left in the array), and sizes beyond the array are refused."""
import ctypes
import sys

import numpy as np
import pytest
import torch

import synth
from spd_testlib import ensure_built

pytestmark = pytest.mark.gpu

spd = ensure_built()
DEV = "cuda"


def _cfg(V, d, top_k=0, top_p=1.0):
    return spd.make_config(L=32, n=8, m=5, d=d, Ls=1, Hq=1, Hkv=1, hd=128, dff=64, V=V, dtype=synth.BF16,
                           top_k=top_k, top_p=top_p)


def _both(cfg, V, d, rows, T, seed):
    print("[case] noalloc", V, d, rows, T, cfg.top_k, flush=True)
    sys.stdout.flush()
    W = synth.normal((V, d), 3.0 / np.sqrt(d), device=DEV, seed=seed, name="w", dtype=torch.bfloat16)
    h = synth.normal((rows, d), 1.0, device=DEV, seed=seed, name="h")
    words = synth.words_tensor(synth.cycle_words(rows, seed=seed)[:, :1].copy(), DEV)
    outs = []
    for mode in ("ws", "noalloc"):
        lg = torch.full((rows, V), float("nan"), device=DEV)
        pr = torch.full((rows, V), float("nan"), device=DEV) if T > 0 else None
        tk = torch.full((rows, cfg.top_k if (T == 0 and cfg.top_k >= 2) else 1), -7, dtype=torch.int32,
                        device=DEV)
        if mode == "ws":
            ws = torch.zeros(spd.spd_workspace_size(spd.SPD_CALL_LM_HEAD, cfg, rows), dtype=torch.uint8,
                             device=DEV)
            spd.spd_lm_head(cfg, W, h, rows, T, words if T > 0 else None, lg, pr, tk, ws)
        else:
            spd.spd_lm_head_noalloc(cfg, W, h, rows, T, words if T > 0 else None, lg, pr, tk)
        torch.cuda.synchronize()
        outs.append((lg, pr, tk))
    (l0, p0, t0), (l1, p1, t1) = outs
    assert torch.equal(l0, l1)
    if T > 0:
        assert torch.equal(p0, p1)
    assert torch.equal(t0, t1)


def test_noalloc_head_matches_workspace_head_twice():
    V, d = 151936, 2560
    # first call: 16 rows, top-k 50 at T = 1 (multi-row path, split-K partials,
    # candidate buffers: 35 MiB of the array)
    _both(_cfg(V, d, top_k=50), V, d, 16, 1.0, 41)
    # second call, smaller: one row, plain softmax at T = 1 (the VALU GEMV path), on
    # the contents the first call left
    _both(_cfg(V, d), V, d, 1, 1.0, 42)
    # and a greedy call on a ragged smaller vocabulary
    _both(_cfg(5003, 512), 5003, 512, 1, 0.0, 43)


def test_noalloc_head_refuses_sizes_beyond_the_array():
    lib = spd.lib()
    fake = 1 << 40
    cfg = _cfg(4_000_000, 2560, top_k=256)
    need = spd.spd_workspace_size(spd.SPD_CALL_LM_HEAD, cfg, 16)
    assert need > spd.SPD_NOALLOC_SCRATCH_BYTES
    rc = lib.spd_lm_head_noalloc(ctypes.byref(cfg), fake, fake, 16, ctypes.c_float(1.0), fake, fake,
                                 fake, fake, None)
    assert rc == spd.SPD_E_WORKSPACE
    for d in (2560, 4096):
        ok = _cfg(151936, d, top_k=256)
        assert spd.spd_workspace_size(spd.SPD_CALL_LM_HEAD, ok, 16) <= spd.SPD_NOALLOC_SCRATCH_BYTES
