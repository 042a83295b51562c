"""Shared helpers of the test suite (conversion and tolerances)."""
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spd.h")

TOL_F32 = 1e-5   # max|gpu - oracle| / rms(oracle), fp32 path
TOL_BF16 = 2e-2  # same, bf16 path


def header_functions():
    """Names of the functions include/spd.h declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(spd_\w+)\s*\(", src, flags=re.M)))


def make_inputs(shape, **kw):
    """synth.cycle_inputs with the anchor store's layers taken from the oracle."""
    import synth
    from oracle import spd as O
    return synth.cycle_inputs(shape, O.store_layers_for(shape.L, shape.n, shape.anchors, shape.anchor_mode),
                              **kw)


def ensure_built():
    import pipeline_draft_step_amd as spd
    if not os.path.exists(spd.LIB_PATH):
        from pipeline_draft_step_amd import build
        build.build(verbose=False)
    return spd


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref)) / max(scale, 1e-30))


def tol_for(dtype_code):
    return TOL_BF16 if dtype_code == 1 else TOL_F32
