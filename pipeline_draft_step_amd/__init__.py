"""Python binding of libspd.so, the MI355X (gfx950) SPD draft-and-verify library.

Argument marshalling only: every step of the cycle runs in the library's HIP
kernels.  Functions carry the C names declared in include/spd.h and take torch
tensors (or raw integer device addresses) for device buffers; torch supplies
device memory and the current stream, nothing else.  A missing library raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspd.so")

SPD_OK, SPD_E_INVALID, SPD_E_UNSUPPORTED, SPD_E_WORKSPACE, SPD_E_HIP = 0, -1, -2, -3, -4
SPD_F32, SPD_BF16 = 0, 1
SPD_ANCHOR_ZERO_MASK, SPD_ANCHOR_CLAMP_MIN = 0, 1
SPD_SCHEDULE_PRE_STEP, SPD_SCHEDULE_POST_STEP, SPD_SCHEDULE_FIRST_STAGE = 0, 1, 2
SPD_CALL_FUSE, SPD_CALL_PDM, SPD_CALL_LM_HEAD, SPD_CALL_VERIFY = 0, 1, 2, 3
SPD_WS_COUNTER_BYTES = 65536
SPD_MAX_ANCHORS = 8
SPD_MAX_STAGES = 32
SPD_TOP_K_MAX = 256
SPD_TREE_MAX_NODES = 64
SPD_NOALLOC_SCRATCH_BYTES = 64 << 20

EXPORTED = (
    "spd_slot_table", "spd_layout", "spd_workspace_size", "spd_fuse_features",
    "spd_pdm_step", "spd_lm_head", "spd_verify", "spd_rollback", "spd_status_string",
    "spd_last_hip_error", "spd_version", "spd_fuse_features_tree", "spd_pdm_step_tree",
    "spd_verify_siblings", "spd_cycle_plan", "spd_lm_head_noalloc", "spd_fuse_features_scaled",
    "spd_fc_prepare", "spd_pdm_prepared_bytes", "spd_pdm_prepare", "spd_pdm_step_prepared",
)


class spd_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("L", "n", "m", "d", "Ls", "Hq", "Hkv", "hd", "dff", "V", "dtype",
                 "anchor_mode", "norm_k0")] + [("rms_eps", ctypes.c_float),
                                               ("rope_theta", ctypes.c_float),
                                               ("feature_schedule", ctypes.c_int32),
                                               ("top_k", ctypes.c_int32),
                                               ("top_p", ctypes.c_float),
                                               ("head_workgroups", ctypes.c_int32)]


class spd_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wqkv", "q_norm", "k_norm", "wo", "mlp_norm", "w_gate_up", "w_down")]


class spd_seq_state(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("t", "a", "commits", "cycles")]


class spd_cycle_info(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("pos0", "M", "verifies", "exiting", "cand", "draft_pos", "ring_draft",
                 "ring_cand")]


class SpdError(RuntimeError):
    def __init__(self, name, rc, hip=0):
        super().__init__(f"{name} failed: {status_string(rc)} ({rc})"
                         + (f", hip error {hip}" if rc == SPD_E_HIP else ""))
        self.status = rc


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float


def lib():
    """The loaded libspd.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with pipeline_draft_step_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        cfgp = ctypes.POINTER(spd_config)
        i32p = ctypes.POINTER(_I32)
        L.spd_slot_table.argtypes = [cfgp, i32p, i32p, i32p, i32p]
        L.spd_layout.argtypes = [_I32, _I32, _I32, i32p, i32p]
        L.spd_cycle_plan.argtypes = [_I32, _I32, _I32, ctypes.POINTER(spd_cycle_info)]
        L.spd_workspace_size.argtypes = [_I32, cfgp, _I32, _I32, _I64]
        L.spd_workspace_size.restype = _SZ
        L.spd_fuse_features.argtypes = [cfgp, _P, _I64, _I32, i32p, _I32, _I32, _I32, _P, _P, _P,
                                        _P, _SZ, _P]
        L.spd_fuse_features_scaled.argtypes = [cfgp, _P, _I64, _I32, i32p, _I32, _I32, _I32, _P, _P,
                                               _P, _P, _P, _SZ, _P]
        L.spd_fc_prepare.argtypes = [cfgp, _P, _P, _P, _P]
        L.spd_pdm_step.argtypes = [cfgp, ctypes.POINTER(spd_layer_weights), _P, _P, _P, _I64, _P,
                                   _I32, _I32, _P, _P, _SZ, _P]
        L.spd_pdm_prepared_bytes.argtypes = [cfgp]
        L.spd_pdm_prepared_bytes.restype = _SZ
        L.spd_pdm_prepare.argtypes = [cfgp, ctypes.POINTER(spd_layer_weights), _P, _SZ, _P]
        L.spd_pdm_step_prepared.argtypes = [cfgp, ctypes.POINTER(spd_layer_weights), _P, _SZ, _P, _P, _P,
                                            _I64, _P, _I32, _I32, _P, _P, _SZ, _P]
        L.spd_lm_head.argtypes = [cfgp, _P, _P, _I32, _F, _P, _P, _P, _P, _P, _SZ, _P]
        L.spd_lm_head_noalloc.argtypes = [cfgp, _P, _P, _I32, _F, _P, _P, _P, _P, _P]
        L.spd_verify.argtypes = [_I32, _I32, _I32, _F, _I32, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
        L.spd_rollback.argtypes = [_P, _I32, _P, _P, _P, _P, _I64, _P]
        L.spd_fuse_features_tree.argtypes = [cfgp, _P, _I64, _I32, i32p, _I32, _I32, _I32, _P, _P,
                                             _P, _P, _P, _SZ, _P]
        L.spd_pdm_step_tree.argtypes = [cfgp, ctypes.POINTER(spd_layer_weights), _P, _P, _P, _I64,
                                        _P, _I32, _I32, _P, _I32, _P, _P, _SZ, _P]
        L.spd_verify_siblings.argtypes = [_I32, _I32, _I32, _F, _P, _P, _P, _P, _P, _P, _P, _SZ,
                                          _P]
        L.spd_status_string.argtypes = [ctypes.c_int]
        L.spd_status_string.restype = ctypes.c_char_p
        L.spd_last_hip_error.restype = ctypes.c_int
        L.spd_version.restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(rc: int) -> str:
    return lib().spd_status_string(rc).decode()


def _check(name, rc):
    if rc < 0:
        raise SpdError(name, rc, lib().spd_last_hip_error())
    return rc


def _ptr(x):
    """Device address of a tensor (must be contiguous), an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_contiguous():
        raise ValueError("device buffers must be contiguous")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _i32_array(values):
    arr = (_I32 * len(values))(*[int(v) for v in values])
    return arr


def make_config(*, L, n, m, d, Ls, Hq, Hkv, hd, dff, V, dtype, anchor_mode=0, norm_k0=0,
                rms_eps=1e-6, rope_theta=1e6, feature_schedule=0, top_k=0,
                top_p=1.0, head_workgroups=0) -> spd_config:
    return spd_config(L, n, m, d, Ls, Hq, Hkv, hd, dff, V, dtype, anchor_mode, norm_k0,
                      rms_eps, rope_theta, feature_schedule, top_k, top_p, head_workgroups)


# ----------------------------------------------------------------- host helpers

def spd_slot_table(cfg: spd_config, anchors):
    m, n = cfg.m, cfg.n
    tab = (_I32 * ((n + 1) * m))()
    layers = (_I32 * (cfg.L + 1))()
    cnt = _I32(0)
    _check("spd_slot_table", lib().spd_slot_table(ctypes.byref(cfg), _i32_array(anchors), tab,
                                                  layers, ctypes.byref(cnt)))
    return list(tab), list(layers)[:cnt.value]


def spd_layout(t: int, a: int, n: int):
    pos = (_I32 * (a + 1))()
    dep = (_I32 * (a + 1))()
    M = _check("spd_layout", lib().spd_layout(t, a, n, pos, dep))
    return list(pos)[:M], list(dep)[:M]


def spd_cycle_plan(t: int, a: int, n: int) -> spd_cycle_info:
    out = spd_cycle_info()
    _check("spd_cycle_plan", lib().spd_cycle_plan(t, a, n, ctypes.byref(out)))
    return out


def spd_workspace_size(call: int, cfg: spd_config, rows: int, gamma: int = 0, T_cap: int = 0) -> int:
    return int(lib().spd_workspace_size(call, ctypes.byref(cfg) if cfg is not None else None,
                                        rows, gamma, T_cap))


# ----------------------------------------------------------------- cycle calls

def spd_fuse_features(cfg, hstore, T_cap, S, slot_tab, pos0, M, a, norm_w, fc_w, g, ws,
                      stream=None):
    _check("spd_fuse_features", lib().spd_fuse_features(
        ctypes.byref(cfg), _ptr(hstore), T_cap, S, _i32_array(slot_tab), pos0, M, a,
        _ptr(norm_w), _ptr(fc_w), _ptr(g), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def spd_fuse_features_scaled(cfg, hstore, T_cap, S, slot_tab, pos0, M, a, norm_w, fc_w, fc_w_scaled,
                             g, ws, stream=None):
    _check("spd_fuse_features_scaled", lib().spd_fuse_features_scaled(
        ctypes.byref(cfg), _ptr(hstore), T_cap, S, _i32_array(slot_tab), pos0, M, a,
        _ptr(norm_w), _ptr(fc_w), _ptr(fc_w_scaled), _ptr(g), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def spd_fc_prepare(cfg, norm_w, fc_w, fc_w_scaled, stream=None):
    _check("spd_fc_prepare", lib().spd_fc_prepare(
        ctypes.byref(cfg), _ptr(norm_w), _ptr(fc_w), _ptr(fc_w_scaled), _stream(stream)))


def layer_weights(layers) -> ctypes.Array:
    """spd_layer_weights[Ls] from a list of dicts of tensors (keys as in include/spd.h)."""
    arr = (spd_layer_weights * len(layers))()
    for i, lw in enumerate(layers):
        for k, _ in spd_layer_weights._fields_:
            setattr(arr[i], k, _ptr(lw[k]))
    return arr


def spd_pdm_prepared_bytes(cfg) -> int:
    """Bytes of the prepared e4m3 weight copies spd_pdm_prepare writes (0: the
    configuration takes none)."""
    return int(lib().spd_pdm_prepared_bytes(ctypes.byref(cfg)))


def spd_pdm_prepare(cfg, layers, prep, stream=None):
    arr = layers if isinstance(layers, ctypes.Array) else layer_weights(layers)
    _check("spd_pdm_prepare", lib().spd_pdm_prepare(
        ctypes.byref(cfg), arr, _ptr(prep), prep.numel() * prep.element_size(), _stream(stream)))


def spd_pdm_step_prepared(cfg, layers, prep, final_norm, k_cache, v_cache, T_cap, g, pos0, M, h_last,
                          ws, stream=None):
    arr = layers if isinstance(layers, ctypes.Array) else layer_weights(layers)
    _check("spd_pdm_step_prepared", lib().spd_pdm_step_prepared(
        ctypes.byref(cfg), arr, _ptr(prep), 0 if prep is None else prep.numel() * prep.element_size(),
        _ptr(final_norm), _ptr(k_cache), _ptr(v_cache), T_cap, _ptr(g), pos0, M, _ptr(h_last), _ptr(ws),
        ws.numel() * ws.element_size(), _stream(stream)))


def spd_pdm_step(cfg, layers, final_norm, k_cache, v_cache, T_cap, g, pos0, M, h_last, ws,
                 stream=None):
    arr = layers if isinstance(layers, ctypes.Array) else layer_weights(layers)
    _check("spd_pdm_step", lib().spd_pdm_step(
        ctypes.byref(cfg), arr, _ptr(final_norm), _ptr(k_cache), _ptr(v_cache), T_cap,
        _ptr(g), pos0, M, _ptr(h_last), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def spd_lm_head(cfg, w_lm, h, rows, temperature, words, logits, probs, token, ws, stream=None):
    _check("spd_lm_head", lib().spd_lm_head(
        ctypes.byref(cfg), _ptr(w_lm), _ptr(h), rows, float(temperature), _ptr(words),
        _ptr(logits), _ptr(probs), _ptr(token), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def spd_lm_head_noalloc(cfg, w_lm, h, rows, temperature, words, logits, probs, token,
                        stream=None):
    _check("spd_lm_head_noalloc", lib().spd_lm_head_noalloc(
        ctypes.byref(cfg), _ptr(w_lm), _ptr(h), rows, float(temperature), _ptr(words),
        _ptr(logits), _ptr(probs), _ptr(token), _stream(stream)))


def spd_verify(B, gamma, V, temperature, bonus, p, q, draft, words, n_accept, next_token, ws,
               stream=None):
    _check("spd_verify", lib().spd_verify(
        B, gamma, V, float(temperature), int(bonus), _ptr(p), _ptr(q), _ptr(draft), _ptr(words),
        _ptr(n_accept), _ptr(next_token), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def spd_rollback(st, n, drafted, n_accept, next_token, tokens, T_cap, stream=None):
    _check("spd_rollback", lib().spd_rollback(
        _ptr(st), n, _ptr(drafted), _ptr(n_accept), _ptr(next_token), _ptr(tokens), T_cap,
        _stream(stream)))


# ----------------------------------------------------------------- draft trees

def spd_fuse_features_tree(cfg, hstore, T_cap, S, slot_tab, pos0, M, a, anc, norm_w, fc_w, g, ws,
                           stream=None):
    _check("spd_fuse_features_tree", lib().spd_fuse_features_tree(
        ctypes.byref(cfg), _ptr(hstore), T_cap, S, _i32_array(slot_tab), pos0, M, a, _ptr(anc),
        _ptr(norm_w), _ptr(fc_w), _ptr(g), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def spd_pdm_step_tree(cfg, layers, final_norm, k_cache, v_cache, T_cap, g, pos0, M, anc, n_out,
                      h_out, ws, stream=None):
    arr = layers if isinstance(layers, ctypes.Array) else layer_weights(layers)
    _check("spd_pdm_step_tree", lib().spd_pdm_step_tree(
        ctypes.byref(cfg), arr, _ptr(final_norm), _ptr(k_cache), _ptr(v_cache), T_cap,
        _ptr(g), pos0, M, _ptr(anc), n_out, _ptr(h_out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream)))


def spd_verify_siblings(B, W, V, temperature, p, q, cand, words, accepted, next_token, ws,
                        stream=None):
    _check("spd_verify_siblings", lib().spd_verify_siblings(
        B, W, V, float(temperature), _ptr(p), _ptr(q), _ptr(cand), _ptr(words), _ptr(accepted),
        _ptr(next_token), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def spd_version() -> int:
    return lib().spd_version()
