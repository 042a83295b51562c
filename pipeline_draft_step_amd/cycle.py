"""Host driver of one SPD draft-and-verify cycle on the device.

Issues the C-ABI calls in the order a cycle needs them ("Speculative Pipeline
Decoding", arXiv 2605.30852, sections 3.1-3.4): features of the rows the cycle
recomputes, the PDM step, the draft head, and -- when the pipeline is saturated
-- the target head on the exiting token's last-layer state, the streaming verify
of its successor, and the commit/rollback.  All arithmetic runs in libspd.so;
this module only allocates buffers and passes pointers.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from . import (SPD_BF16, SPD_CALL_FUSE, SPD_CALL_LM_HEAD, SPD_CALL_PDM, SPD_CALL_VERIFY,
               layer_weights, make_config, spd_config, spd_cycle_plan, spd_fc_prepare,
               spd_fuse_features, spd_fuse_features_scaled,
               spd_lm_head, spd_pdm_prepare, spd_pdm_prepared_bytes, spd_pdm_step_prepared,
               spd_rollback, spd_slot_table, spd_verify, spd_workspace_size)

PREFILL_BLOCK = 256   # rows per PDM prefill call
FEATURE_BLOCK = 2048  # rows per prefill feature call (one large-M FC GEMM)


@dataclass
class DeviceWeights:
    """Device tensors of the synthetic target states and the PDM/heads."""
    store: torch.Tensor       # [T_cap][S][d] anchor states (cfg dtype)
    h_final: torch.Tensor     # [T_cap][d] float32 target last-layer states
    fc_norm: torch.Tensor
    w_fc: torch.Tensor
    layers: list              # dicts with the spd_layer_weights keys
    final_norm: torch.Tensor
    w_dlm: torch.Tensor
    w_tlm: torch.Tensor


class SpdModel:
    def __init__(self, *, L, n, anchors, d, Ls, Hq, Hkv, hd, dff, V, dtype, weights: DeviceWeights,
                 anchor_mode=0, norm_k0=0, eps=1e-6, rope_theta=1e6, feature_schedule=0,
                 top_k=0, top_p=1.0):
        self.cfg = make_config(L=L, n=n, m=len(anchors), d=d, Ls=Ls, Hq=Hq, Hkv=Hkv, hd=hd,
                               dff=dff, V=V, dtype=dtype, anchor_mode=anchor_mode,
                               norm_k0=norm_k0, rms_eps=eps, rope_theta=rope_theta,
                               feature_schedule=feature_schedule, top_k=top_k, top_p=top_p)
        self.anchors = list(anchors)
        self.slot_tab, self.store_layers = spd_slot_table(self.cfg, self.anchors)
        self.w = weights
        self.layer_arr = layer_weights(weights.layers)
        self.T_cap = weights.store.shape[0]
        if weights.store.shape[1] != len(self.store_layers):
            raise ValueError("anchor store does not hold the layers the slot table reads")
        self._fc_scaled = None
        self._pdm_prep = None
        self.use_pdm_prep = True

    def pdm_prep(self):
        """The e4m3 weight copies prefill-sized PDM steps use (prepared on first use on the
        current stream), or None where the configuration takes none or use_pdm_prep is off."""
        if not self.use_pdm_prep:
            return None
        if self._pdm_prep is None:
            nbytes = spd_pdm_prepared_bytes(self.cfg)
            if nbytes == 0:
                return None
            self._pdm_prep = torch.empty(nbytes, dtype=torch.uint8, device=self.w.final_norm.device)
            spd_pdm_prepare(self.cfg, self.layer_arr, self._pdm_prep)
        return self._pdm_prep

    def fc_scaled(self):
        """W_fc with norm_w folded into its columns (bf16; prepared on first use on the
        current stream), or None for fp32 models."""
        if self.cfg.dtype != SPD_BF16:
            return None
        if self._fc_scaled is None:
            self._fc_scaled = torch.empty_like(self.w.w_fc)
            spd_fc_prepare(self.cfg, self.w.fc_norm, self.w.w_fc, self._fc_scaled)
        return self._fc_scaled


class SpdCycle:
    """Buffers of one sequence and the calls of one cycle."""

    def __init__(self, model: SpdModel, temperature: float, device="cuda"):
        c = model.cfg
        # the library refuses stage counts it cannot cycle (n < 2: the token under
        # verification would be the cycle's own draft)
        spd_cycle_plan(c.n + 1, c.n, c.n)
        self.m = model
        self.T = float(temperature)
        self.device = device
        wdt = torch.bfloat16 if c.dtype == SPD_BF16 else torch.float32
        T_cap = model.T_cap
        self.g = torch.empty(max(c.n + 1, PREFILL_BLOCK), c.d, device=device)
        self.g_pre = torch.empty(min(FEATURE_BLOCK, T_cap), c.d, device=device)
        self.h_last = torch.empty(c.d, device=device)
        self.k_cache = torch.zeros(c.Ls, c.Hkv, T_cap, c.hd, dtype=wdt, device=device)
        self.v_cache = torch.zeros(c.Ls, c.Hkv, c.hd, T_cap, dtype=wdt, device=device)
        self.dlogits = torch.empty(c.V, device=device)
        self.ring = torch.empty(c.n, c.V, device=device)
        self.dtoken = torch.zeros(1, dtype=torch.int32, device=device)
        self.tlogits = torch.empty(c.V, device=device)
        self.p = torch.empty(c.V, device=device)
        self.ttoken = torch.zeros(1, dtype=torch.int32, device=device)
        self.n_accept = torch.zeros(1, dtype=torch.int32, device=device)
        self.next_token = torch.zeros(1, dtype=torch.int32, device=device)
        self.state = torch.zeros(4, dtype=torch.int32, device=device)
        self.tokens = torch.zeros(T_cap, dtype=torch.int32, device=device)
        # prefill runs the PDM over whole feature blocks when its large-M path
        # applies (bf16, head size 128), else in PREFILL_BLOCK rows
        self.pdm_block = (min(FEATURE_BLOCK, T_cap) if c.dtype == SPD_BF16 and c.hd == 128
                          else PREFILL_BLOCK)
        ws = max(spd_workspace_size(SPD_CALL_FUSE, c, min(FEATURE_BLOCK, T_cap)),
                 spd_workspace_size(SPD_CALL_FUSE, c, PREFILL_BLOCK),
                 spd_workspace_size(SPD_CALL_PDM, c, self.pdm_block, 0, T_cap),
                 spd_workspace_size(SPD_CALL_PDM, c, PREFILL_BLOCK, 0, T_cap),
                 spd_workspace_size(SPD_CALL_FUSE, c, c.n + 1),
                 spd_workspace_size(SPD_CALL_PDM, c, c.n + 1, 0, T_cap),
                 spd_workspace_size(SPD_CALL_LM_HEAD, c, 1),
                 spd_workspace_size(SPD_CALL_VERIFY, c, 1, 1))
        self.ws = torch.zeros(ws, dtype=torch.uint8, device=device)
        # the target head and verify do not depend on this cycle's draft path: they
        # run on a second stream (default priority) with a workspace of their own
        self.ws_side = torch.zeros(max(spd_workspace_size(SPD_CALL_LM_HEAD, c, 1),
                                       spd_workspace_size(SPD_CALL_VERIFY, c, 1, 1)),
                                   dtype=torch.uint8, device=device)
        self.side = torch.cuda.Stream(device=device)
        # the side stream's head streams beside the latency-bound feature/PDM chain
        # on a capped grid whose waves keep one row's loads in flight at a time.  Its
        # rate should end it about when the chain ends: measured on three workloads
        # (3/4, 1 and 5/4 workgroups per CU), the best cap was 3/4 of the CU count
        # when the head holds less than 1.2x the chain's weight bytes (9B-shaped,
        # n = 16, L_s = 4: 0.7x), one per CU up to 2.5x (n = 8, L_s = 2: 1.8x) and
        # 5/4 above (n = 4, L_s = 1: 3.2x)
        self.cfg_bg = spd_config.from_buffer_copy(c)
        cus = torch.cuda.get_device_properties(device).multi_processor_count
        layer = (c.Hq + 2 * c.Hkv) * c.hd * c.d + c.d * c.Hq * c.hd + 3 * c.dff * c.d
        ratio = c.V * c.d / (c.d * c.m * c.d + c.Ls * layer)
        share = 0.75 if ratio < 1.2 else (1.0 if ratio < 2.5 else 1.25)
        self.cfg_bg.head_workgroups = max(1, int(cus * share))
        self.ev_fork = torch.cuda.Event()
        self.ev_join = torch.cuda.Event()
        self._plans = {}

    # ---------------------------------------------------------------- pieces
    def features(self, pos0, M, a, out=None):
        """Features of rows pos0 .. pos0+M-1 (the last a in flight).  bf16 models pass
        the prepared weights, which prefill-sized calls use to read the anchor store
        directly."""
        m = self.m
        g = self.g if out is None else out
        ws_ = m.fc_scaled()
        if ws_ is None:
            spd_fuse_features(m.cfg, m.w.store, m.T_cap, len(m.store_layers), m.slot_tab, pos0, M, a,
                              m.w.fc_norm, m.w.w_fc, g, self.ws)
        else:
            spd_fuse_features_scaled(m.cfg, m.w.store, m.T_cap, len(m.store_layers), m.slot_tab, pos0,
                                     M, a, m.w.fc_norm, m.w.w_fc, ws_, g, self.ws)
        return g

    def pdm(self, pos0, M, g=None):
        """PDM step over rows pos0 .. pos0+M-1; prefill-sized steps use the model's
        prepared weights where it has them."""
        m = self.m
        spd_pdm_step_prepared(m.cfg, m.layer_arr, m.pdm_prep() if M >= PREFILL_BLOCK else None,
                              m.w.final_norm, self.k_cache, self.v_cache, m.T_cap,
                              self.g if g is None else g, pos0, M, self.h_last, self.ws)
        return self.h_last

    def prefill(self, P: int):
        """Key/value cache of positions 0..P-1, all fully processed (depth n): the
        features of up to FEATURE_BLOCK rows in one call, then the PDM in blocks."""
        for s in range(0, P, FEATURE_BLOCK):
            Mf = min(FEATURE_BLOCK, P - s)
            self.features(s, Mf, 0, out=self.g_pre)
            for b in range(0, Mf, self.pdm_block):
                M = min(self.pdm_block, Mf - b)
                self.pdm(s + b, M, g=self.g_pre[b:b + M])

    def plan(self, t, a):
        """The library's plan of the cycle that starts at length t with a in flight
        (rows, verified and exiting positions, ring rows)."""
        key = (t, a)
        p = self._plans.get(key)
        if p is None:
            p = self._plans[key] = spd_cycle_plan(t, a, self.m.cfg.n)
        return p

    def draft(self, plan, words_block):
        """Draft head on h_last; at T > 0 the q row goes to the plan's ring row."""
        m = self.m
        probs = self.ring[plan.ring_draft] if self.T > 0 else None
        w = None if words_block is None else words_block.data_ptr() + 2 * 8
        spd_lm_head(m.cfg, m.w.w_dlm, self.h_last, 1, self.T, w, self.dlogits, probs, self.dtoken,
                    self.ws)

    def target_and_verify(self, plan, words_block, q_row=None, x_ptr=None, ws=None,
                          background=False):
        """Target head on the exiting token's state and streaming verify of its successor.
        background: the head runs beside the draft chain on a capped grid."""
        m = self.m
        cfg = self.cfg_bg if background else m.cfg
        ws = self.ws if ws is None else ws
        V = m.cfg.V
        h = m.w.h_final[plan.exiting]
        probs = self.p if self.T > 0 else None
        w = None if words_block is None else words_block.data_ptr() + 2 * 8
        spd_lm_head(cfg, m.w.w_tlm, h, 1, self.T, w, self.tlogits, probs, self.ttoken, ws)
        q = q_row if q_row is not None else self.ring[plan.ring_cand]
        draft = x_ptr if x_ptr is not None else self.tokens.data_ptr() + 4 * plan.cand
        spd_verify(1, 1, V, self.T, 0, self.p if self.T > 0 else self.tlogits,
                   q if self.T > 0 else None, draft,
                   None if words_block is None else words_block, self.n_accept, self.next_token,
                   ws)

    def rollback(self):
        m = self.m
        spd_rollback(self.state, m.cfg.n, self.dtoken, self.n_accept, self.next_token,
                     self.tokens, m.T_cap)

    # ---------------------------------------------------------------- a cycle
    def cycle(self, t, a, words_block, q_row=None, x_ptr=None):
        """One cycle at sequence length t with a tokens in flight.  In a saturated
        cycle the target head + verify run on the side stream, concurrently with
        the features -> PDM -> draft chain; rollback waits for both."""
        plan = self.plan(t, a)
        main = torch.cuda.current_stream()
        if plan.verifies:
            self.ev_fork.record(main)
            self.side.wait_event(self.ev_fork)
            with torch.cuda.stream(self.side):
                self.target_and_verify(plan, words_block, q_row, x_ptr, ws=self.ws_side,
                                       background=True)
            self.ev_join.record(self.side)
        self.features(plan.pos0, plan.M, a)
        self.pdm(plan.pos0, plan.M)
        self.draft(plan, words_block)
        if plan.verifies:
            main.wait_event(self.ev_join)
        self.rollback()

    def set_state(self, t, a, tokens=None):
        self.state.copy_(torch.tensor([t, a, 0, 0], dtype=torch.int32))
        if tokens is not None:
            tok = torch.as_tensor(tokens, dtype=torch.int32)
            self.tokens[:tok.numel()].copy_(tok)

    def read_state(self):
        t, a, commits, cycles = self.state.tolist()
        return t, a, commits, cycles
