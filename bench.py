"""Benchmark of the SPD draft-and-verify cycle on one MI355X.

A step is one cycle of the headline workload (Qwen3.5-4B-shaped PDM with d = 2560,
n = 8 stages, L_s = 2 layers, vocabulary 151936, T = 1, context 2048): anchor
gather + RMSNorm + FC, the PDM step, the draft head with sampling, and -- in
saturated cycles -- the target head, streaming verify and rollback.  Cycles run
in independent mode: each cycle's in-flight count comes from a seeded schedule
(50% saturated, 50% partial fill with a ~ U{1..7}), so no host round trip sits
inside the timed region.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
HEAD_EVERY = 4      # draft-head calls timed in the loop: every 4th cycle
REPEATS = 5         # the timed loop runs this many times; value is the median


TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "spd_lm_head_traffic_headline.md")


def measured_traffic():
    """HBM bytes per spd_lm_head launch from the committed counter summary (two
    rocprofv3 passes, FETCH_SIZE and WRITE_SIZE, scaled by a known-size copy), or
    None when the summary is missing or the kernel sources changed since."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(blob)
        h = hashlib.sha256()
        for f in rec["sources"]:
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != rec["source_sha256"]:
            return None
        return int(rec["traffic_bytes_per_launch"])
    except (OSError, IndexError, KeyError, ValueError):
        return None


def algorithmic_bytes(s, a: int) -> dict:
    """Bytes one cycle must move, by call (weights once, KV read, anchors, rows)."""
    esz = 2 if s.dtype == 1 else 4
    d, m, n, V = s.d, s.m, s.n, s.V
    M = a + 1
    pos0 = s.ctx - 1 - a
    depths = [n] + list(range(a - 1, -1, -1))
    eligible = []
    for k in depths:
        if k == 0:
            eligible.append(1)
        else:
            lm = min(s.L, (k * s.L) // n)
            eligible.append(sum(1 for b in s.anchors if b <= lm))
    fc = d * m * d * esz + sum(eligible) * d * esz + M * d * 4
    layer_w = ((s.Hq + 2 * s.Hkv) * s.hd * d + d * s.Hq * s.hd + 2 * s.dff * d + d * s.dff) * esz
    kv_read = (pos0 + M) * 2 * s.Hkv * s.hd * esz
    pdm = s.Ls * (layer_w + kv_read) + M * d * 4 * 2
    head = V * d * esz + d * 4 + V * 4 * (3 if s.temperature > 0 else 1)
    out = {"fuse": fc, "pdm": pdm, "draft_head": head}
    if a == n:
        out["target_head"] = head
        out["verify"] = 2 * 4 + (2 * V * 4 if s.temperature > 0 else V * 4)
    return out


def cpu_baseline(s, ci, sched, words, qstand_np, x, budget_s=12.0, budget_1t=4.0):
    """The oracle (numpy float64, incremental PDM) on this host, on a time-bounded
    sample of the same cycles: with every BLAS thread, then with one."""
    res = _cpu_run(s, ci, sched, words, qstand_np, x, budget_s)
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = _cpu_run(s, ci, sched, words, qstand_np, x, budget_1t)
        res["one_thread"] = {"value": one["value"], "unit": "cycles/s", "cores": 1,
                             "sample": one["sample"]}
    except ImportError:  # pragma: no cover
        pass
    return res


def _cpu_run(s, ci, sched, words, qstand_np, x, budget_s):
    from oracle import cycle as OC
    from oracle import spd as O
    import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    if ci.store_layers != O.store_layers_for(s.L, s.n, s.anchors, s.anchor_mode):
        raise RuntimeError("anchor store layers differ between the library and the oracle")
    om = OC.model_from_inputs(ci)
    k, v = synth.kv_cache(s, ci.T_cap, device=ci.store.device)
    kk = k.float().cpu().numpy().astype(np.float64)
    vv = v.float().cpu().numpy().astype(np.float64)
    t = s.ctx
    done = 0
    t0 = time.perf_counter()
    while True:
        a = sched[done % len(sched)]
        pos0 = t - 1 - a
        cache = O.PdmCache(s.Ls, om.pdm)
        cache.k = [kk[l].transpose(1, 0, 2)[:pos0] for l in range(s.Ls)]
        cache.v = [vv[l].transpose(2, 0, 1)[:pos0] for l in range(s.Ls)]
        tokens = list(range(t))
        tokens[t - s.n + 1] = x
        st = O.SeqState(t=t, a=a, tokens=tokens)
        OC.run_cycle(om, st, cache, {}, s.temperature, words[done % len(words)],
                     q_override=qstand_np)
        done += 1
        el = time.perf_counter() - t0
        if (el >= budget_s and done >= 4) or done >= 200:
            break
    return {"value": done / el, "unit": "cycles/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{done} cycles of the same schedule (numpy float64 oracle, incremental PDM "
                      f"on a seeded committed cache), {el:.1f} s"}


def _model(spd, synth, s, dev, **kw):
    """Seeded device weights and an SpdModel of shape s (the anchor store holds the
    layers the library's slot table reads)."""
    from pipeline_draft_step_amd.cycle import DeviceWeights, SpdModel
    cfg0 = spd.make_config(L=s.L, n=s.n, m=s.m, d=s.d, Ls=s.Ls, Hq=s.Hq, Hkv=s.Hkv, hd=s.hd, dff=s.dff,
                           V=s.V, dtype=s.dtype, anchor_mode=s.anchor_mode, norm_k0=s.norm_k0)
    ci = synth.cycle_inputs(s, spd.spd_slot_table(cfg0, list(s.anchors))[1], device=dev)
    w = DeviceWeights(store=ci.store, h_final=ci.h_final, fc_norm=ci.fc_norm, w_fc=ci.w_fc,
                      layers=ci.layers, final_norm=ci.final_norm, w_dlm=ci.w_dlm, w_tlm=ci.w_tlm)
    model = SpdModel(L=s.L, n=s.n, anchors=s.anchors, d=s.d, Ls=s.Ls, Hq=s.Hq, Hkv=s.Hkv,
                     hd=s.hd, dff=s.dff, V=s.V, dtype=s.dtype, weights=w, eps=s.eps,
                     rope_theta=s.rope_theta, **kw)
    return ci, w, model


def time_prefills(torch, s, model, cyc, P, reps=3):
    """Whole prefills of the P-row prefix (features + PDM over every layer, rebuilding
    the same cache from the same inputs): reps in the plain form, then reps with
    prepared weights."""
    def time_prefill():
        pf0, pf1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        cyc.prefill(P)
        torch.cuda.synchronize()
        pf0.record()
        for _ in range(reps):
            cyc.prefill(P)
        pf1.record()
        torch.cuda.synchronize()
        return pf0.elapsed_time(pf1) / reps * 1000.0

    model.use_pdm_prep = False
    plain_us = time_prefill()
    model.use_pdm_prep = True
    prep_us = time_prefill()
    pf_flops = prefill_flops(s, P)
    return {"rows": P, "us": round(prep_us, 1),
            "includes": "spd_fuse_features + spd_pdm_step_prepared over the prefix, large-M "
                        "MFMA path (activation residuals on the block-scaled fp8 MFMA)",
            "algorithmic_gflop": round(pf_flops / 1e9, 1),
            "achieved_tflops": round(pf_flops / (prep_us * 1e-6) / 1e12, 1),
            "frac_of_bf16_peak": round(pf_flops / (prep_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "plain_form_us": round(plain_us, 1)}


def prefill_flops(s, P):
    """Multiply-add flops a P-row prefix needs: the feature FC of every row, every
    layer but the last in full (QKV, causal attention, O, gate/up, down), and the last
    layer's keys and values (its other outputs feed only the output row, which is
    negligible)."""
    d, hd, Hq, Hkv, dff = s.d, s.hd, s.Hq, s.Hkv, s.dff
    f = 2.0 * P * d * (s.m * d)
    layer = (2.0 * P * d * (Hq + 2 * Hkv) * hd + 2.0 * 2 * (P * P / 2.0) * hd * Hq
             + 2.0 * P * Hq * hd * d + 2.0 * P * d * 2 * dff + 2.0 * P * dff * d)
    return f + (s.Ls - 1) * layer + 2.0 * P * d * 2 * Hkv * hd


def _stats(ms_list):
    ms = sorted(ms_list)
    return {"median_ms": round(float(np.median(ms)), 4), "min_ms": round(ms[0], 4),
            "max_ms": round(ms[-1], 4), "repeats": len(ms)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--repeats", type=int, default=REPEATS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="headline cycles only (no other workloads or per-call breakdowns)")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only whole prefills of the headline prefix (plain form and "
                         "prepared weights, 10 each) and print their JSON; for counter runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="end with a plain 256 MiB device-to-device copy, the known-size "
                         "reference that scales the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py: this build measures one GPU only (the cycle is a single-GPU "
              "hot path); --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import pipeline_draft_step_amd as spd
    from pipeline_draft_step_amd.cycle import SpdCycle, SpdModel

    spd.lib()
    dev = "cuda"
    s = synth.HEADLINE
    ci, w, model = _model(spd, synth, s, dev)
    cyc = SpdCycle(model, s.temperature, device=dev)
    t = s.ctx
    cyc.set_state(t, s.n, list(range(t)))
    if args.prefill_only:
        print(json.dumps({"prefill": time_prefills(torch, s, model, cyc, t - 1 - s.n, reps=10)}))
        return
    cyc.prefill(t - 1 - s.n)

    total = args.warmup + args.steps
    sched = synth.cycle_schedule(s, total)
    words_np = synth.cycle_words(total)
    words = synth.words_tensor(words_np, dev)
    qstand = torch.softmax(synth.draft_row_logits(s.V, 3.0, device=dev, seed=8, name="q_standin"), 0)
    xg = torch.Generator(device=dev)
    xg.manual_seed(99)
    x_dev = torch.multinomial(qstand, 1, generator=xg).to(torch.int32)
    x = int(x_dev.item())
    torch.cuda.synchronize()

    def one_cycle(cyc, t, a, wblock, timed_head=None):
        """SpdCycle.cycle, with optional events around the draft head."""
        main = torch.cuda.current_stream()
        plan = cyc.plan(t, a)
        if plan.verifies:  # target head + verify on the side stream
            cyc.ev_fork.record(main)
            cyc.side.wait_event(cyc.ev_fork)
            with torch.cuda.stream(cyc.side):
                cyc.target_and_verify(plan, wblock, q_row=qstand_of[id(cyc)], x_ptr=x_of[id(cyc)],
                                      ws=cyc.ws_side, background=True)
            cyc.ev_join.record(cyc.side)
        cyc.features(plan.pos0, plan.M, a)
        cyc.pdm(plan.pos0, plan.M)
        if timed_head is not None:
            timed_head[0].record()
        cyc.draft(plan, wblock)
        if timed_head is not None:
            timed_head[1].record()
        if plan.verifies:
            main.wait_event(cyc.ev_join)
        cyc.rollback()

    qstand_of = {id(cyc): qstand}
    x_of = {id(cyc): x_dev.data_ptr()}

    def run_cycles(cyc, t, sched, words, steps, repeats, head_events=True):
        """warmup, then `repeats` timed loops of `steps` cycles; returns (ms per cycle of
        each loop, mean draft-head ms, wall s of the last loop)."""
        for c in range(args.warmup):
            one_cycle(cyc, t, sched[c], words[c])
        torch.cuda.synchronize()
        loops, heads, wall = [], [], 0.0
        for _ in range(repeats):
            # events bracket the draft-head call of every HEAD_EVERY-th cycle (a timing
            # event costs a few us of GPU time; on every cycle they would slow the loop)
            hev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(0, steps, HEAD_EVERY)] if head_events else []
            start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            wall0 = time.perf_counter()
            start.record()
            for i in range(steps):
                c = args.warmup + i
                th = hev[i // HEAD_EVERY] if head_events and i % HEAD_EVERY == 0 else None
                one_cycle(cyc, t, sched[c], words[c], th)
            stop.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - wall0
            loops.append(start.elapsed_time(stop) / steps)
            heads += [e0.elapsed_time(e1) for e0, e1 in hev]
        return loops, (float(np.mean(heads)) if heads else None), wall

    loops, head_ms, wall = run_cycles(cyc, t, sched, words, args.steps, args.repeats)
    ms_per_step = float(np.median(loops))
    cycles_per_s = 1000.0 / ms_per_step

    timed = sched[args.warmup:]
    cyc_bytes = [sum(algorithmic_bytes(s, a).values()) for a in timed]
    mean_bytes = float(np.mean(cyc_bytes))
    head_bytes = algorithmic_bytes(s, s.n)["draft_head"]
    achieved = head_bytes / (head_ms * 1e-3) / 1e9

    result = {
        "metric": "draft+verify cycles/s + achieved HBM GB/s, d=2560 n=8 vocab 151936, 1 GPU",
        "value": round(cycles_per_s, 2),
        "unit": "cycles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "spd_cycle_qwen35_4b_shape_n8_ls2_t1_mix", "d": s.d, "n": s.n,
                   "L": s.L, "anchors": list(s.anchors), "Ls": s.Ls, "heads": [s.Hq, s.Hkv, s.hd],
                   "dff": s.dff, "vocab": s.V, "context": s.ctx, "temperature": s.temperature,
                   "mix": "50% saturated / 50% partial a~U{1..7}", "batch": 1,
                   "mode": "independent cycles"},
        "timed_loops": dict(_stats(loops), steps_each=args.steps,
                            cycles_per_s_each=[round(1000.0 / v, 1) for v in loops]),
        "achieved_hbm_gbs": round(mean_bytes * cycles_per_s / 1e9, 1),
        "algorithmic_MB_per_cycle": round(mean_bytes / 1e6, 2),
        "roofline": {"bound": "hbm", "kernel": "spd_lm_head (vocab GEMV + softmax/sample)",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
                     "avg_us": round(head_ms * 1000.0, 2),
                     "algorithmic_bytes_per_launch": int(head_bytes)},
        "wall_s_timed": round(wall, 3),
    }

    if not args.no_extra:
        extra(args, torch, synth, spd, SpdCycle, SpdModel, s, ci, w, model, cyc, t, sched, words,
              qstand, x_dev, one_cycle, run_cycles, qstand_of, x_of, head_ms, result)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(s, ci, timed[:64],
                                              words_np[args.warmup:], qstand.cpu().numpy(), x,
                                              budget_s=args.cpu_budget)
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(result), flush=True)


def extra(args, torch, synth, spd, SpdCycle, SpdModel, s, ci, w, model, cyc, t, sched, words,
          qstand, x_dev, one_cycle, run_cycles, qstand_of, x_of, head_ms, result):
    """Per-call breakdown, graph-captured cycles, prefill, the sampling filters, the
    draft tree, and the other workloads (n = 4 greedy, 9B-shaped n = 16, the batched
    verify)."""
    dev = "cuda"
    total = len(sched)

    # per-call breakdown (separate instrumented pass over one saturated and one partial cycle)
    calls = {}
    for a in (s.n, 3):
        plan = cyc.plan(t, a)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(7)]
        reps = 20
        acc = np.zeros(6)
        for r in range(reps):
            c = r % total
            ev[0].record()
            cyc.features(plan.pos0, plan.M, a)
            ev[1].record()
            cyc.pdm(plan.pos0, plan.M)
            ev[2].record()
            cyc.draft(plan, words[c])
            ev[3].record()
            if plan.verifies:
                cyc.target_and_verify(plan, words[c], q_row=qstand, x_ptr=x_dev.data_ptr())
            ev[4].record()
            cyc.rollback()
            ev[5].record()
            torch.cuda.synchronize()
            acc += [ev[i].elapsed_time(ev[i + 1]) for i in range(5)] + [ev[0].elapsed_time(ev[5])]
        acc = acc / reps * 1000.0
        calls["saturated" if a == s.n else f"partial_a{a}"] = {
            "fuse_us": round(acc[0], 1), "pdm_us": round(acc[1], 1),
            "draft_head_us": round(acc[2], 1), "target_head_verify_us": round(acc[3], 1),
            "rollback_us": round(acc[4], 1), "cycle_us": round(acc[5], 1),
            "algorithmic_MB": round(sum(algorithmic_bytes(s, a).values()) / 1e6, 1)}
    result["calls"] = calls

    # the same timed schedule captured into HIP graphs (GRAPH_CYCLES cycles per graph,
    # both streams), replayed back to back
    GRAPH_CYCLES = 8
    nsteps = max(GRAPH_CYCLES, (args.steps // GRAPH_CYCLES) * GRAPH_CYCLES)
    graphs = []
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in range(GRAPH_CYCLES):
            one_cycle(cyc, t, sched[c], words[c])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for g0 in range(0, nsteps, GRAPH_CYCLES):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(g0, g0 + GRAPH_CYCLES):
                c = args.warmup + (i % args.steps)
                one_cycle(cyc, t, sched[c], words[c])
        graphs.append(g)
    torch.cuda.synchronize()
    for g in graphs[:2]:
        g.replay()
    torch.cuda.synchronize()
    gl = []
    for _ in range(args.repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for g in graphs:
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        gl.append(e0.elapsed_time(e1) / nsteps)
    result["graph_captured"] = dict(_stats(gl), cycles_per_s=round(1000.0 / float(np.median(gl)), 2),
                                    cycles_per_graph=GRAPH_CYCLES, steps=nsteps)
    del graphs

    # a real trajectory: each cycle starts from the state the previous one left on
    # the device (commit or rollback), read back by the host (one device-to-host
    # read and synchronisation per cycle), with the q ring of the trajectory itself
    cyc.set_state(t, s.n, list(range(t)))
    cyc.prefill(t - 1 - s.n)
    for r in range(s.n):
        cyc.ring[r].copy_(qstand)
    tw = synth.words_tensor(synth.cycle_words(args.warmup + args.steps, seed=41), dev)
    st = cyc.read_state()
    for c in range(args.warmup):
        cyc.cycle(st[0], st[1], tw[c])
        st = cyc.read_state()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    sat = done = 0
    for c in range(args.warmup, args.warmup + args.steps):
        if st[0] + 2 > model.T_cap:   # the sequence would outgrow the cache
            break
        sat += st[1] == s.n
        cyc.cycle(st[0], st[1], tw[c])
        st = cyc.read_state()
        done += 1
    el = time.perf_counter() - t0
    result["trajectory"] = {
        "cycles": done, "cycles_per_s": round(done / el, 2),
        "saturated_fraction": round(sat / max(done, 1), 3), "commits_per_cycle": round(st[2] / max(st[3], 1), 4),
        "note": "host reads (t, a) after every cycle; random weights reject almost every verification, so "
                "each rejection is followed by n-1 draft-only refill cycles"}

    # prefill feature call (every row at depth n), timed as a whole on the launch
    # stream: the fused form (the product reads the anchor store and forms the row
    # statistics; prepared weights) and the two-launch form (gather, then product)
    Mp = min(2048, cyc.g_pre.shape[0])
    m_anch = len(s.anchors)

    def time_call(fn, reps=20):
        for _ in range(3):
            fn()
        pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        pe0.record()
        for _ in range(reps):
            fn()
        pe1.record()
        torch.cuda.synchronize()
        return pe0.elapsed_time(pe1) / reps * 1000.0

    pre_us = time_call(lambda: cyc.features(0, Mp, 0, out=cyc.g_pre))
    gather_us = time_call(lambda: spd.spd_fuse_features(
        model.cfg, w.store, model.T_cap, len(model.store_layers), model.slot_tab, 0, Mp, 0, w.fc_norm,
        w.w_fc, cyc.g_pre, cyc.ws))
    pre_flops = 2.0 * Mp * s.d * (m_anch * s.d)
    pre_tflops = pre_flops / (pre_us * 1e-6) / 1e12
    result["prefill_fc"] = {
        "M": Mp, "N": s.d, "K": m_anch * s.d, "call_us": round(pre_us, 2),
        "includes": "RMSNorm + FC over the anchor store in one launch (spd_fuse_features_scaled, "
                    "weights prepared once by spd_fc_prepare)",
        "achieved_tflops": round(pre_tflops, 1), "bound": "mfma", "peak_tflops": BF16_PEAK_TFLOPS,
        "frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
        "gather_then_gemm_call_us": round(gather_us, 2),
        "gather_then_gemm_frac": round(pre_flops / (gather_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4)}

    # whole prefill of the 2039-row prefix (features + PDM over every layer); it
    # rebuilds the same cache from the same inputs
    result["prefill"] = time_prefills(torch, s, model, cyc, t - 1 - s.n)

    # the pages' sampling setting (T = 1, top-k = 50, top-p = 1.0) on both heads: the
    # same cycles through a second model whose heads filter
    model_k = SpdModel(L=s.L, n=s.n, anchors=s.anchors, d=s.d, Ls=s.Ls, Hq=s.Hq, Hkv=s.Hkv,
                       hd=s.hd, dff=s.dff, V=s.V, dtype=s.dtype, weights=w, eps=s.eps,
                       rope_theta=s.rope_theta, top_k=50, top_p=1.0)
    cyc_k = SpdCycle(model_k, s.temperature, device=dev)
    cyc_k.set_state(t, s.n, list(range(t)))
    cyc_k.prefill(t - 1 - s.n)
    qstand_of[id(cyc_k)], x_of[id(cyc_k)] = qstand, x_dev.data_ptr()
    lk, head_k, _ = run_cycles(cyc_k, t, sched, words, max(args.steps // 2, 1), 3)
    ms_k = float(np.median(lk))
    result["sampling_top_k50"] = {
        "top_k": 50, "top_p": 1.0, "cycles_per_s": round(1000.0 / ms_k, 2),
        "ms_per_step": round(ms_k, 4), "draft_head_us": round(head_k * 1000.0, 2),
        "draft_head_us_unfiltered": round(head_ms * 1000.0, 2)}
    del cyc_k, model_k

    result["draft_tree_w4"] = tree_step(torch, synth, spd, s, w, model, cyc, t)

    # the other workloads: Qwen3.5-4B-shaped n = 4 (L_s = 1, greedy) and 9B-shaped
    # n = 16 (L_s = 4, T = 1, context 4096), saturated every cycle, on a seeded
    # committed cache
    del cyc
    torch.cuda.empty_cache()
    others = {}
    for key, name in (("qwen35_4b_n4_ls1_greedy", "spd_cycle_qwen35_4b_shape_n4_ls1_t0"),
                      ("qwen35_9b_n16_ls4_t1", "spd_cycle_qwen35_9b_shape_n16_ls4_t1")):
        so = synth.SHAPES[key]
        ci_o, w_o, model_o = _model(spd, synth, so, dev)
        cyc_o = SpdCycle(model_o, so.temperature, device=dev)
        k, v = synth.kv_cache(so, model_o.T_cap, device=dev)
        cyc_o.k_cache.copy_(k)
        cyc_o.v_cache.copy_(v)
        del k, v
        to = so.ctx
        cyc_o.set_state(to, so.n, list(range(to)))
        q_o = torch.softmax(synth.draft_row_logits(so.V, 3.0, device=dev, seed=8, name="q_standin"), 0)
        qstand_of[id(cyc_o)], x_of[id(cyc_o)] = q_o, x_dev.data_ptr()
        steps_o = max(args.steps // 4, 8)
        sched_o = [so.n] * (args.warmup + steps_o)
        words_o = synth.words_tensor(synth.cycle_words(args.warmup + steps_o), dev)
        lo, _, _ = run_cycles(cyc_o, to, sched_o, words_o, steps_o, 3, head_events=False)
        ms_o = float(np.median(lo))
        mb = sum(algorithmic_bytes(so, so.n).values())
        gbs = mb * (1000.0 / ms_o) / 1e9
        others[name] = {"d": so.d, "n": so.n, "Ls": so.Ls, "vocab": so.V, "context": so.ctx,
                        "temperature": so.temperature, "saturated": True,
                        "cycles_per_s": round(1000.0 / ms_o, 2), "ms_per_step": round(ms_o, 4),
                        "timed_loops": _stats(lo), "algorithmic_MB_per_cycle": round(mb / 1e6, 1),
                        "achieved_hbm_gbs": round(gbs, 1),
                        "frac_of_hbm_ceiling": round(gbs / HBM_PEAK_GBS, 4)}
        del cyc_o, model_o, w_o, ci_o, q_o
        torch.cuda.empty_cache()

    # batched verify stress: 64 sequences x gamma = 7 drafts, bonus on full accept,
    # 100 back-to-back calls.  Algorithmic bytes of one call: the 2 gamma scalars per
    # sequence it tests, then the rows its outcome needs (residual: p and q of the
    # rejected position; bonus: p of position gamma) read once
    vs = synth.VERIFY_STRESS
    p, q, draft, vwords = synth.verify_stress_inputs(vs, device=dev)
    vw = synth.words_tensor(vwords, dev)
    na = torch.zeros(vs.B, dtype=torch.int32, device=dev)
    nt = torch.zeros(vs.B, dtype=torch.int32, device=dev)
    cfgv = spd.make_config(L=1, n=2, m=1, d=64, Ls=0, Hq=1, Hkv=1, hd=64, dff=64, V=vs.V, dtype=1)
    wsv = torch.zeros(spd.spd_workspace_size(spd.SPD_CALL_VERIFY, cfgv, vs.B, vs.gamma),
                      dtype=torch.uint8, device=dev)
    for _ in range(5):
        spd.spd_verify(vs.B, vs.gamma, vs.V, vs.temperature, vs.bonus, p, q, draft, vw, na, nt, wsv)
    torch.cuda.synchronize()
    nacc = na.cpu().numpy()
    rows_read = sum(1 if int(k) == vs.gamma else 2 for k in nacc)
    scalars = sum(2 * (min(int(k) + 1, vs.gamma)) for k in nacc)
    vbytes = rows_read * vs.V * 4 + scalars * 4 + vs.B * vs.gamma * 4 + vs.B * 8
    vl = []
    for _ in range(args.repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(100):
            spd.spd_verify(vs.B, vs.gamma, vs.V, vs.temperature, vs.bonus, p, q, draft, vw, na, nt,
                           wsv)
        e1.record()
        torch.cuda.synchronize()
        vl.append(e0.elapsed_time(e1) / 100)
    vms = float(np.median(vl))
    others["verify_stress_b64_g7"] = {
        "B": vs.B, "gamma": vs.gamma, "vocab": vs.V, "bonus": vs.bonus, "calls": 100,
        "calls_per_s": round(1000.0 / vms, 1), "us_per_call": round(vms * 1000.0, 2),
        "timed_loops": _stats(vl), "mean_accepted": round(float(nacc.mean()), 3),
        "algorithmic_MB_per_call": round(vbytes / 1e6, 2),
        "achieved_gbs": round(vbytes / (vms * 1e-3) / 1e9, 1),
        "dense_MB_per_call": round((p.numel() + q.numel()) * 4 / 1e6, 1)}
    result["other_workloads"] = others


def tree_step(torch, synth, spd, s, w, model, cyc, t):
    """Greedy width-4 draft tree at the saturated depth: features and PDM over the 29
    tree nodes (root + 7 levels of 4), the top-4 children of the 4 deepest nodes,
    greedy verification of the 4 oldest siblings."""
    dev = "cuda"
    W_tree, a_tree = 4, s.n - 1
    parents, prev = [-1], [0]
    for lvl in range(a_tree):
        cur = []
        for i in range(W_tree):
            parents.append(0 if lvl == 0 else prev[min(i // 2, len(prev) - 1)])
            cur.append(len(parents) - 1)
        prev = cur
    anc = []
    for i, par in enumerate(parents):
        anc.append((1 << i) | (anc[par] if par >= 0 else 0))
    Mt = len(anc)
    anc_d = torch.tensor(anc, dtype=torch.int64, device=dev)
    cfg_t = spd.spd_config.from_buffer_copy(model.cfg)
    cfg_t.top_k = W_tree
    ws_t = torch.zeros(max(spd.spd_workspace_size(spd.SPD_CALL_FUSE, cfg_t, Mt),
                           spd.spd_workspace_size(spd.SPD_CALL_PDM, cfg_t, Mt, 0, model.T_cap),
                           spd.spd_workspace_size(spd.SPD_CALL_LM_HEAD, cfg_t, W_tree),
                           spd.spd_workspace_size(spd.SPD_CALL_VERIFY, cfg_t, 1, 0)),
                       dtype=torch.uint8, device=dev)
    g_t = torch.empty(Mt, s.d, device=dev)
    h_t = torch.empty(W_tree, s.d, device=dev)
    lg_t = torch.empty(W_tree, s.V, device=dev)
    kids = torch.empty(W_tree, W_tree, dtype=torch.int32, device=dev)
    acc_t = torch.empty(1, dtype=torch.int32, device=dev)
    nxt_t = torch.empty(1, dtype=torch.int32, device=dev)
    pos0_t = t - 1 - s.n

    def tree_step(ev=None):
        rec = (lambda i: ev[i].record()) if ev else (lambda i: None)
        rec(0)
        spd.spd_fuse_features_tree(cfg_t, w.store, model.T_cap, len(model.store_layers),
                                   model.slot_tab, pos0_t, Mt, a_tree, anc_d, w.fc_norm, w.w_fc,
                                   g_t, ws_t)
        rec(1)
        spd.spd_pdm_step_tree(cfg_t, model.layer_arr, w.final_norm, cyc.k_cache, cyc.v_cache,
                              model.T_cap, g_t, pos0_t, Mt, anc_d, W_tree, h_t, ws_t)
        rec(2)
        spd.spd_lm_head(cfg_t, w.w_dlm, h_t, W_tree, 0.0, None, lg_t, None, kids, ws_t)
        rec(3)
        spd.spd_verify_siblings(1, W_tree, s.V, 0.0, cyc.tlogits, None, kids, None, acc_t, nxt_t,
                                ws_t)
        rec(4)

    for _ in range(5):
        tree_step()
    tacc = np.zeros(4)
    reps = 20
    for _ in range(reps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(5)]
        tree_step(ev)
        torch.cuda.synchronize()
        tacc += [ev[i].elapsed_time(ev[i + 1]) for i in range(4)]
    tacc = tacc / reps * 1000.0
    # T = 1 sibling verification, worst case: every round rejects (W passes pairs over V)
    rej = np.zeros((W_tree + 1, 2), np.uint64)
    rej[:W_tree, 0] = np.uint64(((1 << 24) - 1) << 40)
    rej_d = synth.words_tensor(rej, dev)
    qrow = cyc.ring[0:1]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    spd.spd_verify_siblings(1, W_tree, s.V, 1.0, cyc.p, qrow, kids, rej_d, acc_t, nxt_t, ws_t)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        spd.spd_verify_siblings(1, W_tree, s.V, 1.0, cyc.p, qrow, kids, rej_d, acc_t, nxt_t, ws_t)
    e1.record()
    torch.cuda.synchronize()
    sib_t1_us = e0.elapsed_time(e1) / reps * 1000.0
    return {"width": W_tree, "levels": a_tree, "nodes": Mt, "fuse_us": round(tacc[0], 1),
            "pdm_us": round(tacc[1], 1), "draft_head_top4_x4rows_us": round(tacc[2], 1),
            "verify_siblings_us": round(tacc[3], 1), "step_us": round(float(tacc.sum()), 1),
            "verify_siblings_t1_all_rejected_us": round(sib_t1_us, 1),
            "note": "calls in sequence, each timed alone (the chain cycle's calls: see calls)"}



if __name__ == "__main__":
    main()
