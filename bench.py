"""Benchmark of the W4A16 MoE layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--also NAME,...]

A step is one pass of the whole hot path over one synthetic batch: for the
indexed layout routing alignment (chord_moe_align) and the layer (tile build,
gate_up GEMM + SiLU*mul, down GEMM, weighted combine), or, where the planner
routes the call inside the gate_up launch (block_m 0: a few thousand slots on
the weight-streaming kernels), the layer alone, whose gate_up derives the
per-expert rows from topk_ids itself; the layer alone for the grouped layouts
(their row maps are the dispatcher's output).  Inputs are
resident in HBM before the timed region.  Weight replicas are rotated across
steps so that every step streams its weights from HBM, not from the 256 MB
Infinity Cache.  Before the W warm-up steps, untimed steps run for at least
--prewarm-ms (default 300 ms): the GPU raises its clocks over tens of
milliseconds of sustained work, so without it the timed steps would measure
the ramp (decode: about 221 instead of 193 us per call), not the steady state
of a busy serving loop.

Prints ONE JSON line (rank 0) for --workload (default: the decode EP share).
`roofline` reports the dominant kernel (the slower of the two GEMMs) against
HBM (8 TB/s) or dense BF16 MFMA (2.5 PFLOP/s), whichever bound the workload's
arithmetic intensity selects, from its algorithmic bytes / FLOPs and its
average duration, measured with HIP events recorded by the library on the
launch stream over a second pass of the same K steps (event records between
kernels would add microseconds to the timed pass itself); `detail` carries
the other fraction of the same kernel too.  Each workload named by --also
(default: the indexed prefill EP share) is measured the same way and reported
under `detail.also`.  `cpu_baseline` times the CPU oracle on a bounded sample
of the main workload.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("W4A16 MoE layer µs/call + achieved HBM TB/s (decode) / MFMA TFLOPS (prefill)")
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
W_BYTES = 0.5625          # one packed nibble + a bf16 scale per 32 weights
DEFAULT_WORKLOAD = "kimi_decode_T64_ep48of384_top8"
DEFAULT_ALSO = "kimi_prefill_T8192_ep48of384_top8"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--also", default=DEFAULT_ALSO,
                    help="comma-separated workloads measured after the main one and reported "
                         "under detail.also ('' or 'none': no others)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=20.0,
                    help="seconds of oracle work (whole experts are run until it is spent)")
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="untimed steps for at least this long before the warm-up steps: the "
                         "GPU's clocks ramp up over tens of ms of sustained work, and the timed "
                         "steps should see the steady state a serving loop runs in")
    ap.add_argument("--copy-probe", type=float, default=0.0, metavar="MIB",
                    help="instead of the layer, run `steps` plain device copies of MIB MiB "
                         "(calibrates rocprofv3 FETCH_SIZE / WRITE_SIZE against known bytes)")
    return ap.parse_args()


def measured_traffic(workload, stage):
    """HBM bytes per launch of `stage` on `workload` from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (profiles/traffic.json, already
    scaled by the copy-kernel calibration), or None when there is none or the
    kernel's source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles", "traffic.json")
    try:
        with open(path) as f:
            entries = json.load(f)["entries"]
    except (OSError, ValueError, KeyError):
        return None
    for e in entries:
        if e.get("workload") != workload or e.get("kernel") != stage:
            continue
        src = os.path.join(os.path.dirname(os.path.abspath(__file__)), e["source"])
        try:
            with open(src, "rb") as f:
                digest = hashlib.sha256(f.read()).hexdigest()[:16]
        except OSError:
            return None
        return int(e["bytes"]) if digest == e.get("source_sha256_16") else None
    return None


def copy_probe(mib, steps):
    import torch
    n = int(mib * 2**20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_probe_bytes": n, "steps": steps, "read_GBs": round(n / dt / 1e9, 1)}),
          flush=True)


# ---------------------------------------------------------------------------
# algorithmic work of one call (from the actual routing draw)
# ---------------------------------------------------------------------------

def algorithmic_work(wl):
    """Per-stage algorithmic HBM bytes and FLOPs of one layer call.

    Weights: each active expert's packed codes and scales read once
    (0.5625 B/weight).  gate_up also reads each routed token row once (for the
    indexed layout: each token with a local slot) and writes h (2 B x I per
    routed row); down reads h and writes y / output rows (2 B x H per routed
    row).  FLOPs count valid rows only: 2*R*H*2I (gate_up) + 2*R*I*H (down).
    """
    H, I = wl.H, wl.I
    if wl.layout == "masked":
        counts = np.asarray(wl.masked_m, dtype=np.int64)
        R = int(counts.sum())
        T_u = R
    else:
        ids = wl.topk_ids - wl.expert_begin
        local = (ids >= 0) & (ids < wl.E_l)
        counts = np.bincount(ids[local], minlength=wl.E_l)
        R = int(local.sum())
        T_u = int(np.any(local, axis=1).sum())
    active = int((counts > 0).sum())
    w13 = active * 2 * I * H * W_BYTES
    w2 = active * H * I * W_BYTES
    gu_bytes = w13 + 2 * H * T_u + 2 * I * R
    dn_bytes = w2 + 2 * I * R + 2 * H * R
    gu_flops = 2.0 * R * H * 2 * I
    dn_flops = 2.0 * R * I * H
    return dict(R=R, T_u=T_u, active=active, gate_up_bytes=gu_bytes, down_bytes=dn_bytes,
                gate_up_flops=gu_flops, down_flops=dn_flops,
                layer_bytes=w13 + w2 + 2 * H * T_u + 4 * I * R + 2 * H * (wl.T or R),
                layer_flops=gu_flops + dn_flops)


# ---------------------------------------------------------------------------
# the same step replayed from a HIP graph (launch-latency-bound small shapes)
# ---------------------------------------------------------------------------

def graph_replay_us(step, n_rep, steps, prewarm_ms):
    """Captures one call per weight replica (alignment + layer, the timed step)
    into a HIP graph and returns the average time per call over `steps`
    replays, bracketed by HIP events on the capturing stream.  The layer's
    default path enqueues no memset, no allocation and no host sync, so it is
    capturable as is.  Capture leaves the GPU idle for tens of milliseconds,
    long enough for its clocks to fall, so the graph is replayed untimed for
    `prewarm_ms` first, as the eager steps are."""
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n_rep):       # plans and workspaces exist before capture
            step(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(n_rep):
            step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < prewarm_ms:
        for _ in range(8):
            g.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return round(e0.elapsed_time(e1) * 1e3 / (steps * n_rep), 2)


# ---------------------------------------------------------------------------
# the steps either side of the grouped layer: dispatch and combine
# ---------------------------------------------------------------------------

def grouped_io(C, wl, rows, steps, dev, d, dbf):
    """Average launch-stream time of the dispatch into both grouped layouts
    (alignment included) and of the standalone combine, on the workload's
    routing, with their algorithmic HBM bytes: each routed row read and
    written once (2*H bytes each way; padding rows of the contiguous layout
    are written), the routing ids read and the slot map written (4 B per
    slot each); the combine reads each routed row and writes each token row."""
    import torch
    x, ids, w = dbf(wl.x), d(wl.topk_ids), d(wl.topk_weights)
    T, k, H, E_l, eb = wl.T, wl.k, wl.H, wl.E_l, wl.expert_begin
    flat = wl.topk_ids.reshape(-1) - eb
    local = (flat >= 0) & (flat < E_l)
    R = int(local.sum())
    counts = np.bincount(flat[local], minlength=E_l)
    padded = int((-(-counts // 128) * 128).sum())
    max_rows = C.chord_moe_dispatch_contiguous_rows(T, k, E_l)
    max_m = 256

    ca = (torch.empty((max_rows, H), dtype=torch.bfloat16, device=dev),
          torch.empty(max_rows, dtype=torch.int32, device=dev),
          torch.empty(T * k, dtype=torch.int32, device=dev),
          torch.empty(1, dtype=torch.int32, device=dev))
    cws = torch.empty(C.chord_moe_dispatch_workspace_bytes(C.MODE_CONTIGUOUS, T, k, E_l),
                      dtype=torch.uint8, device=dev)
    ma = (torch.empty((E_l, max_m, H), dtype=torch.bfloat16, device=dev),
          torch.empty(E_l, dtype=torch.int32, device=dev),
          torch.empty(T * k, dtype=torch.int32, device=dev),
          torch.empty(1, dtype=torch.int32, device=dev))
    mws = torch.empty(C.chord_moe_dispatch_workspace_bytes(C.MODE_MASKED, T, k, E_l),
                      dtype=torch.uint8, device=dev)
    tok = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    C.chord_moe_dispatch_contiguous(x, ids, eb, E_l, max_rows, out=ca, workspace=cws)
    torch.cuda.synchronize()
    f2r = ca[2].clone()
    kept = int(np.minimum(counts, max_m).sum())
    calls = {
        "dispatch_contiguous": (
            lambda: C.chord_moe_dispatch_contiguous(x, ids, eb, E_l, max_rows, out=ca,
                                                    workspace=cws),
            2 * H * R + 2 * H * padded + 8 * T * k),
        "dispatch_masked_maxm256": (
            lambda: C.chord_moe_dispatch_masked(x, ids, eb, E_l, max_m, out=ma, workspace=mws),
            4 * H * kept + 8 * T * k),
        "combine": (lambda: C.chord_moe_combine(rows, f2r, w, out=tok),
                    2 * H * R + 2 * H * T + 8 * T * k),
    }
    res = {}
    for name, (fn, nbytes) in calls.items():
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / steps
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"us": round(us, 2), "algorithmic_bytes": int(nbytes),
                     "GB/s": round(gbs, 1), "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)}
    res["routed_rows"] = R
    return res


# ---------------------------------------------------------------------------
# CPU oracle baseline (bounded sample)
# ---------------------------------------------------------------------------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s):
    """The CPU oracle on whole experts of the workload, each dequantised once
    with all of its routed rows, until `budget_s` is spent; the time scales to
    the call by active experts (the oracle's work per expert is dominated by
    the dequantisation of its weights, which does not depend on its row
    count), and the combine over the sampled slots is timed with it."""
    import oracle
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        blas = None
    if wl.layout == "masked":
        rows_of = {e: np.arange(int(wl.masked_m[e])) for e in range(wl.E_l) if wl.masked_m[e] > 0}
    else:
        flat = wl.topk_ids.reshape(-1).astype(np.int64) - wl.expert_begin
        rows_of = {e: np.nonzero(flat == e)[0] for e in range(wl.E_l) if np.any(flat == e)}
    order = list(np.random.default_rng(0).permutation(sorted(rows_of)))
    x = None if wl.layout == "masked" else oracle.bf16_to_f64(wl.x)
    ys, done, t0 = {}, 0, time.perf_counter()
    for e in order:
        w13 = oracle.dequant_f64(wl.q13[e], wl.s13[e])
        w2 = oracle.dequant_f64(wl.q2[e], wl.s2[e])
        if wl.layout == "masked":
            xr = oracle.bf16_to_f64(wl.a3[e, :len(rows_of[e])])
        else:
            xr = x[rows_of[e] // wl.k]
        y = oracle.expert_mlp(xr, w13, w2)
        if wl.layout != "masked":
            for r, i in enumerate(rows_of[e].tolist()):
                ys[(i // wl.k, i % wl.k)] = y[r]
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    if wl.layout != "masked":
        toks = sorted({t for t, _ in ys})
        sub_ids = np.full_like(wl.topk_ids, -1)          # only the sampled slots are local
        for t, j in ys:
            sub_ids[t, j] = wl.topk_ids[t, j]
        oracle.combine(ys, sub_ids, wl.topk_weights, wl.expert_begin, wl.E_l, wl.H, toks)
    el = time.perf_counter() - t0
    n_active = len(rows_of)
    sample = (f"oracle (fp64 NumPy) on {done} of {n_active} active experts, each dequantised once "
              f"with all its routed rows" + ("" if wl.layout == "masked" else ", plus the combine "
              "of the sampled slots") + (f"; scaled by experts ({n_active}/{done})"
                                         if done < n_active else "; the whole call"))
    return {"value": round(el * n_active / max(done, 1) * 1e6, 1), "unit": "us/call",
            "cores": cores, "kind": "oracle", "sample": sample, "measured_s": round(el, 3),
            "cpu_model": cpu_model(), "blas_threads": blas}


# ---------------------------------------------------------------------------
# one workload: build, time, kernel-time, roofline
# ---------------------------------------------------------------------------

def measure(spec, args, C, dev, with_graph=False, grouped=False):
    """Times `args.steps` steps of `spec` (after the clock pre-warm and
    `args.warmup` untimed steps) and the per-stage kernel durations of a
    second pass; returns (config, result dict, workload)."""
    import torch
    from moe_inputs import gen as G
    from quantized_moe_amd.moe import W4A16MoE

    wl = G.make_workload(spec)

    def d(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def dbf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)

    mode = {"indexed": C.MODE_INDEXED, "contiguous": C.MODE_CONTIGUOUS,
            "masked": C.MODE_MASKED}[wl.layout]
    weight_bytes = (wl.q13.nbytes + wl.q2.nbytes) * 9 // 8
    n_rep = 2 if weight_bytes > 300e6 else int(math.ceil(600e6 / weight_bytes)) + 1
    q13, s13, q2, s2 = d(wl.q13), dbf(wl.s13), d(wl.q2), dbf(wl.s2)
    layers = [W4A16MoE(q13, s13, q2, s2, mode=mode) for _ in range(n_rep)]
    del q13, s13, q2, s2
    torch.cuda.synchronize()

    out_rows = None
    if wl.layout == "indexed":
        x, ids, w = dbf(wl.x), d(wl.topk_ids), d(wl.topk_weights)
        # block_m 0: the planner routes the call inside the gate_up launch
        # (rows from topk_ids), so the step has no alignment launch.
        bm = C.chord_w4a16_moe_indexed_block_m(wl.T, wl.k, wl.E_g, wl.E_l, wl.H, wl.I)
        mp = C.chord_moe_align_max_padded(wl.T, wl.k, wl.E_l, bm) if bm else 0
        out = torch.empty((wl.T, wl.H), dtype=torch.bfloat16, device=dev)
        for L in layers:
            L.workspace(C.chord_w4a16_moe_workspace_bytes(C.MODE_INDEXED, wl.T, wl.k, wl.E_l, wl.H,
                                                          wl.I, mp), dev)
        if bm:
            al_out = (torch.empty(mp, dtype=torch.int32, device=dev),
                      torch.empty((mp + bm - 1) // bm, dtype=torch.int32, device=dev),
                      torch.empty(1, dtype=torch.int32, device=dev))
            al_ws = torch.empty(max(1, C.lib.chord_moe_align_workspace_bytes(wl.T, wl.k, wl.E_l,
                                                                             bm)),
                                dtype=torch.uint8, device=dev)

            def step(i):
                L = layers[i % n_rep]
                C.chord_moe_align(ids, wl.expert_begin, wl.E_l, bm, max_padded=mp, out=al_out,
                                  workspace=al_ws)
                L.indexed(x, ids, w, wl.expert_begin, wl.E_g, align=(*al_out, bm), out=out)
        else:
            def step(i):
                layers[i % n_rep].indexed(x, ids, w, wl.expert_begin, wl.E_g, block_m=0, out=out)
        config = {"workload": spec.name, "layout": "indexed", "T": wl.T, "H": wl.H, "I": wl.I,
                  "E_global": wl.E_g, "E_local": wl.E_l, "top_k": wl.k, "block_m": bm}
    elif wl.layout == "contiguous":
        a, m_idx, f2r, nvalid = G.build_contiguous(wl.topk_ids, wl.x, wl.expert_begin, wl.E_l)
        a_d, m_d = dbf(a), d(m_idx)
        out_rows = torch.empty((a.shape[0], wl.H), dtype=torch.bfloat16, device=dev)

        def step(i):
            layers[i % n_rep].contiguous(a_d, m_d, nvalid, out_rows=out_rows)
        config = {"workload": spec.name, "layout": "contiguous", "T": wl.T, "M": int(a.shape[0]),
                  "H": wl.H, "I": wl.I, "E_local": wl.E_l, "top_k": wl.k}
    else:
        a3, mm = dbf(wl.a3), d(wl.masked_m)
        out = torch.empty((wl.E_l * wl.max_m, wl.H), dtype=torch.bfloat16, device=dev)

        def step(i):
            layers[i % n_rep].masked(a3, mm, wl.expected_m, out=out)
        config = {"workload": spec.name, "layout": "masked", "E_local": wl.E_l, "max_m": wl.max_m,
                  "H": wl.H, "I": wl.I, "expected_m": wl.expected_m,
                  "rows": int(wl.masked_m.sum())}

    # Clock pre-warm (untimed), then the W warm-up steps (untimed).
    prewarm_steps = 0
    t_pre = time.perf_counter()
    while (time.perf_counter() - t_pre) * 1e3 < args.prewarm_ms:
        for _ in range(8):
            step(prewarm_steps)
            prewarm_steps += 1
        torch.cuda.synchronize()
    prewarm_ms = (time.perf_counter() - t_pre) * 1e3
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    plan = C.last_plan()

    # Timed region: exactly K steps between two synchronisations.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # Kernel timing: the same K steps again with the library recording HIP
    # events on the launch stream around each kernel stage (kept out of the
    # timed region above because each event record adds a few microseconds).
    C.chord_profile_reset()
    C.chord_profile_enable(True)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    C.chord_profile_enable(False)
    stage_ms, calls = C.chord_profile_read()

    ms_per_step = elapsed * 1e3 / args.steps
    work = algorithmic_work(wl)
    avg = [m / max(calls, 1) for m in stage_ms]           # ms per call per stage
    name = "down" if avg[2] > avg[1] else "gate_up"
    dur = avg[2] if name == "down" else avg[1]
    alg_b, alg_f = work[f"{name}_bytes"], work[f"{name}_flops"]
    gbs = alg_b / (dur * 1e-3) / 1e9
    tfs = alg_f / (dur * 1e-3) / 1e12
    hbm = {"bound": "hbm", "kernel": name, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
           "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
           "traffic": measured_traffic(spec.name, name), "algorithmic_bytes": int(alg_b),
           "avg_ms": round(dur, 5)}
    mfma = {"bound": "mfma", "kernel": name, "achieved": round(tfs, 1), "peak": BF16_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tfs / BF16_PEAK_TFLOPS, 4),
            "traffic": hbm["traffic"], "algorithmic_flops": alg_f, "avg_ms": round(dur, 5)}
    # The bound the layer's arithmetic intensity selects (HBM below the
    # 312 FLOP/B balance point of 2.5 PFLOP/s over 8 TB/s).
    hbm_bound = work["layer_flops"] / max(work["layer_bytes"], 1) < 2.5e15 / 8e12
    roof, other = (hbm, mfma) if hbm_bound else (mfma, hbm)
    layer_gbs = work["layer_bytes"] / (ms_per_step * 1e-3) / 1e9
    layer_tfs = work["layer_flops"] / (ms_per_step * 1e-3) / 1e12
    res = {"us_per_call": round(ms_per_step * 1e3, 2), "ms_per_step": round(ms_per_step, 5),
           "roofline": roof, "roofline_other": {k: other[k] for k in
                                                ("bound", "kernel", "achieved", "unit", "frac")},
           "stage_ms": [round(m, 5) for m in avg], "layer_kernels_ms": round(sum(avg), 5),
           "layer_algorithmic_bytes": int(work["layer_bytes"]),
           "layer_algorithmic_flops": work["layer_flops"],
           "layer_hbm_GBs": round(layer_gbs, 1), "layer_hbm_frac": round(layer_gbs / HBM_PEAK_GBS, 4),
           "layer_TFLOPs": round(layer_tfs, 2),
           "layer_mfma_frac": round(layer_tfs / BF16_PEAK_TFLOPS, 4),
           "routed_rows": work["R"], "active_experts": work["active"], "plan": plan,
           "weight_replicas": n_rep,
           "prewarm": {"ms": round(prewarm_ms, 1), "steps": prewarm_steps}}
    if grouped and wl.layout == "contiguous":
        res["grouped_io"] = grouped_io(C, wl, out_rows, args.steps, dev, d, dbf)
    if with_graph and wl.layout == "indexed" and wl.T <= 64:
        res["graph_us_per_call"] = graph_replay_us(step, n_rep, args.steps, args.prewarm_ms)
    del layers, step
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return config, res, wl


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.copy_probe > 0:
        copy_probe(args.copy_probe, args.steps)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus N>1 is not supported "
                                   "(the layer takes one GPU's expert share, no collectives)"}))
        sys.exit(2)
    import torch
    from moe_inputs.configs import workload_by_name
    from quantized_moe_amd import chord as C

    dev = torch.device("cuda:0")
    spec = workload_by_name(args.workload)
    config, res, wl = measure(spec, args, C, dev, with_graph=True, grouped=True)

    also = {}
    for name in [n for n in args.also.split(",") if n and n != "none" and n != args.workload]:
        _, r, _ = measure(workload_by_name(name), args, C, dev)
        also[name] = r

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, args.cpu_budget)

    detail = {k: v for k, v in res.items() if k not in ("us_per_call", "ms_per_step", "roofline")}
    if also:
        detail["also"] = also
    line = {"metric": METRIC, "value": res["us_per_call"], "unit": "us/call",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": res["ms_per_step"], "higher_is_better": False, "scaling": "weak",
            "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": config, "roofline": res["roofline"], "cpu_baseline": cpu, "detail": detail}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
