#!/usr/bin/env python3
"""Bench of the fused KV-cache step (one MI355X).

A step is one pass of the whole hot path over one batch: gather X[Q] + QKV
projection + rotary + in-place k/v write (first launch), then split-N
attention over the whole cache with the view mask and the split combine
(second launch).  Inputs are seeded synthetic tensors shaped like the layer
workloads (io_aware_kv_amd.workloads) and already resident in HBM.  Several
independent buffer sets (weights, hidden states, caches, outputs) are used
round robin so that no step finds its data in the 256 MB Infinity Cache.

Prints one JSON line.  `value` is the achieved HBM bandwidth of the whole
step counted in algorithmic bytes (weights once, the gathered X rows, the new
k/v rows, one full read of K and V, O and LSE) divided by the step time;
`roofline` is the dominant kernel's algorithmic bytes over its average
launch time (HIP events on the launch stream) against the 8 TB/s HBM peak;
`cpu_baseline` is the fp64 CPU oracle timed on the host on the same inputs.

  python bench.py [--steps K] [--warmup W] [--config 3] [--sets S] [--no-cpu]
  python bench.py --mode copy      # plain device copy, for counter calibration
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "fused-step latency (us) and achieved HBM GB/s vs peak, 8B-class layer, N=2048"
ATTN_SRC = os.path.join(ROOT, "io_aware_kv_amd", "csrc", "attn_mfma.hip")
PROJ_SRC = os.path.join(ROOT, "io_aware_kv_amd", "csrc", "proj_mfma.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def src_hash(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def algorithmic_bytes(wl):
    """Bytes the method must move per step: weights once, the gathered X
    rows, the new k/v rows (one per distinct position), one full K and V
    read, O and LSE, the mask and the index arrays."""
    ls = wl.shape
    elt = 2 if str(ls.dtype) == "torch.bfloat16" else 4
    B, N, d, H, Hkv, dh, nq = ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, wl.nq
    distinct = sum(len(set(wl.pos_ids[b].tolist())) for b in range(B))
    w = ls.cols * d * elt
    x = B * nq * d * elt
    kv_write = distinct * Hkv * dh * 2 * elt
    kv_read = B * Hkv * N * dh * 2 * elt
    out = B * nq * H * dh * elt + B * nq * H * 4
    mask = B * nq * nq if wl.vis is not None else 0
    idx = 2 * B * nq * 4
    proj = w + x + kv_write + idx
    attn = kv_read + out + mask + B * nq * 4
    return {"proj": proj, "attn": attn, "total": w + x + kv_write + kv_read + out + mask + idx,
            "qkv_flops": 2 * B * nq * d * ls.cols,
            "attn_flops": 4 * B * nq * H * N * dh}


def counters_traffic(kernel_keys, workload_key, src_path):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE scaled by the copy-kernel calibration), summed
    over the kernels of the phase, or None when there is none or the kernel
    source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            data = json.load(f)
        cal = data["calibration"]
        total = 0.0
        found = False
        for key in kernel_keys:
            ent = data["kernels"].get(key, {}).get(workload_key)
            if ent is None:
                continue
            if ent.get("src_hash") != src_hash(src_path):
                return None
            total += ent["fetch_kib"] * 1024 * cal["fetch_factor"] + ent["write_kib"] * 1024 * cal["write_factor"]
            found = True
        return int(total) if found else None
    except (KeyError, ValueError, TypeError):
        return None


def run_copy(args):
    import torch
    n = args.copy_bytes // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 10
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"mode": "copy", "bytes_read": n * 4, "bytes_written": n * 4,
                      "GBps": 2 * n * 4 / dt / 1e9}))


def host_info():
    """CPU model and thread count of the host the bench ran on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


def cpu_oracle_baseline(wl, K0, V0, budget_s):
    """Time the fp64 oracle (as it stands) on the host on the same inputs."""
    import oracle
    from oracle import Shape
    ls = wl.shape
    sh = Shape(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, ls.rope_base)
    rm = oracle.ROUND_BF16 if str(ls.dtype) == "torch.bfloat16" else oracle.ROUND_FP32
    Xh = oracle._f64(wl.X)
    Wh = oracle._f64(wl.W)
    K0h, V0h = oracle._f64(K0), oracle._f64(V0)
    times = []
    r = None
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        r = oracle.step(sh, Xh, wl.Q_idx, wl.pos_ids, wl.vis, Wh, K0h, V0h, rm)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 64:
            break
    return r, sorted(times)[len(times) // 2], len(times), oracle.threads()


def time_selection(fk, wl, sets, stream, iters):
    """Time the tracked-set scores and the top-k selection that follow the
    step (beta_t = 80), over the rotating buffer sets; the handle's q staging
    holds the last step's q, and every set carries the same step inputs."""
    import torch
    from io_aware_kv_amd.workloads import selection_inputs
    ls = wl.shape
    dev = torch.device("cuda")
    sel, cand = selection_inputs(wl)
    sel_d, cand_d = sel.to(dev), cand.to(dev)
    k = 80
    n = len(sets)
    scores = [torch.empty((ls.B, ls.N), dtype=torch.float32, device=dev) for _ in range(n)]
    outs = [torch.empty((ls.B, k), dtype=torch.int32, device=dev) for _ in range(n)]

    def run(i, evs=None):
        st = sets[i % n]
        if evs is not None:
            evs[0].record(stream)
        fk.tracked_scores(st["P"], st["vis"], sel_d, st["Kc"], st["LSE"], scores[i % n], stream=stream)
        if evs is not None:
            evs[1].record(stream)
        fk.select_tracked(scores[i % n], cand_d, k, outs[i % n], stream=stream)
        if evs is not None:
            evs[2].record(stream)

    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(iters)]
    for i in range(iters):
        run(i, evs[i])
    torch.cuda.synchronize()
    sc_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / iters
    tk_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / iters
    elt = 2 if ls.dtype == torch.bfloat16 else 4
    G = ls.H // ls.Hkv
    nsel = int(sel.sum())
    # algorithmic bytes: the cache's K once, the selected rows' q and LSE,
    # the positions, mask and selection flags, the scores written
    nbytes = (ls.B * ls.Hkv * ls.N * ls.dh * elt + nsel * ls.H * ls.dh * 4 + nsel * ls.H * 4
              + ls.B * wl.nq * 5 + (ls.B * wl.nq * wl.nq if wl.vis is not None else 0) + ls.B * ls.N * 4)
    gbps = nbytes / (sc_ms * 1e-3) / 1e9
    return {"k": k, "rows_selected": nsel, "scores_us": round(sc_ms * 1e3, 3), "select_us": round(tk_ms * 1e3, 3),
            "scores_algorithmic_bytes": nbytes, "scores_GBps": round(gbps, 1),
            "scores_hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}


def time_decision(wl, stream, iters):
    """Time the draft-pass decisions for the step's masked rows over the
    synthetic vocabulary: per-row prediction and confidence with the eps
    split, then the sequential acceptance over the same rows."""
    import torch
    from io_aware_kv_amd import binding
    from io_aware_kv_amd.workloads import SYNTH_VOCAB, decision_logits, selection_inputs
    sel, _ = selection_inputs(wl)
    rows = max(1, int(sel.sum()))
    V = SYNTH_VOCAB
    dev = torch.device("cuda")
    host = decision_logits(rows, V, seed=wl.seed)
    bufs = [host.to(dev) for _ in range(2)]   # alternate, so no call finds its rows cached
    pred = torch.empty((rows,), dtype=torch.int32, device=dev)
    conf = torch.empty((rows,), dtype=torch.float32, device=dev)
    over = torch.empty((rows,), dtype=torch.uint8, device=dev)
    B = wl.shape.B
    S = max(1, rows // B)
    n_acc = torch.empty((B,), dtype=torch.int32, device=dev)

    def run(i, evs=None):
        if evs is not None:
            evs[0].record(stream)
        binding.confidence(bufs[i % 2], 126, 0.9, pred, conf, over, stream=stream)
        if evs is not None:
            evs[1].record(stream)
        binding.accept(pred[:B * S].view(B, S), pred[:B * S].view(B, S), conf[:B * S].view(B, S), 0.8, n_acc,
                       stream=stream)
        if evs is not None:
            evs[2].record(stream)

    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(iters)]
    for i in range(iters):
        run(i, evs[i])
    torch.cuda.synchronize()
    c_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / iters
    a_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / iters
    nbytes = rows * V * 2 + rows * 9
    gbps = nbytes / (c_ms * 1e-3) / 1e9
    return {"rows": rows, "vocab": V, "confidence_us": round(c_ms * 1e3, 3), "accept_us": round(a_ms * 1e3, 3),
            "confidence_algorithmic_bytes": nbytes, "confidence_GBps": round(gbps, 1),
            "confidence_hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}


def time_paged(fk, wl, stream, iters, n_sets, warmup, block_size=16):
    """Time the fused step over a paged cache (blocks of 16 positions in a
    seeded random order, full lengths and row counts), with the flat step's
    protocol: n_sets buffer sets in rotation (each its own X, W and pools),
    `warmup` untimed steps, then `iters` timed steps back to back."""
    import torch
    from io_aware_kv_amd.workloads import paged_layout
    ls = wl.shape
    dev = torch.device("cuda")
    table, Kpool, Vpool, L, nb = paged_layout(wl, block_size, ragged=False)
    sets = []
    for _ in range(n_sets):
        sets.append(dict(X=wl.X.to(dev), W=wl.W.to(dev), K=Kpool.to(dev), V=Vpool.to(dev),
                         O=torch.empty((ls.B, wl.nq, ls.H, ls.dh), dtype=ls.dtype, device=dev),
                         LSE=torch.empty((ls.B, wl.nq, ls.H), dtype=torch.float32, device=dev)))
    Q, P = wl.Q_idx.to(dev), wl.pos_ids.to(dev)
    vis = wl.vis.to(dev) if wl.vis is not None else None
    tab, Ld, nbd = table.to(dev), L.to(dev), nb.to(dev)

    def run(i):
        st = sets[i % n_sets]
        fk.step_paged(st["X"], Q, P, vis, st["W"], st["K"], st["V"], st["O"], st["LSE"], block_table=tab,
                      block_size=block_size, num_blocks=Kpool.shape[0], seq_len=Ld, nq_seq=nbd, stream=stream)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(iters):
        run(i)
    e1.record(stream)
    torch.cuda.synchronize()
    del sets
    return {"block_size": block_size, "step_us": round(e0.elapsed_time(e1) / iters * 1e3, 3)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--sets", type=int, default=0, help="buffer sets in rotation (0: auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-select", action="store_true",
                    help="skip timing the steps after the path (selection, decisions) and the paged variant")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--attn-splits", type=int, default=0)
    ap.add_argument("--gemm-splitk", type=int, default=0)
    ap.add_argument("--mode", default="step", choices=["step", "copy"])
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested; run with --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if args.mode == "copy":
        return run_copy(args)

    from io_aware_kv_amd.binding import FusedKVCache
    from io_aware_kv_amd.workloads import initial_cache, make_workload

    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    log("bench: config %d, generating inputs" % args.config)
    wl = make_workload(args.config)
    ls = wl.shape
    ab = algorithmic_bytes(wl)
    per_set = ab["total"] + ls.B * wl.x_rows * ls.d_model * (2 if ls.dtype == torch.bfloat16 else 4)
    n_sets = args.sets or max(3, -(-768 * 2 ** 20 // ab["total"]))

    K0, V0 = initial_cache(wl)
    sets = []
    fk = None
    for s in range(n_sets):
        X = wl.X.to(dev)
        W = wl.W.to(dev)
        Kc = torch.empty((ls.B, ls.Hkv, ls.N, ls.dh), dtype=ls.dtype, device=dev)
        Vc = torch.empty_like(Kc)
        if fk is None:
            fk = FusedKVCache(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, wl.nq, ls.dtype, ls.rope_base)
            if args.attn_splits or args.gemm_splitk:
                fk.set_tuning(attn_splits=args.attn_splits, gemm_splitk=args.gemm_splitk)
        Kc.copy_(K0)
        Vc.copy_(V0)
        O = torch.empty((ls.B, wl.nq, ls.H, ls.dh), dtype=ls.dtype, device=dev)
        LSE = torch.empty((ls.B, wl.nq, ls.H), dtype=torch.float32, device=dev)
        sets.append(dict(X=X, W=W, Kc=Kc, Vc=Vc, O=O, LSE=LSE, Q=wl.Q_idx.to(dev), P=wl.pos_ids.to(dev),
                         vis=wl.vis.to(dev) if wl.vis is not None else None))
    torch.cuda.synchronize()
    plan = fk.plan(wl.nq)
    log("bench: %d buffer sets of %.1f MB, plan %s" % (n_sets, per_set / 1e6, plan))

    stream = torch.cuda.current_stream()

    def step(st, evs=None):
        if evs is not None:
            evs[0].record(stream)
        fk.project(st["X"], st["Q"], st["P"], st["W"], st["Kc"], st["Vc"], stream=stream)
        if evs is not None:
            evs[1].record(stream)
        fk.attend(st["P"], st["vis"], st["Kc"], st["Vc"], st["O"], st["LSE"], stream=stream)
        if evs is not None:
            evs[2].record(stream)

    for i in range(args.warmup):
        step(sets[i % n_sets])
    torch.cuda.synchronize()
    log("bench: warmup done, timing %d steps" % args.steps)

    # the timed steps run back to back with nothing between the launches
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(sets[i % n_sets])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = start.elapsed_time(end) / args.steps
    # phase times from a second pass with an event around each launch (the
    # events add a small gap between the launches, so they stay out of the
    # timed steps above)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(sets[i % n_sets], evs[i])
    torch.cuda.synchronize()
    proj_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    attn_ms = sorted(e[1].elapsed_time(e[2]) for e in evs)
    proj_avg = sum(proj_ms) / len(proj_ms)
    attn_avg = sum(attn_ms) / len(attn_ms)
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in evs)

    def pct(v):
        n = len(v)
        return {"p10": round(v[n // 10] * 1e3, 3), "p50": round(v[n // 2] * 1e3, 3),
                "p90": round(v[min(n - 1, (n * 9) // 10)] * 1e3, 3)}

    # the device's achievable streaming rate beside the 8 TB/s spec: a plain
    # 1 GiB device copy on the same stream (bytes read + written per second)
    cx = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cy = torch.empty_like(cx)
    for _ in range(3):
        cy.copy_(cx)
    ce0, ce1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ce0.record(stream)
    for _ in range(10):
        cy.copy_(cx)
    ce1.record(stream)
    torch.cuda.synchronize()
    copy_GBps = 2 * cx.numel() * 4 / (ce0.elapsed_time(ce1) / 10 * 1e-3) / 1e9
    del cx, cy
    log("bench: %.2f us/step (proj %.2f us, attn %.2f us), wall %.3f s" %
        (ms_per_step * 1e3, proj_avg * 1e3, attn_avg * 1e3, wall))

    # warm-cache reference: the same set every step (Infinity Cache may hold it)
    warm_iters = min(args.steps, 50)
    torch.cuda.synchronize()
    ws, we = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ws.record(stream)
    for _ in range(warm_iters):
        step(sets[0])
    we.record(stream)
    torch.cuda.synchronize()
    warm_ms = ws.elapsed_time(we) / warm_iters

    # the step after the path: tracked-set scores and top-k (not part of value)
    selection = None
    if not args.no_select:
        selection = time_selection(fk, wl, sets, stream, min(args.steps, 50))
        log("bench: tracked-set scores %.2f us, top-k %.2f us" % (selection["scores_us"], selection["select_us"]))
        decision = time_decision(wl, stream, min(args.steps, 50))
        log("bench: decisions over %d rows x %d ids: %.2f us (%.0f GB/s), acceptance %.2f us" %
            (decision["rows"], decision["vocab"], decision["confidence_us"], decision["confidence_GBps"],
             decision["accept_us"]))
        selection["decision"] = decision
        paged = time_paged(fk, wl, stream, args.steps, n_sets, args.warmup)
        log("bench: paged cache (blocks of %d) step %.2f us" % (paged["block_size"], paged["step_us"]))
        selection["paged_step"] = paged

    # dominant kernel roofline
    dom = "attn" if attn_avg >= proj_avg else "proj"
    dom_ms = attn_avg if dom == "attn" else proj_avg
    dom_bytes = ab[dom]
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    wkey = "workload%d" % args.config
    # the attention phase is the split kernel plus, with several cache splits,
    # its combine kernel (same stream, back to back)
    if dom == "attn":
        keys = ["attn_mfma", "attn_combine"] if plan["attn_splits"] > 1 else ["attn_mfma"]
    else:
        keys = ["proj_mfma"]
    traffic = counters_traffic(keys, wkey, ATTN_SRC if dom == "attn" else PROJ_SRC)
    # the bound is whichever of its algorithmic bytes and algorithmic flops
    # takes the longer at peak (a projection over many query rows is a
    # contraction well past the ridge point)
    dom_flops = ab["attn_flops"] if dom == "attn" else ab["qkv_flops"]
    mfma_bound = dom_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > dom_bytes / (HBM_PEAK_GBPS * 1e9)
    if mfma_bound:
        achieved_f = dom_flops / (dom_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved_f, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved_f / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(achieved / HBM_PEAK_GBPS, 4)}
    roofline.update({"traffic": traffic,
                     "kernel": "attn_mfma_kernel" if dom == "attn" else "proj_mfma_kernel",
                     "algorithmic_bytes_per_launch": dom_bytes, "algorithmic_flops_per_launch": dom_flops,
                     "avg_launch_us": round(dom_ms * 1e3, 3)})

    value = ab["total"] / (ms_per_step * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if ls.dtype == torch.bfloat16 else "f32",
        "data": "synthetic (seeded; no model weights or datasets)",
        "config": {"workload": wl.name, "B": ls.B, "N": ls.N, "d_model": ls.d_model, "H": ls.H,
                   "Hkv": ls.Hkv, "dh": ls.dh, "nq": wl.nq, "view_mask": wl.vis is not None,
                   "buffer_sets": n_sets, "plan": plan},
        "latency_us": round(ms_per_step * 1e3, 3),
        "queries_per_s": round(ls.B * wl.nq / (ms_per_step * 1e-3), 1),
        "warm_cache_latency_us": round(warm_ms * 1e3, 3),
        "phases": {
            "proj_us": round(proj_avg * 1e3, 3),
            "attn_us": round(attn_avg * 1e3, 3),
            "proj_GBps": round(ab["proj"] / (proj_avg * 1e-3) / 1e9, 1),
            "attn_GBps": round(ab["attn"] / (attn_avg * 1e-3) / 1e9, 1),
            "proj_mfma_frac": round(ab["qkv_flops"] / (proj_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "attn_hbm_frac": round(ab["attn"] / (attn_avg * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            # distribution over the evented pass (an event around each launch)
            "proj_us_pct": pct(proj_ms),
            "attn_us_pct": pct(attn_ms),
            "step_us_pct": pct(step_ms),
        },
        "algorithmic_bytes_per_step": ab["total"],
        "device_copy_GBps": round(copy_GBps, 1),
        "host": host_info(),
        "next_rows": selection,
        "roofline": roofline,
        "cpu_baseline": None,
    }

    if not args.no_cpu:
        log("bench: timing the CPU oracle (budget %.0f s)" % args.cpu_budget)
        r, cpu_s, reps, threads = cpu_oracle_baseline(wl, K0, V0, args.cpu_budget)
        result["cpu_baseline"] = {"value": round(ab["total"] / cpu_s / 1e9, 4), "unit": "GB/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": "the full step of this workload (all %d sequences), "
                                            "median of %d run(s), %.2f s" % (ls.B, reps, cpu_s)}
        # parity of the timed path against the oracle on set 0
        import numpy as np
        o = sets[0]["O"].double().cpu().numpy()
        lse = sets[0]["LSE"].double().cpu().numpy()
        fin = np.isfinite(r["LSE"])
        result["parity"] = {
            "O_rel": float(np.abs(o - r["O"]).max() / np.abs(r["O"]).max()),
            "LSE_abs": float(np.abs(lse[fin] - r["LSE"][fin]).max()),
        }
        log("bench: cpu oracle %.2f s/step on %d threads; parity %s" % (cpu_s, threads, result["parity"]))

    print(json.dumps(result))


if __name__ == "__main__":
    main()
