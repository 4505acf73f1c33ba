#!/usr/bin/env python3
"""Bench of the fused KV-cache step (one MI355X).

A step is one pass of the whole hot path over one batch through the
library's step entry point (fdllm_fused_step): gather X[Q] + QKV projection +
rotary + in-place k/v write (first launch), then split-N attention over the
whole cache with the view mask and the split combine (second launch).  The
phase figures time the two launches through the step's halves
(fdllm_step_project, fdllm_step_attend).  Inputs are seeded synthetic
tensors shaped like the layer workloads (io_aware_kv_amd.workloads) and
already resident in HBM.  Several
independent buffer sets (weights, hidden states, caches, outputs) are used
round robin so that no step finds its data in the 256 MB Infinity Cache.

Prints one JSON line.  `value` is the achieved HBM bandwidth of the whole
step counted in algorithmic bytes (weights once, the gathered X rows, the new
k/v rows, one full read of K and V, O and LSE) divided by the step time;
`roofline` is the dominant kernel's algorithmic bytes (or flops, past the
ridge point) over its average launch time (HIP events around that launch kind
alone, back to back on the launch stream) against the 8 TB/s HBM peak (or
2.5 PFLOP/s bf16); `configs` carries the same step and phase figures for the
other layer workloads of the target set;
`cpu_baseline` is the fp64 CPU oracle timed on the host on the same inputs.

  python bench.py [--steps K] [--warmup W] [--config 3] [--sets S] [--no-cpu]
                  [--other-configs 1,2,4]
  python bench.py --mode copy      # plain device copy, for counter calibration
  python bench.py --mode stream    # the device's streaming read and copy rates
  python bench.py --mode stack --steps 5 --warmup 1   # the large-batch workload's 32-layer stack
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
    step (beta_t = 80), over the rotating buffer sets, each call repeated back
    to back on the stream; the handle's q staging holds the last step's q, and
    every set carries the same step inputs."""
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

    def scores_call(i):
        st = sets[i % n]
        fk.tracked_scores(st["P"], st["vis"], sel_d, st["Kc"], st["LSE"], scores[i % n], stream=stream)

    def select_call(i):
        fk.select_tracked(scores[i % n], cand_d, k, outs[i % n], stream=stream)

    def timed(call):
        # back to back on the stream, one event pair around all the calls
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(iters):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    sc_ms = timed(scores_call)
    tk_ms = timed(select_call)
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
    split, then the sequential acceptance over the same rows, each call
    repeated back to back on the stream (the acceptance kernel is shorter
    than a host call, so its figure is the call rate)."""
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

    def conf_call(i):
        binding.confidence(bufs[i % 2], 126, 0.9, pred, conf, over, stream=stream)

    xs, cs = pred[:B * S].view(B, S), conf[:B * S].view(B, S)

    def accept_call(i):
        binding.accept(xs, xs, cs, 0.8, n_acc, stream=stream)

    def timed(call):
        # back to back on the stream, one event pair around all the calls
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(iters):
            call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters

    c_ms = timed(conf_call)
    a_ms = timed(accept_call)
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


def build_sets(wl, n_sets, dev, attn_splits=0, gemm_splitk=0, proj_tile=0):
    """The layer's handle and n_sets independent buffer sets (hidden states,
    weights, caches from the seeded initial cache, outputs, indices)."""
    import torch
    from io_aware_kv_amd.binding import FusedKVCache
    from io_aware_kv_amd.workloads import initial_cache
    ls = wl.shape
    K0, V0 = initial_cache(wl)
    fk = FusedKVCache(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, wl.nq, ls.dtype, ls.rope_base)
    if attn_splits or gemm_splitk or proj_tile:
        fk.set_tuning(attn_splits=attn_splits, gemm_splitk=gemm_splitk, proj_tile=proj_tile)
    sets = []
    for _ in range(n_sets):
        Kc = K0.to(dev).contiguous()
        Vc = V0.to(dev).contiguous()
        sets.append(dict(X=wl.X.to(dev), W=wl.W.to(dev), Kc=Kc, Vc=Vc,
                         O=torch.empty((ls.B, wl.nq, ls.H, ls.dh), dtype=ls.dtype, device=dev),
                         LSE=torch.empty((ls.B, wl.nq, ls.H), dtype=torch.float32, device=dev),
                         Q=wl.Q_idx.to(dev), P=wl.pos_ids.to(dev),
                         vis=wl.vis.to(dev) if wl.vis is not None else None))
    torch.cuda.synchronize()
    return fk, sets, K0, V0


def n_sets_for(ab):
    """Buffer sets in rotation: enough that no step finds its data in the
    256 MB Infinity Cache (at least 768 MB across the sets, at least 3; at
    most 12: a layer far smaller than the cache stays warm whatever the
    count)."""
    return min(12, max(3, -(-768 * 2 ** 20 // ab["total"])))


def time_launches(fn, sets, stream, steps, warmup):
    """Average time of fn(set) launched `steps` times back to back (sets in
    rotation), after `warmup` untimed calls: one event pair around the run."""
    import torch
    for i in range(warmup):
        fn(sets[i % len(sets)])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        fn(sets[i % len(sets)])
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_graph_steps(fk, sets, steps, warmup):
    """The step (projection + attention) captured once per buffer set into a
    HIP graph and replayed back to back over the sets: the device time per
    step without the host's launch calls between the kernels.  The library
    issues no memset and allocates nothing inside a step, so each graph holds
    only the step's kernel nodes."""
    import torch
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())

    def step(st):
        fk.step(st["X"], st["Q"], st["P"], st["vis"], st["W"], st["Kc"], st["Vc"], st["O"], st["LSE"], stream=cs)

    with torch.cuda.stream(cs):
        for st in sets:
            step(st)
    torch.cuda.synchronize()
    graphs = []
    for st in sets:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            step(st)
        graphs.append(g)
    torch.cuda.synchronize()
    with torch.cuda.stream(cs):
        for i in range(warmup):
            graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(cs)
        for i in range(steps):
            graphs[i % len(graphs)].replay()
        e1.record(cs)
        torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def phase_fraction(nbytes, flops, us):
    """Roofline fraction of a phase: against HBM bytes, or against bf16 MFMA
    flops when those take the longer at peak."""
    mfma = flops / (MFMA_BF16_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBPS * 1e9)
    if mfma:
        ach = flops / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "unit": "TFLOP/s",
                "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4)}
    ach = nbytes / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBPS, 4)}


def read_floor_us(nbytes, dev, stream, reps=20):
    """Time of one streaming read of nbytes with the library's read probe
    (best of four grid sizes), over rotating buffers (enough that a phase of
    more than 12 MB never finds its bytes in the 256 MB Infinity Cache):
    what this GPU needs to read a phase's bytes once, latency and ramp
    included."""
    import torch
    from io_aware_kv_amd import binding
    n16 = max(1, nbytes // 16)
    # (at most 64 buffers: a phase of a few MB stays in the caches whatever
    # the rotation, and its read is latency-bound anyway)
    nbuf = min(64, max(3, -(-768 * 2 ** 20 // (n16 * 16))))
    bufs = [torch.empty(n16 * 4, dtype=torch.int32, device=dev) for _ in range(nbuf)]
    for b in bufs:
        b.fill_(1)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    best = None
    for wgs in (256, 512, 1024, 2048):
        ms = time_launches(lambda buf: binding.probe_read(buf, sink, workgroups=wgs, stream=stream), bufs, stream,
                           max(reps, nbuf), 3)
        best = ms if best is None else min(best, ms)
    del bufs
    return best * 1e3


def measure_config(cid, steps, warmup, dev, read_GBps=None):
    """Step, projection and attention times of one layer workload, each launch
    kind timed alone back to back over rotating buffer sets, with the
    phases' roofline fractions."""
    import torch
    from io_aware_kv_amd.workloads import make_workload
    wl = make_workload(cid)
    ab = algorithmic_bytes(wl)
    n_sets = n_sets_for(ab)
    fk, sets, _, _ = build_sets(wl, n_sets, dev)
    stream = torch.cuda.current_stream()

    def proj(st):
        fk.project(st["X"], st["Q"], st["P"], st["W"], st["Kc"], st["Vc"], stream=stream)

    def attn(st):
        fk.attend(st["P"], st["vis"], st["Kc"], st["Vc"], st["O"], st["LSE"], stream=stream)

    def step(st):
        fk.step(st["X"], st["Q"], st["P"], st["vis"], st["W"], st["Kc"], st["Vc"], st["O"], st["LSE"], stream=stream)

    step_ms = time_launches(step, sets, stream, steps, warmup)
    proj_ms = time_launches(proj, sets, stream, steps, warmup)
    attn_ms = time_launches(attn, sets, stream, steps, warmup)
    graph_ms = time_graph_steps(fk, sets, steps, warmup)
    plan = fk.plan(wl.nq)
    fk.close()
    del sets
    attn_GBps = ab["attn"] / (attn_ms * 1e-3) / 1e9
    out = {"workload": wl.name, "plan": plan, "buffer_sets": n_sets,
           "step_us": round(step_ms * 1e3, 3), "graph_step_us": round(graph_ms * 1e3, 3),
           "proj_us": round(proj_ms * 1e3, 3), "attn_us": round(attn_ms * 1e3, 3),
           "proj_bytes": ab["proj"], "proj_flops": ab["qkv_flops"],
           "proj_roofline": phase_fraction(ab["proj"], ab["qkv_flops"], proj_ms * 1e3),
           "attn_bytes": ab["attn"], "attn_flops": ab["attn_flops"],
           "attn_GBps": round(attn_GBps, 1), "attn_hbm_frac": round(attn_GBps / HBM_PEAK_GBPS, 4)}
    if read_GBps:
        out["attn_frac_of_read_ceiling"] = round(attn_GBps / read_GBps, 4)
    floor = read_floor_us(ab["attn"], dev, stream)
    out["attn_read_floor_us"] = round(floor, 3)
    out["attn_frac_of_read_floor"] = round(floor / (attn_ms * 1e3), 4)
    return out


def device_rates(dev, stream):
    """The device's streaming rates beside the 8 TB/s spec, on the launch
    stream: a plain 1 GiB device copy (bytes read + written per second) and
    the library's read probe over 1 GiB (bytes read per second, the best of
    five grid sizes)."""
    import torch
    from io_aware_kv_amd import binding
    cx = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cy = torch.empty_like(cx)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(3):
        cy.copy_(cx)
        binding.probe_read(cx, sink, stream=stream)
    torch.cuda.synchronize()
    copy_ms = time_launches(lambda _: cy.copy_(cx), [None], stream, 10, 0)
    # the read probe's best grid (one to sixteen workgroups per CU)
    read_ms = min(time_launches(lambda _: binding.probe_read(cx, sink, workgroups=wgs, stream=stream), [None],
                                stream, 10, 2) for wgs in (256, 512, 1024, 2048, 4096))
    nbytes = cx.numel() * 4
    del cx, cy
    return 2 * nbytes / (copy_ms * 1e-3) / 1e9, nbytes / (read_ms * 1e-3) / 1e9


def run_stream(args):
    import torch
    torch.cuda.set_device(0)
    copy_GBps, read_GBps = device_rates(torch.device("cuda"), torch.cuda.current_stream())
    print(json.dumps({"mode": "stream", "bytes": 1 << 30, "read_GBps": round(read_GBps, 1),
                      "copy_GBps": round(copy_GBps, 1), "hbm_peak_GBps": HBM_PEAK_GBPS}))


def run_probes(args):
    """Device rates the step's kernels are bound by: streaming reads, the bf16
    MFMA issue rate (four and eight waves per CU), and LDS-DMA loads from an
    L2-resident 2 MB buffer with one to eight issuing waves per CU."""
    import torch
    from io_aware_kv_amd import binding
    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    copy_GBps, read_GBps = device_rates(dev, stream)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    wgs, iters = 256, 8192
    mfma = {}
    for waves in (4, 8):
        ms = time_launches(lambda _: binding.probe_mfma(sink, wgs, waves, iters, stream=stream), [None], stream, 5, 2)
        mfma["waves%d" % waves] = round(wgs * waves * iters * 8 * 16384 / (ms * 1e-3) / 1e12, 1)
    buf = torch.ones(2 << 20, dtype=torch.uint8, device=dev)
    dma = {}
    for waves in (1, 2, 4, 8):
        ms = time_launches(lambda _: binding.probe_lds_dma(buf, sink, wgs, waves, iters, stream=stream), [None],
                           stream, 5, 2)
        gbps = wgs * waves * iters * 1024 / (ms * 1e-3) / 1e9
        dma["waves%d" % waves] = {"GBps": round(gbps, 1), "per_cu_GBps": round(gbps / 256, 1)}
    print(json.dumps({"mode": "probes", "read_GBps": round(read_GBps, 1), "copy_GBps": round(copy_GBps, 1),
                      "mfma_bf16_TFLOPs": mfma, "mfma_bf16_peak_TFLOPs": MFMA_BF16_PEAK_TFLOPS,
                      "lds_dma_l2_resident": dma, "hbm_peak_GBps": HBM_PEAK_GBPS}))


def run_decisions(args):
    """The decision kernel over the synthetic vocabulary (131,072 seeded bf16
    logits per row) at several row counts: below the CU count each row is
    spread over id ranges, from 256 rows on every row has its own workgroup.
    Each count is timed over 50 calls back to back (two buffers alternated, so
    no call finds its rows cached); one JSON line with the per-count times and
    rates."""
    import torch
    from io_aware_kv_amd import binding
    from io_aware_kv_amd.workloads import SYNTH_VOCAB, decision_logits
    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    V = SYNTH_VOCAB
    res = {}
    for rows in (1, 8, 32, 64, 128, 256, 512, 1024):
        host = decision_logits(rows, V, seed=rows)
        bufs = [host.to(dev) for _ in range(2)]
        pred = torch.empty((rows,), dtype=torch.int32, device=dev)
        conf = torch.empty((rows,), dtype=torch.float32, device=dev)
        over = torch.empty((rows,), dtype=torch.uint8, device=dev)
        for i in range(3):
            binding.confidence(bufs[i % 2], 126, 0.9, pred, conf, over, stream=stream)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        iters = 50
        e0.record(stream)
        for i in range(iters):
            binding.confidence(bufs[i % 2], 126, 0.9, pred, conf, over, stream=stream)
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / iters * 1e3
        nbytes = rows * V * 2 + rows * 9
        res[str(rows)] = {"confidence_us": round(us, 3), "GBps": round(nbytes / (us * 1e-6) / 1e9, 1)}
        log("bench: decisions, %d rows: %.2f us (%.0f GB/s)" % (rows, us, nbytes / (us * 1e-6) / 1e9))
        del bufs
    print(json.dumps({"mode": "decisions", "vocab": V, "dtype": "bf16", "rows": res}))


def run_stack(args):
    """The large-batch workload as a whole stack: --layers consecutive layers
    (32 by default), each with its own weights and its own K/V cache in HBM,
    the same hidden states and query rows, one fused step per layer back to
    back.  Layer l's weights are drawn on the device from seed 20265 + 1000 l
    (N(0, 0.02^2), cast once to bf16); every layer's cache starts from the
    layer-0 seeded content (the step's timing does not depend on the values).
    Reports the stack's time, the time per layer and the algorithmic bytes of
    the stack over that time."""
    import torch
    from io_aware_kv_amd.binding import FusedKVCache
    from io_aware_kv_amd.workloads import initial_cache, make_workload
    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    stream = torch.cuda.current_stream()
    log("bench: stack of %d layers, generating inputs" % args.layers)
    wl = make_workload(5)
    ls = wl.shape
    ab = algorithmic_bytes(wl)
    K0, V0 = initial_cache(wl)
    X, Q, P = wl.X.to(dev), wl.Q_idx.to(dev), wl.pos_ids.to(dev)
    layers = []
    for l in range(args.layers):
        g = torch.Generator(device=dev).manual_seed(20265 + 1000 * l)
        W = (torch.randn(tuple(wl.W.shape), generator=g, device=dev) * 0.02).to(ls.dtype)
        layers.append(dict(W=W, Kc=K0.to(dev).contiguous(), Vc=V0.to(dev).contiguous(),
                           O=torch.empty((ls.B, wl.nq, ls.H, ls.dh), dtype=ls.dtype, device=dev),
                           LSE=torch.empty((ls.B, wl.nq, ls.H), dtype=torch.float32, device=dev)))
    fk = FusedKVCache(ls.B, ls.N, ls.d_model, ls.H, ls.Hkv, ls.dh, wl.nq, ls.dtype, ls.rope_base)
    torch.cuda.synchronize()
    hbm = sum(t.numel() * t.element_size() for st in layers for t in st.values()) + X.numel() * X.element_size()
    log("bench: %.1f GB of weights, caches and outputs in HBM" % (hbm / 1e9))

    def stack(_):
        for st in layers:
            fk.step(X, Q, P, None, st["W"], st["Kc"], st["Vc"], st["O"], st["LSE"], stream=stream)

    ms = time_launches(stack, [None], stream, args.steps, args.warmup)
    fk.close()
    total = ab["total"] * args.layers
    print(json.dumps({"mode": "stack", "workload": wl.name, "layers": args.layers, "steps": args.steps,
                      "stack_ms": round(ms, 4), "layer_us": round(ms * 1e3 / args.layers, 3),
                      "queries_per_s": round(ls.B * wl.nq / (ms * 1e-3), 1),
                      "algorithmic_bytes_per_stack": total, "GBps": round(total / (ms * 1e-3) / 1e9, 1),
                      "hbm_resident_GB": round(hbm / 1e9, 2)}))


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
    ap.add_argument("--other-configs", default="1,2,4",
                    help="other layer workloads measured into the line's `configs` (comma list; '' for none)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--attn-splits", type=int, default=0)
    ap.add_argument("--gemm-splitk", type=int, default=0)
    ap.add_argument("--proj-tile", type=int, default=0, help="projection tile choice override (0: the library's)")
    ap.add_argument("--mode", default="step", choices=["step", "copy", "stream", "probes", "stack", "decisions"])
    ap.add_argument("--layers", type=int, default=32, help="--mode stack: layers of the large-batch stack")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(--gpus %d requested; run with --gpus 1)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    if args.mode == "copy":
        return run_copy(args)
    if args.mode == "stream":
        return run_stream(args)
    if args.mode == "probes":
        return run_probes(args)
    if args.mode == "stack":
        return run_stack(args)
    if args.mode == "decisions":
        return run_decisions(args)

    from io_aware_kv_amd.workloads import make_workload

    torch.cuda.set_device(0)
    dev = torch.device("cuda")
    log("bench: config %d, generating inputs" % args.config)
    wl = make_workload(args.config)
    ls = wl.shape
    ab = algorithmic_bytes(wl)
    per_set = ab["total"] + ls.B * wl.x_rows * ls.d_model * (2 if ls.dtype == torch.bfloat16 else 4)
    n_sets = args.sets or n_sets_for(ab)
    fk, sets, K0, V0 = build_sets(wl, n_sets, dev, args.attn_splits, args.gemm_splitk, args.proj_tile)
    plan = fk.plan(wl.nq)
    log("bench: %d buffer sets of %.1f MB, plan %s" % (n_sets, per_set / 1e6, plan))

    stream = torch.cuda.current_stream()

    def proj(st):
        fk.project(st["X"], st["Q"], st["P"], st["W"], st["Kc"], st["Vc"], stream=stream)

    def attn(st):
        fk.attend(st["P"], st["vis"], st["Kc"], st["Vc"], st["O"], st["LSE"], stream=stream)

    def step(st, evs=None):
        if evs is None:
            # the library's step entry point
            fk.step(st["X"], st["Q"], st["P"], st["vis"], st["W"], st["Kc"], st["Vc"], st["O"], st["LSE"],
                    stream=stream)
            return
        # the phases as separate launches, an event around each
        evs[0].record(stream)
        proj(st)
        evs[1].record(stream)
        attn(st)
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
    # each launch kind alone, back to back (the per-kernel average a kernel
    # trace reports): the roofline's launch time
    proj_avg = time_launches(proj, sets, stream, args.steps, 3)
    attn_avg = time_launches(attn, sets, stream, args.steps, 3)
    # the distribution over a pass with an event around each launch (the
    # events add a small gap between launches; not used for the averages)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(sets[i % n_sets], evs[i])
    torch.cuda.synchronize()
    proj_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    attn_ms = sorted(e[1].elapsed_time(e[2]) for e in evs)
    step_ms = sorted(e[0].elapsed_time(e[2]) for e in evs)

    def pct(v):
        n = len(v)
        return {"p10": round(v[n // 10] * 1e3, 3), "p50": round(v[n // 2] * 1e3, 3),
                "p90": round(v[min(n - 1, (n * 9) // 10)] * 1e3, 3)}

    # host cost of submitting a step: the enqueue loop alone (the launches
    # queue up on the device; this is the Python binding's and the library's
    # time per step, not the device's)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(sets[i % n_sets])
    host_submit_us = (time.perf_counter() - t0) / args.steps * 1e6
    torch.cuda.synchronize()

    copy_GBps, read_GBps = device_rates(dev, stream)
    log("bench: %.2f us/step (proj %.2f us, attn %.2f us alone), wall %.3f s, host submit %.1f us/step; "
        "device copy %.0f GB/s, read %.0f GB/s" %
        (ms_per_step * 1e3, proj_avg * 1e3, attn_avg * 1e3, wall, host_submit_us, copy_GBps, read_GBps))

    # warm-cache reference: the same set every step (Infinity Cache may hold it)
    warm_ms = time_launches(lambda st: step(st), [sets[0]], stream, min(args.steps, 50), 0)
    # the same step replayed from HIP graphs (no host launch calls between kernels)
    graph_ms = time_graph_steps(fk, sets, args.steps, 5)
    log("bench: graph-replayed step %.2f us" % (graph_ms * 1e3))

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
    pf = phase_fraction(dom_bytes, dom_flops, dom_ms * 1e3)
    roofline = {"bound": pf["bound"], "achieved": pf["achieved"],
                "peak": MFMA_BF16_PEAK_TFLOPS if pf["bound"] == "mfma" else HBM_PEAK_GBPS,
                "unit": pf["unit"], "frac": pf["frac"]}
    roofline.update({"traffic": traffic,
                     "kernel": "attn_mfma_kernel" if dom == "attn" else "proj_mfma_kernel",
                     "algorithmic_bytes_per_launch": dom_bytes, "algorithmic_flops_per_launch": dom_flops,
                     "avg_launch_us": round(dom_ms * 1e3, 3)})

    value = ab["total"] / (ms_per_step * 1e-3) / 1e9
    attn_GBps = ab["attn"] / (attn_avg * 1e-3) / 1e9
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
        "graph_step_us": round(graph_ms * 1e3, 3),
        "host_submit_us_per_step": round(host_submit_us, 2),
        "phases": {
            # each launch kind alone, back to back
            "proj_us": round(proj_avg * 1e3, 3),
            "attn_us": round(attn_avg * 1e3, 3),
            "proj_GBps": round(ab["proj"] / (proj_avg * 1e-3) / 1e9, 1),
            "attn_GBps": round(attn_GBps, 1),
            "proj_mfma_frac": round(ab["qkv_flops"] / (proj_avg * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "attn_hbm_frac": round(attn_GBps / HBM_PEAK_GBPS, 4),
            "attn_frac_of_read_ceiling": round(attn_GBps / read_GBps, 4),
            # one streaming read of the phase's bytes with the read probe
            "attn_read_floor_us": round(read_floor_us(ab["attn"], dev, stream), 3),
            # distribution over the evented pass (an event around each launch)
            "proj_us_pct": pct(proj_ms),
            "attn_us_pct": pct(attn_ms),
            "step_us_pct": pct(step_ms),
        },
        "algorithmic_bytes_per_step": ab["total"],
        "device_copy_GBps": round(copy_GBps, 1),
        "device_read_GBps": round(read_GBps, 1),
        "host": host_info(),
        "next_rows": selection,
        "roofline": roofline,
        "cpu_baseline": None,
    }
    fk.close()
    sets_main = sets

    # the other layer workloads of the target set, measured the same way
    others = {}
    for c in [int(x) for x in args.other_configs.split(",") if x.strip()]:
        if c == args.config:
            continue
        log("bench: workload %d" % c)
        others["workload%d" % c] = measure_config(c, min(args.steps, 100), 10, dev, read_GBps)
        o = others["workload%d" % c]
        log("bench: workload %d: step %.2f us (graph %.2f us), proj %.2f us, attn %.2f us (%.0f GB/s, %.3f of 8 TB/s)" %
            (c, o["step_us"], o["graph_step_us"], o["proj_us"], o["attn_us"], o["attn_GBps"], o["attn_hbm_frac"]))
    result["configs"] = others

    if not args.no_cpu:
        log("bench: timing the CPU oracle (budget %.0f s)" % args.cpu_budget)
        r, cpu_s, reps, threads = cpu_oracle_baseline(wl, K0, V0, args.cpu_budget)
        result["cpu_baseline"] = {"value": round(ab["total"] / cpu_s / 1e9, 4), "unit": "GB/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": "the full step of this workload (all %d sequences), "
                                            "median of %d run(s), %.2f s" % (ls.B, reps, cpu_s)}
        # parity of the timed path against the oracle on set 0
        import numpy as np
        o = sets_main[0]["O"].double().cpu().numpy()
        lse = sets_main[0]["LSE"].double().cpu().numpy()
        fin = np.isfinite(r["LSE"])
        result["parity"] = {
            "O_rel": float(np.abs(o - r["O"]).max() / np.abs(r["O"]).max()),
            "LSE_abs": float(np.abs(lse[fin] - r["LSE"][fin]).max()),
        }
        log("bench: cpu oracle %.2f s/step on %d threads; parity %s" % (cpu_s, threads, result["parity"]))

    print(json.dumps(result))


if __name__ == "__main__":
    main()
