#!/usr/bin/env python3
"""Benchmark of the fused LayerAdam update on one MI355X.

A step is one LayerAdam update of one whole decoder layer (gradient sum over
the R replicas, unscale, AdamW moments and step, BF16 cast), one call of
layer_adam_step. Default workload: the Qwen3-14B-shaped decoder layer
(330,311,680 parameters in 9 tensors) with R = 8 BF16 gradient replicas.
Inputs are seeded synthetic tensors (synth/), uploaded to HBM before the
timed region.

Prints one JSON line:
  value        Gparam/s over the timed region (N * steps / wall time)
  roofline     HBM roofline of the kernel: algorithmic bytes per launch
               ((2R + 26) * N) over the mean launch time from HIP events on
               the launch stream, against 8 TB/s; traffic = HBM bytes per
               launch from the committed rocprofv3 counter summary (null if
               the kernel source changed since it was taken); the update's
               rate also against the stream probe, the reference copy, and
               (with the extras) its own loads and stores issued at once by
               two kernels or one after the other
  stream_probe the library's stream probe on the same layer: the update's
               loads, stores and launch shape without its arithmetic -- the
               rate HBM gives this mix of R + 3 read and 4 write streams
  per_workload every workload in turn (inputs drawn, uploaded, timed, freed):
               mean launch time of the update and of the probe, Gparam/s,
               GB/s and fraction of 8 TB/s
  extras       the neighbouring entry points on the same layer (chunked
               range updates, finite check and gated step, other copy
               formats, one GPU's shard, host-resident state), the
               the update and the stream probe with 1, 2, 4 and all R
               replicas, the per-chunk overlap of the update with two
               gradient producers, and the update's traffic split by
               direction (its loads alone, its stores alone, in sequence, at
               once, alternating by slice)
  cpu_baseline the CPU oracle timed on this host (one core) on a bounded
               prefix of the same layer, with its parity against the GPU's
               first step on that prefix

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME | --config NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "LayerAdam Gparam/s + HBM GB/s (% of peak), Qwen3-14B-shaped layer, R=8"
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
WARM_MS = 50.0  # untimed traffic before each per-workload measurement
KERNEL_SOURCES = ("optimizer_step_layeradam_amd/csrc/la_kernel.hip",
                  "optimizer_step_layeradam_amd/csrc/la_internal.h")
COUNTERS = os.path.join(ROOT, "profiles", "layeradam_counters.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed counter summary, if it was
    taken on this workload with the current kernel source."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    entry = c.get("workloads", {}).get(workload)
    if not entry or c.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def upload(L, torch):
    import numpy as np
    w = L.workload
    dev = torch.device("cuda:0")
    gdt = torch.float16 if w.grad_dtype == "fp16" else torch.bfloat16
    params = []
    for i, (_, n) in enumerate(w.tensors):
        params.append((torch.from_numpy(L.master[i]).to(dev),
                       torch.from_numpy(L.exp_avg[i]).to(dev),
                       torch.from_numpy(L.exp_avg_sq[i]).to(dev),
                       torch.empty(n, dtype=torch.bfloat16, device=dev)))
    flat = [torch.from_numpy(g.view(np.int16)).to(dev).view(gdt) for g in L.grad_flat]
    grads = [[g[off:off + n] for g in flat] for off, (_, n) in zip(L.grad_offsets, w.tensors)]
    return params, grads, flat


def cpu_baseline(L, first, budget_s: float):
    """Time the oracle (single-threaded, pinned to one core) on a prefix of
    every tensor, growing until about budget_s of CPU time; check it against
    the GPU's first step on the same elements."""
    import numpy as np
    import oracle
    w = L.workload
    try:
        old_aff = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(old_aff)})
    except (AttributeError, OSError):
        old_aff = None
    done = [0] * len(w.tensors)
    elapsed = 0.0
    worst_ulp = 0
    nonzero = 0
    bf16_bad = 0
    piece = 1 << 22
    try:
        while elapsed < budget_s and any(d < n for d, (_, n) in zip(done, w.tensors)):
            for i, (_, n) in enumerate(w.tensors):
                if done[i] >= n or elapsed >= budget_s:
                    continue
                a, b = done[i], min(n, done[i] + piece)
                t = oracle.Tensor(L.master[i][a:b].copy(), L.exp_avg[i][a:b].copy(),
                                  L.exp_avg_sq[i][a:b].copy(), np.zeros(b - a, np.uint16),
                                  [np.ascontiguousarray(L.grad(r, i)[a:b])
                                   for r in range(w.replicas)])
                t0 = time.perf_counter()
                oracle.step([t], dtype=w.grad_dtype, step=w.step, unscale=w.unscale,
                            with_flag=w.with_flag, **w.hyper)
                elapsed += time.perf_counter() - t0
                for field in ("master", "exp_avg", "exp_avg_sq"):
                    g = first[field][i][a:b].view(np.int32).astype(np.int64)
                    o = getattr(t, field).view(np.int32).astype(np.int64)
                    g = np.where(g < 0, -(g & 0x7FFFFFFF), g)
                    o = np.where(o < 0, -(o & 0x7FFFFFFF), o)
                    d = np.abs(g - o)
                    worst_ulp = max(worst_ulp, int(d.max()))
                    nonzero += int(np.count_nonzero(d))
                bf16_bad += int(np.count_nonzero(first["weight_out"][i][a:b] != t.weight_out))
                done[i] = b
    finally:
        if old_aff is not None:
            os.sched_setaffinity(0, old_aff)
    params = sum(done)
    gps = params / elapsed / 1e9
    return {
        "value": gps, "unit": "Gparam/s", "cores": 1, "kind": "oracle",
        "sample": (f"the first {params} of {w.numel} parameters of the same layer "
                   f"(a prefix of each of its {len(w.tensors)} tensors), one step at t={w.step}, "
                   f"single-threaded C oracle pinned to one core"),
        "seconds": elapsed,
        "hbm_model_gbs": gps * w.bytes_per_param,
        "host_cpu": _cpu_model(),
        "host_threads": os.cpu_count(),
        "parity_vs_gpu_first_step": {"params": params, "max_ulp": worst_ulp,
                                     "nonzero_ulp": nonzero, "bf16_mismatch": bf16_bad},
    }


def cpu_parallel(L, threads: int):
    """Context only: the same oracle over disjoint slices of the whole layer
    on `threads` host threads (ctypes releases the GIL), one step, wall time.
    Comparable in kind to the pages' multi-core host Adam."""
    import threading
    import numpy as np
    import oracle
    w = L.workload
    work = []
    for i, (_, n) in enumerate(w.tensors):
        for a in range(0, n, 1 << 22):
            b = min(n, a + (1 << 22))
            work.append(oracle.Tensor(L.master[i][a:b].copy(), L.exp_avg[i][a:b].copy(),
                                      L.exp_avg_sq[i][a:b].copy(), np.zeros(b - a, np.uint16),
                                      [np.ascontiguousarray(L.grad(r, i)[a:b])
                                       for r in range(w.replicas)]))
    lock = threading.Lock()
    queue = list(range(len(work)))

    def run():
        while True:
            with lock:
                if not queue:
                    return
                k = queue.pop()
            oracle.step([work[k]], dtype=w.grad_dtype, step=w.step, unscale=w.unscale,
                        **w.hyper)

    pool = [threading.Thread(target=run) for _ in range(threads)]
    t0 = time.perf_counter()
    for t in pool:
        t.start()
    for t in pool:
        t.join()
    seconds = time.perf_counter() - t0
    gps = w.numel / seconds / 1e9
    return {"value": gps, "unit": "Gparam/s", "cores": threads, "kind": "oracle, disjoint slices",
            "sample": f"the whole layer ({w.numel} parameters), one step", "seconds": seconds,
            "hbm_model_gbs": gps * w.bytes_per_param}


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def copy_reference(torch, la, mib: int = 2048, reps: int = 10):
    """Bandwidth of a plain two-stream copy on this GPU, the context for the
    roofline: the library's reference copy (la_copy_reference: the update's
    access style, one read and one write stream, no arithmetic) and torch's
    Tensor.copy_, each over the same buffers, HIP events around `reps` copies."""
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)

    def rate(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return 2 * n * reps / (a.elapsed_time(b) / 1e3) / 1e9

    gbs = rate(lambda: la.copy_reference(dst, src))
    torch_gbs = rate(lambda: dst.copy_(src))
    del src, dst
    torch.cuda.empty_cache()
    return {"gbs": gbs, "frac_of_peak": gbs / PEAK_HBM_GBS, "bytes_per_copy": 2 * n,
            "kernel": "la_copy_reference (copy_kernel)", "torch_copy_gbs": torch_gbs}


def host_link_reference(torch, mib: int = 1024, reps: int = 5):
    """Bandwidth of the host link for pinned buffers: DMA copies host to
    device, device to host, and both at once on two streams. An update whose
    state lives in host memory moves as many bytes each way; its ceiling is
    the sum of the two one-way rates (a full-duplex link), which the two
    concurrent copies need not reach."""
    n = mib << 20
    h_in = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    h_out = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    d_in = torch.empty(n, dtype=torch.uint8, device="cuda:0")
    d_out = torch.zeros(n, dtype=torch.uint8, device="cuda:0")
    h_in.fill_(1)
    up, down = torch.cuda.Stream(), torch.cuda.Stream()

    def wall_ms(fn):
        fn()
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        return (time.perf_counter() - t_start) / reps * 1e3

    def h2d():
        with torch.cuda.stream(up):
            d_in.copy_(h_in, non_blocking=True)

    def d2h():
        with torch.cuda.stream(down):
            h_out.copy_(d_out, non_blocking=True)

    def both():
        h2d()
        d2h()

    out = {"bytes_per_direction": n, "kernel": "Tensor.copy_ (DMA, pinned host)"}
    for name, fn, moved in (("h2d", h2d, n), ("d2h", d2h, n), ("both", both, 2 * n)):
        out[f"{name}_gbs"] = moved / wall_ms(fn) / 1e6
    del h_in, h_out, d_in, d_out
    torch.cuda.empty_cache()
    return out


def time_launches(torch, fn, reps=10, warm=2, warm_ms=0.0):
    """Mean milliseconds of fn() over reps, HIP events on the current stream,
    after `warm` untimed calls and then more until warm_ms of wall time has
    passed (a freshly uploaded layer runs a few percent slower for its first
    tens of milliseconds of traffic)."""
    for _ in range(warm):
        fn()
    torch.cuda.synchronize()
    t_end = time.perf_counter() + warm_ms / 1e3
    while time.perf_counter() < t_end:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return statistics.fmean(a.elapsed_time(b) for a, b in ev)


def rates(w, ms):
    """Gparam/s, GB/s under the (2R + 26)-byte model and fraction of 8 TB/s for
    one launch of ms milliseconds over workload w."""
    gbs = w.traffic_bytes / ms / 1e6
    return {"ms": ms, "gparams": w.numel / ms / 1e6, "gbs": gbs, "frac": gbs / PEAK_HBM_GBS}


def stream_probe(torch, layer, w, reps=20):
    """The stream probe on the resident layer (mean launch time, HIP events)."""
    return dict(rates(w, time_launches(torch, layer.stream_probe, reps=reps, warm=3,
                                       warm_ms=WARM_MS)),
                kernel="layer_adam_kernel (probe mode: no arithmetic)")


def per_workload(torch, la, synth, reps=20):
    """Every workload in turn: draw, upload, time the update and the probe
    (mean launch time over reps launches, HIP events), free."""
    out = {}
    for name, w in synth.WORKLOADS.items():
        t_draw = time.time()
        L = synth.make_layer(w)
        params, grads, flat = upload(L, torch)
        del L
        log(f"bench: per-workload {name}: inputs resident after {time.time() - t_draw:.1f}s")
        flag = torch.zeros(1, dtype=torch.int32, device="cuda:0") if w.with_flag else None
        layer = la.Layer(params, grads)
        t = [w.step]

        def one():
            layer.step(step=t[0], grad_unscale=w.unscale, overflow_flag=flag, **w.hyper)
            t[0] += 1

        entry = {"params": w.numel, "replicas": w.replicas, "grad_dtype": w.grad_dtype,
                 "bytes_per_param": w.bytes_per_param,
                 "update": rates(w, time_launches(torch, one, reps=reps, warm=3,
                                                  warm_ms=WARM_MS)),
                 "probe": stream_probe(torch, layer, w, reps=reps)}
        entry["update_over_probe"] = entry["update"]["gbs"] / entry["probe"]["gbs"]
        if flag is not None:
            entry["overflow_flag"] = int(flag.item())
        if w.traffic_bytes < 256 << 20:
            entry["note"] = ("cache-resident (the whole layer fits in the caches) and "
                             "launch-bound: not an HBM measurement")
        out[name] = entry
        del layer, params, grads, flat, flag
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def producer_overlap(torch, la, w, L, params, grads, flat, t0, k=1024, reps=3,
                     host_link=True):
    """Per-chunk release behind a gradient producer, with 64 MiB chunks per
    replica. Producers (synth.producer): a GEMM on the GPU (the gradients
    times the k x k identity, 2k flops per element, values unchanged) and DMA
    from pinned host memory over the host link. After each chunk the producer
    stream records an event; on a side stream the update of that chunk waits
    on it and runs while the producer continues. Reports, per producer, the
    producer alone, the chunked update alone and the two overlapped (wall
    time between HIP events), and whether the gradients came out unchanged."""
    from synth.producer import GemmProducer, HostLinkProducer, flat_to_layer
    chunk = (64 << 20) // 2
    sizes = [n for _, n in w.tensors]
    layer = la.Layer(params, grads)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    t = [t0]

    def hp():
        t[0] += 1
        return dict(step=t[0], grad_unscale=w.unscale, **w.hyper)

    def timed(body):
        ms = []
        for rep in range(reps + 1):
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(main)
            end_stream = body(a)
            b.record(end_stream)
            torch.cuda.synchronize()
            if rep:
                ms.append(a.elapsed_time(b))
        return statistics.fmean(ms)

    def measure(prod, src):
        ranges = [tuple(flat_to_layer(L.grad_offsets, sizes, x) for x in ab)
                  for ab in prod.bounds]

        def producer_alone(_):
            for c in range(len(prod.bounds)):
                prod.produce(c)
            return main

        def update_alone(_):
            for lo, hi in ranges:
                layer.step_range(lo, hi, **hp())
            return main

        def overlapped(start):
            side.wait_event(start)
            for c, (lo, hi) in enumerate(ranges):
                prod.produce(c)
                ready = torch.cuda.Event()
                ready.record(main)
                side.wait_event(ready)
                layer.step_range(lo, hi, stream=side, **hp())
            return side

        p_ms, u_ms, o_ms = timed(producer_alone), timed(update_alone), timed(overlapped)
        main.wait_stream(side)
        torch.cuda.synchronize()
        # the producer wrote the original values back (+0 and -0 alike)
        same = all(bool(((s.to(d.device).view(torch.int16) == d.view(torch.int16)) |
                         ((s.to(d.device) == 0) & (d == 0))).all())
                   for s, d in zip(src, flat))
        return {"chunks": len(prod.bounds), "producer_ms": p_ms, "update_ms": u_ms,
                "overlapped_ms": o_ms, "serial_ms": p_ms + u_ms,
                "overlapped_over_max": o_ms / max(p_ms, u_ms),
                "update_hidden_fraction": (p_ms + u_ms - o_ms) / u_ms,
                "gradients_reproduced": same}

    out = {"chunk_bytes_per_replica": chunk * 2}
    src = [g.clone() for g in flat]
    prod = GemmProducer(src, flat, chunk_elems=chunk, k=k)
    out["gemm"] = measure(prod, src)
    out["gemm"]["gemm_k"] = k
    out["gemm"]["producer_tflops"] = (prod.flops_per_chunk * len(prod.bounds) /
                                      out["gemm"]["producer_ms"] / 1e9)
    del src, prod
    torch.cuda.empty_cache()
    if not host_link:
        return out
    host = [torch.empty(g.shape, dtype=g.dtype, pin_memory=True) for g in flat]
    for h, g in zip(host, flat):
        h.copy_(g)
    prod = HostLinkProducer(host, flat, chunk_elems=chunk)
    out["host_link"] = measure(prod, host)
    out["host_link"]["producer_gbs"] = (prod.bytes_per_chunk * len(prod.bounds) /
                                        out["host_link"]["producer_ms"] / 1e6)
    del host, prod
    return out


def replica_sweep(torch, la, w, params, grads, t0, reps=10):
    """The update and its stream probe on the resident layer with the first R
    of its gradient replicas, R = 1, 2, 4 and the layer's own: (2R + 26)
    B/param, so fewer read streams and a smaller read share."""
    out = {}
    t = [t0]
    for R in sorted({1, 2, 4, w.replicas}):
        if R > w.replicas:
            continue
        layer = la.Layer(params, [g[:R] for g in grads])
        nbytes = (2 * R + 26) * w.numel

        def one():
            layer.step(step=t[0], grad_unscale=w.unscale, **w.hyper)
            t[0] += 1

        entry = {}
        for k, fn in (("update", one), ("probe", layer.stream_probe)):
            ms = time_launches(torch, fn, reps=reps, warm=3, warm_ms=WARM_MS)
            entry[k] = {"ms": ms, "gbs": nbytes / ms / 1e6, "frac": nbytes / ms / 1e6 / PEAK_HBM_GBS}
        entry["bytes_per_param"] = 2 * R + 26
        out[str(R)] = entry
    return out


def direction_split(torch, la, layer, w, update_ms, reps=10):
    """The update's traffic taken apart by direction on the resident layer,
    with the library's direction probe: its loads alone ((2R + 12) B/param),
    its stores alone (14 B/param), the two in sequence, the two at once on
    two streams, and the two alternating over P consecutive slices of the
    layer (a read phase, then the write phase of the same slice), against the
    update itself. The write part overwrites the state (with zeros), so this
    runs after every measurement that needs it."""
    n = w.numel
    read_b = (2 * w.replicas + 12) * n
    write_b = w.traffic_bytes - read_b
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()

    def entry(ms, nbytes):
        gbs = nbytes / ms / 1e6
        return {"ms": ms, "gbs": gbs, "frac": gbs / PEAK_HBM_GBS}

    def reads(lo=0, hi=n, stream=None):
        layer.direction_probe(la.PROBE_READS, lo, hi, stream=stream)

    def writes(lo=0, hi=n, stream=None):
        layer.direction_probe(la.PROBE_WRITES, lo, hi, fill=0, stream=stream)

    def at_once():
        start = torch.cuda.Event()
        start.record(main)
        side.wait_event(start)
        writes(stream=side)
        reads()
        done = torch.cuda.Event()
        done.record(side)
        main.wait_event(done)

    r_ms = time_launches(torch, reads, reps=reps, warm=3, warm_ms=WARM_MS)
    w_ms = time_launches(torch, writes, reps=reps, warm=3)
    out = {"read_bytes_per_param": 2 * w.replicas + 12,
           "write_bytes_per_param": w.bytes_per_param - 2 * w.replicas - 12,
           "kernel": "direction_kernel (la_direction_probe)",
           "reads_alone": entry(r_ms, read_b), "writes_alone": entry(w_ms, write_b),
           "in_sequence": entry(r_ms + w_ms, w.traffic_bytes),
           "at_once_two_streams": entry(time_launches(torch, at_once, reps=reps, warm=2),
                                        w.traffic_bytes),
           "update": entry(update_ms, w.traffic_bytes)}
    phases = {}
    for p in (1, 4, 16, 64):
        cuts = [n * k // p for k in range(p + 1)]

        def alternate():
            for lo, hi in zip(cuts, cuts[1:]):
                reads(lo, hi)
                writes(lo, hi)

        phases[str(p)] = dict(entry(time_launches(torch, alternate, reps=5, warm=2),
                                    w.traffic_bytes), params_per_phase=n // p)
    out["alternating_phases"] = phases
    return out


def extras(torch, la, w, params, grads, t0):
    """The neighbouring entry points on the same resident layer, timed after
    the main region: the layer released in 64 MiB gradient chunks through the
    range entry point, the finite-check pre-pass, check + gated step, the
    FP16 and no compute copies, the host cost of a call, one GPU's shard of
    the layer split 2, 4 or 8 ways, and the state held in pinned host memory."""
    n = w.numel
    t = [t0]

    def hp():
        t[0] += 1
        return dict(step=t[0], grad_unscale=w.unscale, **w.hyper)

    out = {}
    chunk = (64 << 20) // 2  # elements of one 64 MiB chunk of a 16-bit gradient replica

    def by_chunks():
        for lo in range(0, n, chunk):
            la.step_range(params, grads, lo, min(n, lo + chunk), **hp())

    ms_whole = time_launches(torch, lambda: la.step(params, grads, **hp()))
    ms = time_launches(torch, by_chunks)
    out["range_64MiB_chunks"] = {"chunks": -(-n // chunk), "ms": ms, "whole_layer_ms": ms_whole,
                                 "overhead": ms / ms_whole - 1.0,
                                 "gbs": w.traffic_bytes / ms / 1e6}
    found = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    layer = la.Layer(params, grads)
    ms = time_launches(torch, lambda: layer.check_gradients(found, grad_unscale=w.unscale),
                       warm_ms=WARM_MS)
    out["check_gradients"] = {"ms": ms, "bytes_per_param": 2 * w.replicas,
                              "gbs": 2 * w.replicas * n / ms / 1e6}

    def gated():
        found.zero_()
        layer.check_gradients(found, grad_unscale=w.unscale)
        layer.step_gated(found, **hp())

    ms = time_launches(torch, gated)
    out["check_then_gated_step"] = {"ms": ms, "bytes_per_param": 4 * w.replicas + 26,
                                    "gbs": (4 * w.replicas + 26) * n / ms / 1e6}
    as_fp16 = [(p, m, v, wb.view(torch.float16)) for p, m, v, wb in params]
    ms = time_launches(torch, lambda: la.step(as_fp16, grads, **hp()))
    out["fp16_compute_copy"] = {"ms": ms, "gbs": w.traffic_bytes / ms / 1e6}
    no_copy = [(p, m, v, None) for p, m, v, _ in params]
    ms = time_launches(torch, lambda: la.step(no_copy, grads, **hp()))
    out["no_compute_copy"] = {"ms": ms, "bytes_per_param": 2 * w.replicas + 24,
                              "gbs": (2 * w.replicas + 24) * n / ms / 1e6}
    # Host cost of one call (the GPU work stays the same): the functional form
    # rebuilds the layer descriptor from the tensors each time, a Layer object
    # describes it once. Measured as host wall time of enqueuing 20 steps.
    def host_us(fn, reps=20):
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(reps):
            fn()
        host = (time.perf_counter() - t_start) / reps * 1e6
        torch.cuda.synchronize()
        return host

    out["host_us_per_call"] = {
        "functional": host_us(lambda: la.step(params, grads, **hp())),
        "layer_object": host_us(lambda: layer.step(**hp())),
        "tensors": len(params)}
    # One GPU's share of a layer sharded G ways by element range (each GPU
    # owning the master, m and v of its range): the middle shard, which
    # crosses tensor boundaries, updated alone through the range entry point.
    shards = {}
    for g in (2, 4, 8):
        lo, hi = n * (g // 2) // g, n * (g // 2 + 1) // g
        ms = time_launches(torch, lambda: layer.step_range(lo, hi, **hp()))
        shards[str(g)] = {"elements": hi - lo, "ms": ms,
                          "gbs": w.traffic_bytes * (hi - lo) / n / ms / 1e6}
    out["one_shard_of_g"] = shards
    # Host-resident state: master, m, v in pinned host memory; gradients and
    # the compute copy stay in HBM. 24 B/param cross the host link.
    host = []
    for p, m, v, wb in params:
        hp_, hm, hv = (torch.empty(x.shape, dtype=x.dtype, pin_memory=True) for x in (p, m, v))
        hp_.copy_(p)
        hm.copy_(m)
        hv.copy_(v)
        host.append((hp_, hm, hv, wb))
    ms = time_launches(torch, lambda: la.step(host, grads, **hp()), reps=3, warm=1)
    del host
    link = host_link_reference(torch)
    out["host_resident_state"] = {"ms": ms, "gparams": n / ms / 1e6,
                                  "host_link_bytes_per_param": 24,
                                  "host_link_gbs": 24 * n / ms / 1e6,
                                  "frac_of_dma_h2d_plus_d2h":
                                      24 * n / ms / 1e6 / (link["h2d_gbs"] + link["d2h_gbs"]),
                                  "host_link_reference": link}
    return out


def calibrate_copy(mib: int, reps: int):
    """A plain device-to-device copy of known size, for scaling the HBM byte
    counters (run under rocprofv3 --pmc)."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": n * 4, "reps": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", "--config", dest="workload", default=None,
                    help="workload to time (default qwen3_14b_layer): " + ", ".join(
                        ("tiny", "qwen3_4b_layer", "qwen3_14b_layer", "flat_800m",
                         "qwen25_72b_layer")))
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU time budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the neighbouring entry points timed after the main region")
    ap.add_argument("--no-per-workload", action="store_true",
                    help="skip timing every workload after the main region")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: the LayerAdam library drives one GPU; --gpus {args.gpus} is not "
              "supported (sharding the update across GPUs is described, not implemented)",
              file=sys.stderr, flush=True)
        sys.exit(2)
    if args.calibrate_copy_mib:
        calibrate_copy(args.calibrate_copy_mib, max(1, args.steps))
        return

    import numpy as np
    import torch

    import optimizer_step_layeradam_amd as la
    import synth

    name = args.workload or synth.BENCH_WORKLOAD
    w = synth.WORKLOADS[name]
    log(f"bench: {name} N={w.numel} tensors={len(w.tensors)} R={w.replicas} {w.grad_dtype}; "
        f"library {la.version()}")
    t0 = time.time()
    L = synth.make_layer(w)
    log(f"bench: inputs drawn in {time.time() - t0:.1f}s; uploading")
    params, grads, _flat = upload(L, torch)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda:0") if w.with_flag else None
    stream = torch.cuda.current_stream()

    # The layer is described once; every step then passes only t (the
    # library still checks every argument on each call).
    layer = la.Layer(params, grads)

    def one_step(t):
        layer.step(step=t, grad_unscale=w.unscale, overflow_flag=flag, stream=stream,
                   **w.hyper)

    # first step on the fresh inputs: its outputs feed the CPU-baseline parity
    one_step(w.step)
    torch.cuda.synchronize()
    first = None
    if not args.no_cpu_baseline:
        first = {"master": [], "exp_avg": [], "exp_avg_sq": [], "weight_out": []}
        for p, m, v, wb in params:
            first["master"].append(p.cpu().numpy())
            first["exp_avg"].append(m.cpu().numpy())
            first["exp_avg_sq"].append(v.cpu().numpy())
            first["weight_out"].append(wb.view(torch.int16).cpu().numpy().view(np.uint16))
    flag_first = int(flag.item()) if flag is not None else None

    # The stream probe (the update's bytes and launch shape, no arithmetic),
    # measured before the timed region: its 50+ ms of traffic over the same
    # buffers also settle the memory system, which runs a fresh layer a few
    # percent slower for its first tens of milliseconds. The probe leaves
    # master, m and v unchanged; the next update rewrites the compute copy it
    # overwrites. Nothing is freed on the device before the timed region:
    # releasing memory (as the reference copy does, after it) slows the next
    # ~100 ms of kernels by about 1 %.
    probe = stream_probe(torch, layer, w)

    t = w.step + 1
    for _ in range(args.warmup):
        one_step(t)
        t += 1
    torch.cuda.synchronize()

    K = args.steps
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    region0.record(stream)
    for k in range(K):
        starts[k].record(stream)
        one_step(t)
        ends[k].record(stream)
        t += 1
    region1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    region_ms = region0.elapsed_time(region1)
    launch_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    mean_ms = statistics.fmean(launch_ms)
    ms_per_step = region_ms / K
    value = w.numel * K / (region_ms / 1e3) / 1e9
    algo_bytes = w.traffic_bytes
    achieved = algo_bytes / (mean_ms / 1e3) / 1e9
    log(f"bench: {K} steps in {region_ms:.3f} ms (wall {wall * 1e3:.1f} ms); launch mean "
        f"{mean_ms:.4f} ms median {statistics.median(launch_ms):.4f} min {min(launch_ms):.4f} "
        f"max {max(launch_ms):.4f}; {achieved:.0f} GB/s")

    out = {
        "metric": METRIC,
        "value": value,
        "unit": "Gparam/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": name, "params": w.numel, "tensors": len(w.tensors),
                   "replicas": w.replicas, "grad_dtype": w.grad_dtype, "step": w.step,
                   "bytes_per_param": w.bytes_per_param, "parallelism": "single GPU"},
        "hbm_gbs": w.traffic_bytes * K / (region_ms / 1e3) / 1e9,
        "pct_of_peak_hbm": 100.0 * w.traffic_bytes * K / (region_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": measured_traffic(name),
                     "kernel": "layer_adam_kernel", "algorithmic_bytes_per_launch": algo_bytes,
                     "mean_launch_ms": mean_ms,
                     "median_launch_ms": statistics.median(launch_ms),
                     "min_launch_ms": min(launch_ms), "max_launch_ms": max(launch_ms)},
        "overflow_flag_first_step": flag_first,
        "stream_probe": probe,
        "hbm_copy_reference": copy_reference(torch, la),
        "extras": None,
        "per_workload": None,
        "cpu_baseline": None,
    }
    # the update's rate against the probe of its own stream mix and launch
    # shape, and against a plain two-stream copy
    out["roofline"]["stream_probe_gbs"] = out["stream_probe"]["gbs"]
    out["roofline"]["frac_of_stream_probe"] = achieved / out["stream_probe"]["gbs"]
    out["roofline"]["frac_of_copy_reference"] = achieved / out["hbm_copy_reference"]["gbs"]
    if not args.no_extras:
        out["extras"] = extras(torch, la, w, params, grads, t)
        out["extras"]["replica_sweep"] = replica_sweep(torch, la, w, params, grads, t + 500)
        log("bench: producer overlap")
        out["extras"]["producer_overlap"] = producer_overlap(torch, la, w, L, params, grads,
                                                             _flat, t + 1000)
        log("bench: direction split")
        ds = direction_split(torch, la, layer, w, mean_ms)
        out["extras"]["direction_split"] = ds
        # the update against its own loads and stores issued at once by two
        # kernels (how HBM serves the two directions interleaved) and against
        # the two run one after the other (what separating them in time
        # would give)
        out["roofline"]["mixed_reference_gbs"] = ds["at_once_two_streams"]["gbs"]
        out["roofline"]["frac_of_mixed_reference"] = achieved / ds["at_once_two_streams"]["gbs"]
        out["roofline"]["frac_of_in_sequence"] = achieved / ds["in_sequence"]["gbs"]
    del layer, params, grads, _flat
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not args.no_per_workload:
        out["per_workload"] = per_workload(torch, la, synth)
    if first is not None:
        log("bench: CPU oracle baseline")
        out["cpu_baseline"] = cpu_baseline(L, first, args.cpu_seconds)
        threads = min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                      else (os.cpu_count() or 1))
        log(f"bench: CPU oracle on {threads} threads (context)")
        out["cpu_parallel_context"] = cpu_parallel(L, threads)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
