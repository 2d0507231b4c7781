"""The update captured in a HIP graph (torch.cuda.graph) and replayed: with t
on the host every replay applies the same step t again, with t in device
memory the next one, and an overflow-gated step skips replays whose gradients
overflowed; after each replay, with eager work and a synchronisation in
between, the state must equal the oracle's. The library makes no allocation,
synchronisation or memset on this path, so capture is legal. Also here: the
combined entry point (layer_adam_step_ex) with every combination of its
options."""
import numpy as np
import pytest
import torch

import optimizer_step_layeradam_amd as la
import synth
from lahelpers import GpuLayer, compare, log, oracle_step, oracle_tensors

pytestmark = pytest.mark.gpu


def test_graph_replays_equal_repeated_oracle_steps():
    w = synth.Workload(name="graph", seed=5000,
                       tensors=(("a", 3), ("b", 2049), ("c", 70001), ("d", 4096)),
                       replicas=4, grad_dtype="bf16", step=9, with_flag=True)
    log("case graph capture")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    ts = oracle_tensors(L)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        # eager step first: the library reads its device facts outside capture
        gl.step()
    side.synchronize()
    oracle_step(L, ts)
    compare(gl.download(), ts, label="eager")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gl.step()
    scratch = torch.zeros(1 << 20, device="cuda")
    for replay in range(3):
        graph.replay()
        scratch.add_(1.0)              # unrelated eager work between replays
        torch.cuda.synchronize()
        oracle_step(L, ts)
        rep = compare(gl.download(), ts, label=f"replay{replay}")
        assert rep.max_ulp == 0 and gl.flag.item() == 0
        log(f"  replay {replay}: {rep}")
    gl.free()


def test_device_step_count_eager_and_at_zero():
    w = synth.Workload(name="dstep", seed=5100, tensors=(("a", 5), ("b", 4099), ("c", 30001)),
                       replicas=2, grad_dtype="bf16", step=11)
    log("case device step eager")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    t_dev = torch.zeros(1, dtype=torch.int64, device="cuda")
    before = gl.download()
    la.step_device_step(gl.params, gl.grads, t_dev, **w.hyper)   # t = 0: no-op
    after_zero = gl.download()
    for f in ("master", "exp_avg", "exp_avg_sq", "weight_out"):
        for a, b in zip(before[f], after_zero[f]):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f
    t_dev.fill_(w.step)
    la.step_device_step(gl.params, gl.grads, t_dev, **w.hyper)
    ts = oracle_tensors(L)
    oracle_step(L, ts)
    log(f"  {compare(gl.download(), ts, label='dstep')}")
    gl.free()


def test_graph_with_a_device_step_counter_advances_t_every_replay():
    w = synth.Workload(name="dstep_graph", seed=5200,
                       tensors=(("a", 3), ("b", 2049), ("c", 70001)),
                       replicas=4, grad_dtype="fp16", step=1, m_std=None, v_high=None,
                       grad_prescale=1024.0, unscale=1 / 1024, with_flag=True)
    log("case graph with device step")
    L = synth.make_layer(w)
    gl = GpuLayer(L, out="fp16")
    t_dev = torch.ones(1, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    kw = dict(w.hyper, grad_unscale=w.unscale, overflow_flag=gl.flag)
    with torch.cuda.stream(side):          # warm-up outside capture, t = 1
        la.step_device_step(gl.params, gl.grads, t_dev, **kw)
        t_dev.add_(1)
    side.synchronize()
    ts = oracle_tensors(L)
    oracle_step(L, ts, t=1, out="fp16")
    compare(gl.download(), ts, label="t=1", out="fp16")
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        la.step_device_step(gl.params, gl.grads, t_dev, **kw)
        t_dev.add_(1)
    for t in range(2, 7):
        graph.replay()
        torch.cuda.synchronize()
        oracle_step(L, ts, t=t, out="fp16")
        rep = compare(gl.download(), ts, label=f"t={t}", out="fp16")
        log(f"  replay t={t}: {rep}")
    assert int(t_dev.item()) == 7 and gl.flag.item() == 0
    gl.free()


def test_device_step_matches_the_host_step_over_many_t():
    """The constants that depend on t formed on the GPU (device pow in
    double) against the host's: over about 270 step counts from 1 to 2^31 - 1,
    m and v are bit-identical (they do not depend on t), the master is within
    one FP32 ulp, and where the masters agree so do the compute copies."""
    log("case device t vs host t")
    n = 4096 + 13
    w = synth.Workload(name="dstep_sweep", seed=5100, tensors=(("x", n),), replicas=2,
                       grad_dtype="bf16", step=1)
    L = synth.make_layer(w)
    a, b = GpuLayer(L), GpuLayer(L)
    la_a, la_b = la.Layer(a.params, a.grads), la.Layer(b.params, b.grads)
    init = [x.clone() for x in a.params[0][:3]]
    t_dev = torch.zeros(1, dtype=torch.int64, device="cuda")
    ts = sorted(set([1, 2, 3, 10, 100, 1000, 2**31 - 1]
                    + np.unique(np.geomspace(1, 2**31 - 1, 293).astype(np.int64)).tolist()))
    worst = 0
    for t in ts:
        for gl in (a, b):
            for dst, src in zip(gl.params[0][:3], init):
                dst.copy_(src)
        t_dev.fill_(int(t))
        la_a.step(step=int(t), **w.hyper)
        la_b.step_device_step(t_dev, **w.hyper)
        pa, pb = a.params[0], b.params[0]
        assert torch.equal(pa[1], pb[1]) and torch.equal(pa[2], pb[2]), t
        ia = pa[0].view(torch.int32).cpu().numpy().astype(np.int64)
        ib = pb[0].view(torch.int32).cpu().numpy().astype(np.int64)
        ia = np.where(ia < 0, -(ia & 0x7FFFFFFF), ia)
        ib = np.where(ib < 0, -(ib & 0x7FFFFFFF), ib)
        d = int(np.abs(ia - ib).max())
        worst = max(worst, d)
        assert d <= 1, (t, d)
        if d == 0:
            assert torch.equal(pa[3].view(torch.int16), pb[3].view(torch.int16)), t
    log(f"  {len(ts)} step counts, worst master difference {worst} ulp")
    a.free()
    b.free()


def _range_index(w, lo, hi):
    """Per-tensor index arrays of the layer elements [lo, hi)."""
    idx, off = [], 0
    for _, n in w.tensors:
        a, b = max(lo - off, 0), min(hi - off, n)
        idx.append(np.arange(a, b) if a < b else np.arange(0))
        off += n
    return idx


@pytest.mark.parametrize("dstep", [False, True])
@pytest.mark.parametrize("skip", ["none", "clear", "set"])
@pytest.mark.parametrize("use_range", [False, True])
def test_step_ex_every_combination_of_options(use_range, skip, dstep):
    """layer_adam_step_ex with a range or not, a skip flag absent, clear or
    set, and t on the host or the device: a set skip flag leaves everything
    untouched (state, copy, overflow flag); otherwise the range (or the whole
    layer) equals the oracle's step and every other element is untouched."""
    w = synth.Workload(name="step_ex", seed=5300,
                       tensors=(("a", 5), ("b", 4099), ("c", 30001), ("d", 257)),
                       replicas=3, grad_dtype="bf16", step=7, with_flag=True)
    log(f"case step_ex range={use_range} skip={skip} device_step={dstep}")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    before = gl.download()
    lo, hi = (3, w.numel - 100) if use_range else (0, w.numel)
    skip_t = None if skip == "none" else \
        torch.tensor([1 if skip == "set" else 0], dtype=torch.int32, device="cuda")
    t_dev = torch.tensor([w.step], dtype=torch.int64, device="cuda") if dstep else None
    rng = (lo, hi) if use_range else ()
    la.step_ex(gl.params, gl.grads, *rng, step=None if dstep else w.step, step_on_device=t_dev,
               skip_if_nonzero=skip_t, overflow_flag=gl.flag, grad_unscale=w.unscale,
               **w.hyper)
    got = gl.download()
    idx = _range_index(w, lo, hi)
    for i, (_, n) in enumerate(w.tensors):
        outside = np.ones(n, bool)
        if skip != "set":
            outside[idx[i]] = False
        for f in ("master", "exp_avg", "exp_avg_sq", "weight_out"):
            assert np.array_equal(got[f][i][outside].view(np.uint8),
                                  before[f][i][outside].view(np.uint8)), (f, i)
    assert got["flag"] == 0
    if skip != "set":
        ts = oracle_tensors(L, idx)
        oracle_step(L, ts)
        log(f"  {compare(got, ts, idx=idx, label='step_ex')}")
    gl.free()


def test_graph_of_an_overflow_gated_step_with_a_device_step_count():
    """A whole loss-scaled step of an FP16-gradient layer captured once: clear
    the flag (a fill kernel), the finite check, layer_adam_step_ex skipping on
    that flag with t read from the device, and t += 1 only when the flag is
    clear. Replayed with an overflow injected into one replay's gradients: that
    replay writes nothing and does not advance t, the others apply t = 1, 2, 3
    exactly as the oracle does."""
    w = synth.Workload(name="gated_graph", seed=5400,
                       tensors=(("a", 3), ("b", 2049), ("c", 70001)),
                       replicas=2, grad_dtype="fp16", step=1, m_std=None, v_high=None,
                       grad_prescale=1024.0, unscale=1 / 1024, with_flag=True)
    log("case graph of a gated step with a device step count")
    L = synth.make_layer(w)
    gl = GpuLayer(L, out="fp16")
    found = torch.zeros(1, dtype=torch.int32, device="cuda")
    t_dev = torch.ones(1, dtype=torch.int64, device="cuda")
    kw = dict(w.hyper, grad_unscale=w.unscale)

    def one_step():
        found.zero_()
        la.check_gradients(gl.grads, found, grad_unscale=w.unscale)
        la.step_ex(gl.params, gl.grads, skip_if_nonzero=found, step_on_device=t_dev, **kw)
        t_dev.add_((found == 0).to(torch.int64))

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):     # eager warm-up outside capture: t = 1
        one_step()
    side.synchronize()
    ts = oracle_tensors(L)
    oracle_step(L, ts, t=1, out="fp16")
    compare(gl.download(), ts, label="eager t=1", out="fp16")
    assert int(t_dev.item()) == 2

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        one_step()
    # replay 1: t = 2; replay 2: an overflowing gradient, skipped; replay 3: t = 3
    g = gl.grad_flat[1]
    k = L.grad_offsets[2] + 12345
    saved = g[k].clone()
    for replay, overflow in enumerate((False, True, False)):
        if overflow:
            g[k] = float("inf")
        before = gl.download()
        graph.replay()
        torch.cuda.synchronize()
        if overflow:
            g[k] = saved
            after = gl.download()
            for f in ("master", "exp_avg", "exp_avg_sq", "weight_out"):
                for a, b in zip(before[f], after[f]):
                    assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f
            assert int(found.item()) == 1
            log(f"  replay {replay}: overflow, skipped, t stays {int(t_dev.item())}")
            continue
        t = int(t_dev.item()) - 1
        oracle_step(L, ts, t=t, out="fp16")
        rep = compare(gl.download(), ts, label=f"replay {replay} t={t}", out="fp16")
        assert int(found.item()) == 0
        log(f"  replay {replay}: t={t} {rep}")
    assert int(t_dev.item()) == 4 and gl.flag.item() == 0
    gl.free()
