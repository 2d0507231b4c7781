"""The update captured in a HIP graph (torch.cuda.graph) and replayed: every
replay applies the same step t again; after each replay, with eager work and
a synchronisation in between, the state must equal the oracle's after the
same number of steps. The library makes no allocation, synchronisation or
memset on this path, so capture is legal."""
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
