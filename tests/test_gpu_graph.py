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
