"""The stream probe and the chunked release at full size, in the launch
configuration bench.py times, on MI355X.

The whole-layer update is compared with the oracle on every element in
test_gpu_parity.py; here the other two paths bench.py times on the same
layers are checked against it on the GPU, bit for bit: the probe must leave
master, m and v unchanged, and the layer updated as 64 MiB gradient chunks
through the range entry point must equal one whole-layer step."""
import pytest
import torch

import optimizer_step_layeradam_amd as la
import synth
from lahelpers import GpuLayer, log

pytestmark = pytest.mark.gpu


def _state_equal(a, b) -> bool:
    return all(torch.equal(x.view(torch.int32), y.view(torch.int32))
               for (x, y) in zip(a, b))


@pytest.mark.parametrize("name", ["qwen3_14b_layer", "flat_800m"])
def test_stream_probe_leaves_the_state_at_full_size(name):
    w = synth.WORKLOADS[name]
    log(f"case probe full {name}: N={w.numel} R={w.replicas}")
    gl = GpuLayer(synth.make_layer(w))
    before = [t.clone() for p, m, v, _ in gl.params for t in (p, m, v)]
    layer = la.Layer(gl.params, gl.grads)
    for _ in range(3):
        layer.stream_probe()
    torch.cuda.synchronize()
    after = [t for p, m, v, _ in gl.params for t in (p, m, v)]
    assert _state_equal(before, after)
    # the compute copy holds the XOR of the replicas
    for (_, _, _, wb), gs in zip(gl.params, gl.grads):
        x = gs[0].view(torch.int16).clone()
        for g in gs[1:]:
            x ^= g.view(torch.int16)
        assert torch.equal(wb.view(torch.int16), x)
    gl.free()


def test_chunked_release_equals_one_step_at_full_size():
    w = synth.WORKLOADS["qwen3_14b_layer"]
    log(f"case chunked release full: N={w.numel} R={w.replicas}, 64 MiB chunks")
    L = synth.make_layer(w)
    whole, chunked = GpuLayer(L), GpuLayer(L)
    chunk = (64 << 20) // 2           # elements of one 64 MiB chunk of a 16-bit replica
    hp = dict(step=w.step, grad_unscale=w.unscale, **w.hyper)
    la.Layer(whole.params, whole.grads).step(**hp)
    layer = la.Layer(chunked.params, chunked.grads)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for lo in range(0, w.numel, chunk):
        layer.step_range(lo, min(w.numel, lo + chunk), stream=side, **hp)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for (p0, m0, v0, w0), (p1, m1, v1, w1) in zip(whole.params, chunked.params):
        assert _state_equal((p0, m0, v0), (p1, m1, v1))
        assert torch.equal(w0.view(torch.int16), w1.view(torch.int16))
    whole.free()
    chunked.free()
