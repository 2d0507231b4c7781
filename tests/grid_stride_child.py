"""Child process of tests/test_gpu_grid_stride.py, run with LAYERADAM_MAX_GRID
set so that every launch has far fewer workgroups than chunks and each
kernel's striding loop runs: the update (three launches of a ragged layer),
its range form with the device step count and a clear skip flag, the finite
check, both probes and the reference copy, each against the oracle or its
exact expected result. Prints 'grid stride ok' at the end."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
sys.path.insert(0, os.path.dirname(HERE))

import numpy as np  # noqa: E402
import torch  # noqa: E402

import optimizer_step_layeradam_amd as la  # noqa: E402
import synth  # noqa: E402
from lahelpers import RAGGED, GpuLayer, compare, log, oracle_step, oracle_tensors  # noqa: E402


def main():
    grid = os.environ.get("LAYERADAM_MAX_GRID")
    assert grid, "LAYERADAM_MAX_GRID must be set"
    sizes = RAGGED + tuple((f"x{k}", 1 + (k * 7919) % 30000) for k in range(20))
    w = synth.Workload(name="stride", seed=7000, tensors=sizes, replicas=3, grad_dtype="fp16",
                       step=5, grad_prescale=256.0, unscale=1 / 256, with_flag=True)
    log(f"grid cap {grid}: {len(sizes)} tensors, N={w.numel}")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    before = gl.download()

    # the finite check, clean
    found = torch.zeros(1, dtype=torch.int32, device="cuda")
    la.check_gradients(gl.grads, found, grad_unscale=w.unscale)
    torch.cuda.synchronize()
    assert int(found.item()) == 0

    # the stream probe and the read part of the direction probe leave the state
    la.stream_probe(gl.params, gl.grads)
    la.direction_probe(gl.params, gl.grads, la.PROBE_READS)
    got = gl.download()
    for i in range(len(sizes)):
        for f in ("master", "exp_avg", "exp_avg_sq"):
            assert np.array_equal(got[f][i].view(np.uint32), before[f][i].view(np.uint32)), (f, i)
        x = L.grad(0, i) ^ L.grad(1, i) ^ L.grad(2, i)
        assert np.array_equal(got["weight_out"][i], x), i
    log("  check, stream probe and read probe ok")

    # step t = 5 whole, then t = 6 as three ranges with t on the device
    gl.step()
    ts = oracle_tensors(L)
    oracle_step(L, ts)
    log(f"  update: {compare(gl.download(), ts, label='stride update')}")
    t_dev = torch.tensor([6], dtype=torch.int64, device="cuda")
    clear = torch.zeros(1, dtype=torch.int32, device="cuda")
    cuts = [0, 5, w.numel // 2 + 3, w.numel]
    for lo, hi in zip(cuts, cuts[1:]):
        la.step_ex(gl.params, gl.grads, lo, hi, step_on_device=t_dev, skip_if_nonzero=clear,
                   grad_unscale=w.unscale, overflow_flag=gl.flag, **w.hyper)
    oracle_step(L, ts, t=6)
    log(f"  ranges: {compare(gl.download(), ts, label='stride ranges')}")
    assert gl.flag.item() == 0

    # the finite check finds an overflow in the last tensor
    g = gl.grad_flat[2]
    k = L.grad_offsets[-1] + sizes[-1][1] - 1
    g[k] = float("inf")
    la.check_gradients(gl.grads, found, grad_unscale=w.unscale)
    torch.cuda.synchronize()
    assert int(found.item()) == 1
    log("  check finds the overflow")

    # the write part of the direction probe sets every element
    la.direction_probe(gl.params, gl.grads, la.PROBE_WRITES, fill=0x3F800000)
    got = gl.download()
    for i in range(len(sizes)):
        for f in ("master", "exp_avg", "exp_avg_sq"):
            assert np.all(got[f][i].view(np.uint32) == 0x3F800000), (f, i)
        assert np.all(got["weight_out"][i] == 0x0000), i

    # the reference copy, with a partial last chunk
    n = 16 * (3 * 4096 + 77)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros(n + 4096, dtype=torch.uint8, device="cuda")
    la.copy_reference(dst[:n], src)
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src) and int(dst[n:].count_nonzero()) == 0
    log("  write probe and reference copy ok")
    gl.free()
    print("grid stride ok", flush=True)


if __name__ == "__main__":
    main()
