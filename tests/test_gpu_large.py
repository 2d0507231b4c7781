"""Maximum sizes: one tensor of more than 2^31 elements (64-bit element and
byte offsets), and a layer at the 256-tensor limit (sixteen launches).

The large tensor's inputs are drawn on the GPU by torch's seeded generator
(not by this library) and copied back at the sampled elements before the
update, so the oracle's inputs never come from the HIP path."""
import numpy as np
import pytest
import torch

import optimizer_step_layeradam_amd as la
import oracle
import synth
from lahelpers import compare, log, oracle_step, oracle_tensors, GpuLayer

pytestmark = pytest.mark.gpu

HP = dict(lr=1e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


def test_tensor_of_more_than_2_31_elements():
    n = (1 << 31) + (1 << 20) + 3
    R, t = 2, 77
    log(f"case large tensor n={n}")
    gen = torch.Generator(device="cuda").manual_seed(6000)
    dev = "cuda"
    p = torch.randn(n, device=dev, generator=gen).mul_(0.02)
    m = torch.randn(n, device=dev, generator=gen).mul_(1e-4)
    v = torch.rand(n, device=dev, generator=gen).mul_(1e-6)
    gs = [torch.randn(n, device=dev, generator=gen).mul_(1e-3).to(torch.bfloat16)
          for _ in range(R)]
    w = torch.empty(n, dtype=torch.bfloat16, device=dev)
    rng = np.random.default_rng(1)
    idx = np.unique(np.concatenate([
        np.arange(n - 4096, n), np.arange((1 << 31) - 4096, (1 << 31) + 4096),
        np.arange(0, 4096), rng.integers(0, n, 200_000)])).astype(np.int64)
    it = torch.from_numpy(idx).to(dev)
    x = oracle.Tensor(p[it].cpu().numpy(), m[it].cpu().numpy(), v[it].cpu().numpy(),
                      np.zeros(idx.size, np.uint16),
                      [g[it].view(torch.int16).cpu().numpy().view(np.uint16) for g in gs])
    torch.cuda.synchronize()
    la.step([(p, m, v, w)], [gs], step=t, **HP)
    torch.cuda.synchronize()
    got = {"master": [p[it].cpu().numpy()], "exp_avg": [m[it].cpu().numpy()],
           "exp_avg_sq": [v[it].cpu().numpy()],
           "weight_out": [w[it].view(torch.int16).cpu().numpy().view(np.uint16)]}
    oracle.step([x], dtype="bf16", step=t, **HP)
    log(f"  {compare(got, [x], label='large')}")
    # every element: the BF16 copy is the round-to-nearest-even cast of the master
    assert torch.equal(p.to(torch.bfloat16).view(torch.int16), w.view(torch.int16))
    del p, m, v, gs, w
    torch.cuda.empty_cache()


def test_layer_at_the_tensor_limit():
    sizes = tuple((f"t{k}", 1 + (k * 2654435761) % 5000) for k in range(la.MAX_TENSORS))
    w = synth.Workload(name="256_tensors", seed=6100, tensors=sizes, replicas=2,
                       grad_dtype="bf16", step=3, with_flag=True)
    log(f"case {len(sizes)} tensors N={w.numel}")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    gl.step()
    ts = oracle_tensors(L)
    flag = oracle_step(L, ts)
    got = gl.download()
    log(f"  {compare(got, ts, label='256')}")
    assert got["flag"] == flag == 0
    gl.free()
