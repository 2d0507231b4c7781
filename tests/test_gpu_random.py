"""Seeded random layers against the oracle on MI355X. Each case draws, from
its own seed, a layer shape (1-40 tensors; sizes at the update's chunk and
tile boundaries, random sizes up to 100K, some empty), the replica count,
the gradient format (FP16 with a power-of-two loss scale that the update
removes), the compute-copy format, whether the overflow flag is used, the
hyperparameters (within their domains, including beta1 = 0 and beta2 = 0)
and the step count; then applies the step as one call, as a random
partition of the layer into element ranges, or through layer_adam_step_ex
(ranges, a clear skip flag, t in device memory), and compares every element
and the flag with the oracle."""
import numpy as np
import pytest
import torch

import optimizer_step_layeradam_amd as la
import synth
from lahelpers import GpuLayer, compare, log, oracle_step, oracle_tensors

pytestmark = pytest.mark.gpu

EDGE = (1, 2, 3, 7, 8, 9, 63, 64, 65, 255, 256, 257, 511, 512, 513, 1023, 1024, 1025,
        4095, 4096, 4097)


def draw_case(case: int):
    rng = np.random.default_rng(9000 + case)
    sizes = []
    for k in range(int(rng.integers(1, 41))):
        u = rng.random()
        n = 0 if u < 0.1 else int(rng.choice(EDGE)) if u < 0.55 else int(rng.integers(1, 100_000))
        sizes.append((f"t{k}", n))
    if sum(n for _, n in sizes) == 0:
        sizes[0] = ("t0", 1000)
    fp16 = bool(rng.random() < 0.4)
    prescale = float(2.0 ** int(rng.integers(0, 11))) if fp16 else 1.0
    hyper = dict(lr=float(10 ** rng.uniform(-6, -2)),
                 beta1=float(rng.choice([0.0, 0.5, 0.9, 0.95])),
                 beta2=float(rng.choice([0.0, 0.9, 0.99, 0.999, 0.9999])),
                 eps=float(rng.choice([1e-8, 1e-6, 1e-3])),
                 weight_decay=float(rng.choice([0.0, 0.01, 0.1])))
    w = synth.Workload(
        name=f"random{case}", seed=9100 + case, tensors=tuple(sizes),
        replicas=int(rng.integers(1, 9)), grad_dtype="fp16" if fp16 else "bf16",
        step=int(rng.choice([1, 2, 7, 100, 12345, 10**6])),
        m_std=None if rng.random() < 0.2 else 1e-4, v_high=None if rng.random() < 0.2 else 1e-6,
        grad_prescale=prescale,
        unscale=1.0 / prescale if fp16 else float(rng.choice([1.0, 0.5, 0.125])),
        with_flag=bool(rng.random() < 0.5), hyper=hyper)
    out = str(rng.choice(["bf16", "fp16", "none"]))
    mode = str(rng.choice(["whole", "ranges", "ex"]))
    cuts = np.unique(np.concatenate([[0, w.numel],
                                     rng.integers(0, w.numel + 1, int(rng.integers(1, 6)))]))
    return w, out, mode, [int(c) for c in cuts]


@pytest.mark.parametrize("case", range(24))
def test_random_layer_matches_the_oracle(case):
    w, out, mode, cuts = draw_case(case)
    log(f"case random {case}: {len(w.tensors)} tensors N={w.numel} R={w.replicas} "
        f"{w.grad_dtype} out={out} flag={w.with_flag} t={w.step} mode={mode} "
        f"pieces={len(cuts) - 1} hyper={w.hyper}")
    L = synth.make_layer(w)
    gl = GpuLayer(L, out=out)
    kw = dict(w.hyper, grad_unscale=w.unscale,
              overflow_flag=gl.flag if w.with_flag else None)
    if mode == "whole":
        la.step(gl.params, gl.grads, step=w.step, **kw)
    elif mode == "ranges":
        layer = la.Layer(gl.params, gl.grads)
        for lo, hi in zip(cuts, cuts[1:]):
            layer.step_range(lo, hi, step=w.step, **kw)
    else:
        t_dev = torch.tensor([w.step], dtype=torch.int64, device="cuda")
        clear = torch.zeros(1, dtype=torch.int32, device="cuda")
        for lo, hi in zip(cuts, cuts[1:]):
            la.step_ex(gl.params, gl.grads, lo, hi, step_on_device=t_dev,
                       skip_if_nonzero=clear, **kw)
    got = gl.download()
    ts = oracle_tensors(L)
    flag = oracle_step(L, ts, out=out)
    rep = compare(got, ts, label=f"random {case}", out=out)
    if w.with_flag:
        assert got["flag"] == flag
    else:
        assert got["flag"] == 0
    log(f"  {rep}")
    gl.free()
