"""Host-resident state: master, m and v in pinned host memory, updated by the
kernel over the host link, against the oracle on MI355X. The binding maps
each pinned tensor to its device-side address first and refuses anything
that is not mapped, so no kernel is launched on an unmapped pointer."""
import numpy as np
import pytest
import torch

import optimizer_step_layeradam_amd as la
import synth
from lahelpers import RAGGED, compare, log, oracle_step, oracle_tensors

pytestmark = pytest.mark.gpu


def pinned(a: np.ndarray) -> torch.Tensor:
    t = torch.empty(a.shape, dtype=torch.from_numpy(a[:0]).dtype, pin_memory=True)
    t.copy_(torch.from_numpy(a))
    return t


def test_pinned_tensors_are_mapped_for_the_gpu():
    t = pinned(np.arange(1024, dtype=np.float32))
    addr = la.device_address(t)
    log(f"pinned host {t.data_ptr():#x} -> device {addr:#x}")
    assert addr != 0
    assert la.device_address(t[8:]) == addr + 32      # interior views keep their offset
    with pytest.raises(TypeError):
        la.device_address(torch.zeros(16))           # pageable host memory is refused


@pytest.mark.parametrize("where", ["state", "everything"])
def test_host_resident_update_matches_the_oracle(where):
    w = synth.Workload(name=f"host_{where}", seed=4000, tensors=RAGGED, replicas=4,
                       grad_dtype="bf16", step=7, with_flag=True)
    log(f"case host-resident {where}")
    L = synth.make_layer(w)
    params, grads = [], []
    for i, (_, n) in enumerate(w.tensors):
        p, m, v = pinned(L.master[i]), pinned(L.exp_avg[i]), pinned(L.exp_avg_sq[i])
        if where == "everything":
            wb = torch.empty(n, dtype=torch.bfloat16, pin_memory=True)
            gs = [pinned(L.grad(r, i).copy()).view(torch.bfloat16) for r in range(w.replicas)]
        else:
            wb = torch.empty(n, dtype=torch.bfloat16, device="cuda")
            gs = [torch.from_numpy(L.grad(r, i).view(np.int16)).cuda().view(torch.bfloat16)
                  for r in range(w.replicas)]
        params.append((p, m, v, wb))
        grads.append(gs)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    la.step(params, grads, step=w.step, overflow_flag=flag, **w.hyper)
    torch.cuda.synchronize()
    got = {"master": [p.numpy().copy() for p, _, _, _ in params],
           "exp_avg": [m.numpy().copy() for _, m, _, _ in params],
           "exp_avg_sq": [v.numpy().copy() for _, _, v, _ in params],
           "weight_out": [wb.view(torch.int16).cpu().numpy().view(np.uint16)
                          for _, _, _, wb in params],
           "flag": int(flag.item())}
    ts = oracle_tensors(L)
    want_flag = oracle_step(L, ts)
    log(f"  {compare(got, ts, label=where)}")
    assert got["flag"] == want_flag == 0


def test_host_resident_update_at_size():
    """The 14B layer's tensor shapes divided by 32 (10.3M parameters, R = 8,
    1 % outliers): master, m and v in pinned host memory, gradients and the
    compute copy in HBM, two consecutive steps; every element against the
    oracle."""
    w = synth.shrink(synth.WORKLOADS["qwen3_14b_layer"], 32)
    assert w.numel > 10_000_000
    log(f"case host-resident at size: N={w.numel} R={w.replicas}")
    L = synth.make_layer(w)
    params, grads = [], []
    flat = [torch.from_numpy(g.view(np.int16)).cuda().view(torch.bfloat16) for g in L.grad_flat]
    for i, (_, n) in enumerate(w.tensors):
        params.append((pinned(L.master[i]), pinned(L.exp_avg[i]), pinned(L.exp_avg_sq[i]),
                       torch.empty(n, dtype=torch.bfloat16, device="cuda")))
        off = L.grad_offsets[i]
        grads.append([g[off:off + n] for g in flat])
    layer = la.Layer(params, grads)
    ts = oracle_tensors(L)
    for t in (w.step, w.step + 1):
        layer.step(step=t, **w.hyper)
        oracle_step(L, ts, t=t)
    torch.cuda.synchronize()
    got = {"master": [p.numpy().copy() for p, _, _, _ in params],
           "exp_avg": [m.numpy().copy() for _, m, _, _ in params],
           "exp_avg_sq": [v.numpy().copy() for _, _, v, _ in params],
           "weight_out": [wb.view(torch.int16).cpu().numpy().view(np.uint16)
                          for _, _, _, wb in params]}
    rep = compare(got, ts, label="host-resident at size")
    assert rep.compared == w.numel
    log(f"  {rep}")
