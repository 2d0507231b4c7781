"""Parity of the HIP path (through the C ABI) with the CPU oracle, on MI355X.

Bar: master, m, v within 2 FP32 ulp of the oracle (the sequence of FP32
operations is the same on both sides, so 0 ulp is expected); the compute copy
bit-exact; the overflow flag equal. Every input comes from the seeded
generator (synth) or is written out here; nothing is taken from the GPU side.
"""
import numpy as np
import pytest
import torch

import optimizer_step_layeradam_amd as la
import oracle
import synth
from lahelpers import (RAGGED, GpuLayer, Report, compare, compare_every_element, log,
                       oracle_step, oracle_tensors)

pytestmark = pytest.mark.gpu


def run_case(w: synth.Workload, mutate=None, steps=(None,), label="", **hp):
    log(f"case {label or w.name}: tensors={len(w.tensors)} N={w.numel} R={w.replicas} "
        f"{w.grad_dtype}")
    L = synth.make_layer(w)
    if mutate is not None:
        mutate(L)
    gl = GpuLayer(L)
    ts = oracle_tensors(L)
    flags = []
    for t in steps:
        gl.step(t=t, **hp)
        flags.append(oracle_step(L, ts, t=t, **hp))
    got = gl.download()
    rep = compare(got, ts, label=label or w.name)
    if w.with_flag or hp.get("with_flag"):
        assert got["flag"] == max(f or 0 for f in flags)
    gl.free()
    log(f"  {rep}")
    return got, ts, rep


# ---------------------------------------------------------------------------
# The workloads at reduced size: every tensor spans several chunks and ends
# in a ragged tail
# ---------------------------------------------------------------------------
SHRINK = {"tiny": 1, "qwen3_4b_layer": 64, "qwen3_14b_layer": 256, "flat_800m": 512,
          "qwen25_72b_layer": 512}


@pytest.mark.parametrize("name", list(SHRINK))
def test_workload_reduced(name):
    w = synth.WORKLOADS[name]
    if SHRINK[name] > 1:
        w = synth.shrink(w, SHRINK[name])
    _, _, rep = run_case(w)
    assert rep.max_ulp <= 2


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("R", range(1, 9))
def test_every_replica_count_and_dtype(R, dtype):
    w = synth.Workload(name=f"ragged_R{R}_{dtype}", seed=2000 + R, tensors=RAGGED,
                       replicas=R, grad_dtype=dtype, step=3, with_flag=True,
                       grad_prescale=1024.0 if dtype == "fp16" else 1.0,
                       unscale=1 / 1024 if dtype == "fp16" else 1.0)
    got, _, _ = run_case(w)
    assert got["flag"] == 0


def test_many_tensors_over_several_launches_with_empty_ones():
    sizes = []
    for k in range(40):
        sizes.append((f"t{k}", 0 if k % 7 == 3 else 1 + (k * 7919) % 20000))
    w = synth.Workload(name="forty_tensors", seed=2100, tensors=tuple(sizes), replicas=3,
                       grad_dtype="bf16", step=2)
    run_case(w)


def test_layer_of_empty_tensors_is_a_no_op():
    log("case empty layer")
    p = torch.ones(16, device="cuda")
    before = p.clone()
    la.step([(p[:0], p[:0], p[:0], torch.empty(0, dtype=torch.bfloat16, device="cuda"))],
            [[torch.empty(0, dtype=torch.bfloat16, device="cuda")] * 2],
            lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=1)
    la.step([], [], lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=1)
    torch.cuda.synchronize()
    assert torch.equal(p, before)


# ---------------------------------------------------------------------------
# Formats and special values
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_every_gradient_bit_pattern(dtype):
    """All 65536 patterns of the gradient format (subnormals, Inf, NaN), one
    replica, first step: decode, flag and propagation match."""
    w = synth.Workload(name=f"all_{dtype}", seed=2200, tensors=(("all", 65536),),
                       replicas=1, grad_dtype=dtype, step=1, with_flag=True)

    def mutate(L):
        L.grad_flat[0][:65536] = np.arange(65536, dtype=np.uint16)

    got, _, _ = run_case(w, mutate)
    assert got["flag"] == 1


@pytest.mark.parametrize("code", ["+inf", "-inf", "nan"])
def test_injected_non_finite_gradients(code):
    bits = {"+inf": 0x7F80, "-inf": 0xFF80, "nan": 0x7FC1}[code]
    w = synth.Workload(name=f"inject_{code}", seed=2300, tensors=RAGGED, replicas=4,
                       grad_dtype="bf16", step=5, with_flag=True)
    hits = []

    def mutate(L):
        rng = np.random.default_rng(1)
        for i, (_, n) in enumerate(w.tensors):
            for j in {0, n - 1, int(rng.integers(0, n))}:
                r = int(rng.integers(0, w.replicas))
                L.grad(r, i)[j] = bits
                hits.append((i, j))

    got, _, _ = run_case(w, mutate)
    assert got["flag"] == 1
    for i, j in hits:
        assert np.isnan(got["master"][i][j]) and got["weight_out"][i][j] == 0x7FC0


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_sums_past_the_gradient_format(dtype):
    """The replicas are summed in FP32: eight FP16 gradients of +-65504 sum to
    +-524032, far outside FP16 yet finite, so nothing is flagged; two BF16
    gradients at the largest finite BF16 overflow FP32 itself, which is."""
    w = synth.Workload(name=f"wide_sum_{dtype}", seed=2350, tensors=RAGGED, replicas=8,
                       grad_dtype=dtype, step=5, with_flag=True)
    ix = {name: i for i, (name, _) in enumerate(w.tensors)}

    def mutate(L):
        if dtype == "fp16":
            for r in range(8):
                L.grad(r, ix["k"])[:100] = 0x7BFF       # +65504
                L.grad(r, ix["l"])[100:300] = 0xFBFF    # -65504
        else:
            for r in (3, 6):
                L.grad(r, ix["n"])[77] = 0x7F7F         # largest finite BF16

    got, _, _ = run_case(w, mutate)
    assert got["flag"] == (1 if dtype == "bf16" else 0)


def test_flag_stays_zero_and_is_never_cleared():
    w = synth.shrink(synth.WORKLOADS["flat_800m"], 4096)
    log("case flag sticky")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    gl.step()
    torch.cuda.synchronize()
    assert gl.flag.item() == 0
    gl.flag.fill_(1)
    gl.step()
    torch.cuda.synchronize()
    assert gl.flag.item() == 1  # the library only ever writes 1
    gl.free()


def test_subnormal_state_and_gradients():
    w = synth.Workload(name="subnormal", seed=2400, tensors=RAGGED, replicas=2,
                       grad_dtype="fp16", step=4, master_std=1e-39, m_std=1e-40, v_high=1e-42,
                       grad_std=1e-7)
    _, ts, _ = run_case(w, lr=1e-3)
    tiny = np.concatenate([np.abs(x.exp_avg) for x in ts])
    assert np.any((tiny > 0) & (tiny < np.finfo(np.float32).tiny))


@pytest.mark.parametrize("case", range(6))
def test_hyperparameter_variants(case):
    hp = [dict(lr=1e-3, beta1=0.0, beta2=0.0, eps=1e-8, weight_decay=0.0),
          dict(lr=3e-4, beta1=0.5, beta2=0.95, eps=0.0, weight_decay=0.1),
          dict(lr=0.0, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01),
          dict(lr=1e-2, beta1=0.99, beta2=0.9999, eps=1e-6, weight_decay=1.0),
          dict(lr=1e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, unscale=1 / 3),
          dict(lr=1e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)][case]
    t = [1, 7, 2, 1_000_000, 50, 123_456_789][case]
    w = synth.Workload(name=f"hp{case}", seed=2500 + case, tensors=RAGGED, replicas=3,
                       grad_dtype="bf16", step=t)
    run_case(w, **hp)


def test_a_hundred_consecutive_steps():
    """t = 1..100 from zero moments on a reduced Qwen3-4B layer; the state is
    compared with the oracle's after every 25 steps (no drift, no stale
    element)."""
    w = synth.replace(synth.shrink(synth.WORKLOADS["qwen3_4b_layer"], 256), step=1,
                      m_std=None, v_high=None)
    log(f"case 100 steps N={w.numel}")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    ts = oracle_tensors(L)
    for t in range(1, 101):
        gl.step(t=t)
        oracle_step(L, ts, t=t)
        if t % 25 == 0:
            rep = compare(gl.download(), ts, label=f"t={t}")
            assert rep.max_ulp == 0
    gl.free()


def test_three_consecutive_steps():
    w = synth.Workload(name="three_steps", seed=2600, tensors=RAGGED, replicas=2,
                       grad_dtype="bf16", step=1, m_std=None, v_high=None)
    run_case(w, steps=(1, 2, 3))


# ---------------------------------------------------------------------------
# Buffers: aliasing replicas, output coverage, streams, host-side refusal
# ---------------------------------------------------------------------------
def test_one_gradient_buffer_passed_R_times():
    log("case aliased replicas")
    w = synth.Workload(name="alias", seed=2700, tensors=RAGGED, replicas=1,
                       grad_dtype="bf16", step=9)
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    gl.grads = [[g[0]] * 5 for g in gl.grads]
    la.step(gl.params, gl.grads, step=9, **w.hyper)
    ts = oracle_tensors(L)
    for x in ts:
        x.grads = x.grads * 5
    oracle.step(ts, dtype="bf16", step=9, **w.hyper)
    compare(gl.download(), ts, label="alias")
    gl.free()


def test_every_bf16_element_is_written():
    # GpuLayer pre-fills the BF16 outputs with 0x7FAA, a NaN payload the cast
    # never produces
    w = synth.Workload(name="coverage", seed=2800, tensors=RAGGED, replicas=1,
                       grad_dtype="bf16", step=1)
    got, _, _ = run_case(w)
    for wb in got["weight_out"]:
        assert not np.any(wb == 0x7FAA)


def test_runs_on_the_callers_stream():
    log("case side stream")
    w = synth.Workload(name="stream", seed=2900, tensors=RAGGED, replicas=2,
                       grad_dtype="bf16", step=11)
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gl.step()
    s.synchronize()
    ts = oracle_tensors(L)
    oracle_step(L, ts)
    compare(gl.download(), ts, label="stream")
    gl.free()


def test_bad_buffers_are_refused_before_any_work():
    log("case refusal")
    dev = "cuda"
    n = 4096
    p = torch.randn(n + 8, device=dev)
    m = torch.zeros(n + 8, device=dev)
    v = torch.zeros(n + 8, device=dev)
    wb = torch.zeros(n + 8, dtype=torch.bfloat16, device=dev)
    g = torch.randn(n + 8, device=dev).to(torch.bfloat16)
    before = [x.clone() for x in (p, m, v, wb)]
    hp = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, step=1)
    with pytest.raises(la.LayerAdamError) as e:  # 4-byte offset view
        la.step([(p[1:n + 1], m[:n], v[:n], wb[:n])], [[g[:n]]], **hp)
    assert e.value.status == 2
    with pytest.raises(la.LayerAdamError) as e:  # m written over master
        la.step([(p[:n], p[:n], v[:n], wb[:n])], [[g[:n]]], **hp)
    assert e.value.status == 3
    with pytest.raises(la.LayerAdamError) as e:  # gradient overlapping the BF16 output
        la.step([(p[:n], m[:n], v[:n], wb[:n])], [[wb[:n]]], **hp)
    assert e.value.status == 3
    with pytest.raises(la.LayerAdamError) as e:
        la.step([(p[:n], m[:n], v[:n], wb[:n])], [[g[:n]]], **dict(hp, step=0))
    assert e.value.status == 1
    torch.cuda.synchronize()
    for x, y in zip((p, m, v, wb), before):
        assert torch.equal(x.view(torch.int32 if x.dtype == torch.float32 else torch.int16),
                           y.view(torch.int32 if y.dtype == torch.float32 else torch.int16))


# ---------------------------------------------------------------------------
# Full sizes, in the benchmark's launch configuration: every element of every
# workload against the oracle, slice by slice on 16 host threads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_full_size(name):
    w = synth.WORKLOADS[name]
    log(f"case full {name}: N={w.numel} R={w.replicas} {w.grad_dtype}; generating inputs")
    L = synth.make_layer(w)
    log("  uploading")
    gl = GpuLayer(L)
    log("  GPU step")
    gl.step()
    torch.cuda.synchronize()
    log("  oracle on every element, slice by slice")
    rep, flag = compare_every_element(gl, L, label=name)
    got_flag = int(gl.flag.item())
    gl.free()
    if w.with_flag:
        assert got_flag == flag == 0
    log(f"  {rep}")
