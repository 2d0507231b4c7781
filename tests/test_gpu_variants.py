"""The other entry points and output formats, against the oracle, on MI355X:
FP16 and no compute copy, element-range updates, the gradient finite check
and the overflow-gated step."""
import numpy as np
import pytest
import torch

import optimizer_step_layeradam_amd as la
import oracle
import synth
from lahelpers import RAGGED, GpuLayer, compare, log, oracle_step, oracle_tensors

pytestmark = pytest.mark.gpu


def ragged(R, dtype="bf16", seed=3000, **kw):
    return synth.Workload(name=f"ragged_R{R}_{dtype}", seed=seed + R, tensors=RAGGED,
                          replicas=R, grad_dtype=dtype, step=5, **kw)


# ---------------------------------------------------------------------------
# Compute-copy formats
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("out", ["fp16", "none"])
@pytest.mark.parametrize("R", [1, 4, 8])
def test_compute_copy_format(R, out):
    w = ragged(R)
    log(f"case out={out} R={R}")
    L = synth.make_layer(w)
    gl = GpuLayer(L, out=out)
    gl.step()
    ts = oracle_tensors(L)
    oracle_step(L, ts, out=out)
    log(f"  {compare(gl.download(), ts, label=w.name, out=out)}")
    gl.free()


@pytest.mark.parametrize("out", ["bf16", "fp16"])
def test_cast_of_every_rounding_case(out):
    """lr = 0, zero gradients and moments: the new master equals the old bit
    for bit, so the compute copy is the cast of chosen FP32 patterns: every
    exponent and sign with the rounding-relevant low bits, plus Inf and NaN."""
    highs = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x0FFF, 0x1000, 0x1001, 0x1FFF, 0x2000, 0x3FFF, 0x4000,
                     0x7FFF, 0x8000, 0x8001, 0xBFFF, 0xC000, 0xEFFF, 0xF000, 0xFFFF],
                    dtype=np.uint32)
    pats = (highs[:, None] | lows[None, :]).ravel()
    n = pats.size
    log(f"case cast {out}: {n} patterns")
    w = synth.Workload(name=f"cast_{out}", seed=3100, tensors=(("x", n),), replicas=1,
                       grad_dtype="bf16", step=1, m_std=None, v_high=None)
    L = synth.make_layer(w)
    L.master[0][:] = pats.view(np.float32)
    L.grad_flat[0][:] = 0
    gl = GpuLayer(L, out=out)
    gl.step(lr=0.0)
    got = gl.download()
    gl.free()
    x = got["master"][0]
    num = ~np.isnan(pats.view(np.float32))              # p * 1 - 0 quiets a NaN
    assert np.array_equal(x.view(np.uint32)[num], pats[num])   # master unchanged
    assert np.all(np.isnan(x[~num]))
    cast = oracle.round_fp16 if out == "fp16" else oracle.round_bf16
    want = cast(pats.view(np.float32))
    bad = np.nonzero(got["weight_out"][0] != want)[0]
    assert bad.size == 0, (f"{bad.size} mismatches, first pattern {hex(int(pats[bad[0]]))}: "
                           f"gpu {got['weight_out'][0][bad[0]]:#06x} oracle {want[bad[0]]:#06x}")


# ---------------------------------------------------------------------------
# Element ranges
# ---------------------------------------------------------------------------
def _partition(n, rng, pieces):
    cuts = np.sort(rng.integers(0, n + 1, pieces - 1))
    bounds = np.concatenate([[0], cuts, [n]])
    return list(zip(bounds[:-1].tolist(), bounds[1:].tolist()))


@pytest.mark.parametrize("pieces", [1, 2, 7, 40])
def test_ranges_over_a_partition_equal_one_whole_step(pieces):
    w = ragged(3, with_flag=True)
    log(f"case ranges pieces={pieces}")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    rng = np.random.default_rng(pieces)
    parts = _partition(w.numel, rng, pieces)
    # include ranges that end exactly at tensor boundaries and empty ones
    for lo, hi in reversed(parts):
        la.step_range(gl.params, gl.grads, lo, hi, step=w.step, overflow_flag=gl.flag,
                      **w.hyper)
        la.step_range(gl.params, gl.grads, hi, hi, step=w.step, **w.hyper)  # empty: no-op
    ts = oracle_tensors(L)
    flag = oracle_step(L, ts)
    got = gl.download()
    rep = compare(got, ts, label=f"ranges{pieces}")
    assert rep.max_ulp == 0 and got["flag"] == flag == 0
    gl.free()


def test_fixed_size_chunks_over_a_layer():
    """The layer released in fixed-size chunks, as a producer would hand over
    reduced gradients chunk by chunk, on a side stream that waits on an
    event per chunk."""
    w = synth.shrink(synth.WORKLOADS["qwen3_4b_layer"], 16)
    log(f"case chunks N={w.numel}")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    chunk = 1_000_003
    side = torch.cuda.Stream()
    for lo in range(0, w.numel, chunk):
        ready = torch.cuda.Event()
        ready.record(torch.cuda.current_stream())
        side.wait_event(ready)
        la.step_range(gl.params, gl.grads, lo, min(w.numel, lo + chunk), step=w.step,
                      stream=side, **w.hyper)
    side.synchronize()
    ts = oracle_tensors(L)
    oracle_step(L, ts)
    log(f"  {compare(gl.download(), ts, label='chunks')}")
    gl.free()


@pytest.mark.parametrize("name", ["qwen3_14b_layer", "flat_800m"])
def test_update_overlaps_a_gradient_producer(name):
    """Per-chunk release with a real producer: on one stream a GEMM writes each
    chunk of every gradient replica (the seeded gradients times the identity,
    so the values are exactly the seeded ones); after each chunk it records an
    event, and on a second stream the update of that chunk waits on the event
    and runs while the producer moves on. Every element is compared with the
    oracle afterwards."""
    w = synth.shrink(synth.WORKLOADS[name], 16)
    log(f"case producer overlap {w.name}: N={w.numel} R={w.replicas}")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    from synth.producer import GemmProducer, flat_to_layer
    src = [g.clone() for g in gl.grad_flat]
    for g in gl.grad_flat:
        g.zero_()
    k = 256
    prod = GemmProducer(src, gl.grad_flat, chunk_elems=2048 * k, k=k)
    sizes = [n for _, n in w.tensors]
    layer = la.Layer(gl.params, gl.grads)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    side.wait_stream(main)
    for c, (a, b) in enumerate(prod.bounds):
        prod.produce(c)
        ready = torch.cuda.Event()
        ready.record(main)
        side.wait_event(ready)
        lo, hi = (flat_to_layer(L.grad_offsets, sizes, x) for x in (a, b))
        layer.step_range(lo, hi, step=w.step, grad_unscale=w.unscale,
                         overflow_flag=gl.flag if w.with_flag else None, stream=side, **w.hyper)
    main.wait_stream(side)
    torch.cuda.synchronize()
    assert len(prod.bounds) > 10
    for s, d in zip(src, gl.grad_flat):  # the producer wrote the seeded values (+-0 aside)
        same = (s.view(torch.int16) == d.view(torch.int16)) | ((s == 0) & (d == 0))
        assert bool(same.all())
    ts = oracle_tensors(L)
    flag = oracle_step(L, ts)
    got = gl.download()
    rep = compare(got, ts, label="producer overlap")
    if w.with_flag:
        assert got["flag"] == flag == 0
    log(f"  {rep}")
    gl.free()


def test_range_with_fp16_gradients_and_copy():
    w = ragged(2, "fp16", grad_prescale=1024.0, unscale=1 / 1024)
    L = synth.make_layer(w)
    gl = GpuLayer(L, out="fp16")
    for lo, hi in _partition(w.numel, np.random.default_rng(9), 13):
        la.step_range(gl.params, gl.grads, lo, hi, step=w.step, grad_unscale=w.unscale,
                      **w.hyper)
    ts = oracle_tensors(L)
    oracle_step(L, ts, out="fp16")
    compare(gl.download(), ts, label="range_fp16", out="fp16")
    gl.free()


# ---------------------------------------------------------------------------
# Gradient check and gated step
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("inject", [None, "inf", "nan", "cancel", "unscale"])
def test_gradient_check_matches_the_oracle(dtype, inject):
    w = ragged(4, dtype)
    log(f"case check {dtype} {inject}")
    L = synth.make_layer(w)
    ix = {name: i for i, (name, _) in enumerate(w.tensors)}
    unscale = 1.0
    codes = {"bf16": (0x7F80, 0xFF80, 0x7FC1, 0x7F7F), "fp16": (0x7C00, 0xFC00, 0x7E01, 0x7BFF)}
    inf, ninf, nan, big = codes[dtype]
    if inject == "inf":
        L.grad(2, ix["i"])[65536 + 12] = inf     # last element of the longest tensor
    elif inject == "nan":
        L.grad(0, ix["d"])[1000] = nan
    elif inject == "cancel":
        L.grad(1, ix["f"])[7], L.grad(3, ix["f"])[7] = inf, ninf
    elif inject == "unscale":
        for r in range(4):
            L.grad(r, ix["g"])[5] = big
        unscale = 2.0 ** 112 if dtype == "fp16" else 1.0
    gl = GpuLayer(L)
    found = torch.zeros(1, dtype=torch.int32, device="cuda")
    la.check_gradients(gl.grads, found, grad_unscale=unscale)
    torch.cuda.synchronize()
    want = oracle.check_finite(oracle_tensors(L), dtype=dtype, unscale=unscale)
    assert int(found.item()) == want
    assert want == (0 if inject is None else 1)
    gl.free()


def test_every_fp16_pattern_through_the_check():
    n = 65536
    w = synth.Workload(name="check_all", seed=3200, tensors=(("x", n),), replicas=1,
                       grad_dtype="fp16", step=1)
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    for lo, hi, want in ((0, 0x7C00, 0), (0x7C00, 0x8000, 1), (0x8000, 0xFC00, 0),
                         (0xFC00, 0x10000, 1)):
        bits = np.zeros(n, np.uint16)
        bits[: hi - lo] = np.arange(lo, hi, dtype=np.uint32).astype(np.uint16)
        g = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.float16)
        found = torch.zeros(1, dtype=torch.int32, device="cuda")
        la.check_gradients([[g]], found)
        torch.cuda.synchronize()
        assert int(found.item()) == want, (hex(lo), hex(hi))
    gl.free()


def test_gated_step_runs_when_clear_and_skips_when_set():
    w = ragged(2, with_flag=True)
    log("case gated")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    skip = torch.zeros(1, dtype=torch.int32, device="cuda")
    la.step_gated(gl.params, gl.grads, skip, step=w.step, overflow_flag=gl.flag, **w.hyper)
    ts = oracle_tensors(L)
    oracle_step(L, ts)
    after_one = gl.download()
    compare(after_one, ts, label="gated_clear")
    skip.fill_(1)
    gl.flag.fill_(0)
    la.step_gated(gl.params, gl.grads, skip, step=w.step + 1, overflow_flag=gl.flag, **w.hyper)
    after_skip = gl.download()
    for f in ("master", "exp_avg", "exp_avg_sq", "weight_out"):
        for a, b in zip(after_one[f], after_skip[f]):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f
    assert after_skip["flag"] == 0
    gl.free()


def test_check_then_gated_steps_over_two_layers_without_host_sync():
    """Loss-scaling flow: one flag for the whole step; the check runs over
    every layer first, then every layer's gated update; one layer overflows,
    so no layer changes."""
    log("case two layers gated")
    layers = []
    for k in range(2):
        w = ragged(2, "fp16", seed=3300 + 10 * k, grad_prescale=1024.0, unscale=1 / 1024)
        L = synth.make_layer(w)
        if k == 1:
            L.grad(0, [n for n, _ in w.tensors].index("h"))[123] = 0x7C00  # +Inf, 2nd layer
        layers.append((w, L, GpuLayer(L)))
    found = torch.zeros(1, dtype=torch.int32, device="cuda")
    for w, L, gl in layers:
        la.check_gradients(gl.grads, found, grad_unscale=w.unscale)
    before = [gl.download() for _, _, gl in layers]
    for w, L, gl in layers:
        la.step_gated(gl.params, gl.grads, found, step=w.step, grad_unscale=w.unscale,
                      **w.hyper)
    torch.cuda.synchronize()
    assert int(found.item()) == 1
    for (w, L, gl), b in zip(layers, before):
        a = gl.download()
        for f in ("master", "exp_avg", "exp_avg_sq", "weight_out"):
            for x, y in zip(a[f], b[f]):
                assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f
        gl.free()


def test_layer_object_matches_the_functional_calls():
    w = ragged(3, with_flag=True)
    L = synth.make_layer(w)
    a, b = GpuLayer(L), GpuLayer(L)
    layer = la.Layer(b.params, b.grads)
    assert layer.numel == w.numel and layer.traffic_bytes() == w.traffic_bytes
    for t in (5, 6):
        la.step(a.params, a.grads, step=t, overflow_flag=a.flag, **w.hyper)
        layer.step(step=t, overflow_flag=b.flag, **w.hyper)
    la.step_range(a.params, a.grads, 10, 70000, step=7, **w.hyper)
    layer.step_range(10, 70000, step=7, **w.hyper)
    ga, gb = a.download(), b.download()
    for f in ("master", "exp_avg", "exp_avg_sq", "weight_out"):
        for x, y in zip(ga[f], gb[f]):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f
    found = torch.zeros(1, dtype=torch.int32, device="cuda")
    layer.check_gradients(found)
    assert int(found.item()) == 0
    a.free()
    b.free()


def test_concurrent_calls_from_host_threads():
    """Four host threads update four layers at once, each on its own stream
    (the binding releases the interpreter lock inside the call), while a
    fifth thread keeps making a call the library refuses: every layer ends
    equal to three oracle steps, and each refusal reports its own error."""
    import threading
    log("case host threads")
    layers = []
    for k in range(4):
        w = synth.replace(ragged(1 + 2 * k, seed=3400 + 10 * k), step=1, m_std=None,
                          v_high=None)
        L = synth.make_layer(w)
        layers.append((w, L, GpuLayer(L)))
    streams = [torch.cuda.Stream() for _ in layers]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    barrier = threading.Barrier(len(layers) + 1)
    failures, refusals = [], []

    def updater(k):
        w, _, gl = layers[k]
        layer = la.Layer(gl.params, gl.grads)
        barrier.wait()
        try:
            for t in (1, 2, 3):
                layer.step(step=t, grad_unscale=w.unscale, stream=streams[k], **w.hyper)
        except Exception as e:  # reported below, on the main thread
            failures.append(repr(e))

    def refuser():
        w, _, gl = layers[0]
        barrier.wait()
        for _ in range(200):
            try:
                la.step(gl.params, gl.grads, step=0, **w.hyper)  # t = 0 is refused
                failures.append("step 0 accepted")
            except la.LayerAdamError as e:
                refusals.append(str(e))
            except Exception as e:  # reported below, on the main thread
                failures.append(repr(e))

    threads = [threading.Thread(target=updater, args=(k,)) for k in range(len(layers))]
    threads.append(threading.Thread(target=refuser))
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    for s in streams:
        s.synchronize()
    assert not failures, failures
    assert len(refusals) == 200 and all("step = 0" in r for r in refusals), set(refusals)
    for w, L, gl in layers:
        ts = oracle_tensors(L)
        for t in (1, 2, 3):
            oracle_step(L, ts, t=t)
        rep = compare(gl.download(), ts, label=w.name)
        log(f"  {rep}")
        assert rep.max_ulp == 0
        gl.free()


def test_binding_refuses_bad_device_scalars_without_launching():
    """A device step count that is not int64, and flags that are not int32 or
    have no element, are refused before anything is enqueued: the layer's
    state is unchanged afterwards."""
    log("case bad device scalars")
    w = ragged(2)
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    layer = la.Layer(gl.params, gl.grads)
    before = gl.download()
    hp = dict(w.hyper)
    int32_step = torch.ones(1, dtype=torch.int32, device="cuda")  # 4 bytes, not 8
    empty_flag = torch.zeros(0, dtype=torch.int32, device="cuda")
    float_flag = torch.zeros(1, dtype=torch.float32, device="cuda")
    with pytest.raises(TypeError):
        layer.step_device_step(int32_step, **hp)
    with pytest.raises(TypeError):
        la.step_device_step(gl.params, gl.grads, int32_step, **hp)
    with pytest.raises(ValueError):
        layer.step(step=3, overflow_flag=empty_flag, **hp)
    with pytest.raises(TypeError):
        layer.step(step=3, overflow_flag=float_flag, **hp)
    with pytest.raises(ValueError):
        layer.step_gated(empty_flag, step=3, **hp)
    with pytest.raises(ValueError):
        layer.check_gradients(empty_flag)
    after = gl.download()
    for f in ("master", "exp_avg", "exp_avg_sq", "weight_out"):
        for x, y in zip(before[f], after[f]):
            assert np.array_equal(x.view(np.uint8), y.view(np.uint8)), f
    gl.free()


@pytest.mark.parametrize("units", [0, 1, 255, 256, 257, 1025, 3 * 4096 + 7, 25_000_003])
def test_copy_reference_copies_exactly(units):
    """The bandwidth-reference copy: every byte arrives, nothing past the end
    is written (16-byte units; the kernel's chunk is 256 units)."""
    log(f"case copy reference {units} x 16 B")
    n = 16 * units
    g = torch.Generator(device="cuda").manual_seed(units)
    src = torch.randint(0, 256, (n,), dtype=torch.uint8, device="cuda", generator=g)
    big = torch.zeros(n + 4096, dtype=torch.uint8, device="cuda")
    la.copy_reference(big[:n], src)
    torch.cuda.synchronize()
    assert torch.equal(big[:n], src)
    assert int(big[n:].count_nonzero()) == 0
    if n >= 32:
        with pytest.raises(la.LayerAdamError, match="MISALIGNED"):
            la.copy_reference(big[8:8 + n - 16], src[:n - 16])


# ---------------------------------------------------------------------------
# The stream probe (measurement aid): the update's traffic, no arithmetic
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("out", ["bf16", "fp16", "none"])
@pytest.mark.parametrize("R", [1, 2, 5, 8])
def test_stream_probe_rewrites_state_and_xors_the_replicas(R, out):
    w = ragged(R, seed=3900)
    log(f"case probe R={R} out={out}")
    L = synth.make_layer(w)
    gl = GpuLayer(L, out=out)
    la.stream_probe(gl.params, gl.grads)
    got = gl.download()
    for i in range(len(w.tensors)):
        for field, want in (("master", L.master), ("exp_avg", L.exp_avg),
                            ("exp_avg_sq", L.exp_avg_sq)):
            assert np.array_equal(got[field][i].view(np.uint32), want[i].view(np.uint32)), \
                (field, i)
        x = L.grad(0, i).copy()
        for r in range(1, R):
            x ^= L.grad(r, i)
        if out == "none":
            assert np.all(got["weight_out"][i] == 0x7FAA)
        else:
            assert np.array_equal(got["weight_out"][i], x), i
    assert got["flag"] == 0
    # the next update rewrites the copy: one step equals the oracle's
    gl.step()
    ts = oracle_tensors(L)
    oracle_step(L, ts, out=out)
    compare(gl.download(), ts, label=f"after probe R={R}", out=out)
    gl.free()


def test_update_overlaps_gradients_arriving_over_the_host_link():
    """Per-chunk release behind DMA: each chunk of every replica is copied from
    pinned host memory on one stream; the update of that chunk waits on its
    event on a second stream. Every element is compared with the oracle."""
    w = synth.shrink(synth.WORKLOADS["qwen3_14b_layer"], 32)
    log(f"case host-link producer {w.name}: N={w.numel} R={w.replicas}")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    from synth.producer import HostLinkProducer, flat_to_layer
    host = [torch.from_numpy(g.view(np.int16)).view(torch.bfloat16).pin_memory()
            for g in L.grad_flat]
    for g in gl.grad_flat:
        g.zero_()
    prod = HostLinkProducer(host, gl.grad_flat, chunk_elems=(1 << 20) + 8)
    sizes = [n for _, n in w.tensors]
    layer = la.Layer(gl.params, gl.grads)
    main, side = torch.cuda.current_stream(), torch.cuda.Stream()
    side.wait_stream(main)
    for c, (a, b) in enumerate(prod.bounds):
        prod.produce(c)
        ready = torch.cuda.Event()
        ready.record(main)
        side.wait_event(ready)
        lo, hi = (flat_to_layer(L.grad_offsets, sizes, x) for x in (a, b))
        layer.step_range(lo, hi, step=w.step, stream=side, **w.hyper)
    main.wait_stream(side)
    torch.cuda.synchronize()
    assert len(prod.bounds) > 5
    ts = oracle_tensors(L)
    oracle_step(L, ts)
    log(f"  {compare(gl.download(), ts, label='host-link overlap')}")
    gl.free()


def test_stream_probe_over_several_launches_with_empty_tensors():
    """40 tensors (some empty) split into several launches: the probe leaves
    every state element unchanged and writes the XOR copy of every element."""
    sizes = [(f"t{k}", 0 if k % 7 == 3 else 1 + (k * 7919) % 20000) for k in range(40)]
    w = synth.Workload(name="probe_forty", seed=3950, tensors=tuple(sizes), replicas=3,
                       grad_dtype="bf16", step=2)
    log(f"case probe forty tensors N={w.numel}")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    la.Layer(gl.params, gl.grads).stream_probe()
    got = gl.download()
    for i, (_, n) in enumerate(w.tensors):
        for field, want in (("master", L.master), ("exp_avg", L.exp_avg),
                            ("exp_avg_sq", L.exp_avg_sq)):
            assert np.array_equal(got[field][i].view(np.uint32), want[i].view(np.uint32))
        x = L.grad(0, i) ^ L.grad(1, i) ^ L.grad(2, i)
        assert np.array_equal(got["weight_out"][i], x), i
    gl.free()


# ---------------------------------------------------------------------------
# The direction probe (the update's loads only, its stores only)
# ---------------------------------------------------------------------------
def _grads_unchanged(gl, L):
    for gf, want in zip(gl.grad_flat, L.grad_flat):
        assert np.array_equal(gf.view(torch.int16).cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("R", [1, 3, 8])
def test_direction_probe_reads_change_nothing(R):
    """The read part, at its default, uncapped and capped residency, over the
    whole layer and over a range that starts unaligned: no state, copy,
    gradient or flag changes."""
    w = ragged(R, seed=4000)
    log(f"case direction reads R={R}")
    L = synth.make_layer(w)
    gl = GpuLayer(L)
    layer = la.Layer(gl.params, gl.grads)
    for wg in (-1, 0, 3):
        layer.direction_probe(la.PROBE_READS, workgroups_per_cu=wg)
    layer.direction_probe(la.PROBE_READS, 5, w.numel - 3)
    got = gl.download()
    for i in range(len(w.tensors)):
        for field, want in (("master", L.master), ("exp_avg", L.exp_avg),
                            ("exp_avg_sq", L.exp_avg_sq)):
            assert np.array_equal(got[field][i].view(np.uint32), want[i].view(np.uint32))
        assert np.all(got["weight_out"][i] == 0x7FAA), i
    assert got["flag"] == 0
    _grads_unchanged(gl, L)
    gl.free()


@pytest.mark.parametrize("out", ["bf16", "none"])
def test_direction_probe_writes_exactly_the_range(out):
    """The write part over ranges that start and end inside tensors, at
    unaligned elements, across tensor boundaries, and empty: every element in
    a range holds the pattern (the copy its low half), every other element is
    untouched, and no gradient changes."""
    w = ragged(2, seed=4100)
    log(f"case direction writes out={out}")
    L = synth.make_layer(w)
    gl = GpuLayer(L, out=out)
    layer = la.Layer(gl.params, gl.grads)
    bounds = np.cumsum([0] + [n for _, n in w.tensors])
    want = {f: np.concatenate([a.view(np.uint32) for a in getattr(L, f)])
            for f in ("master", "exp_avg", "exp_avg_sq")}
    want_w = np.full(w.numel, 0x7FAA, np.uint16)
    cases = [(3, 260, 0x11111111), (bounds[5] - 1, bounds[9] + 5, 0xA5A5C3C3),
             (bounds[12] + 7, bounds[12] + 7, 0x22222222), (bounds[13] + 1, w.numel - 2, 0x3C003C00),
             (0, 1, 0xFFFF0001)]
    for k, (lo, hi, fill) in enumerate(cases):
        layer.direction_probe(la.PROBE_WRITES, int(lo), int(hi), fill=fill,
                              workgroups_per_cu=(-1, 0, 5)[k % 3])
        for f in want:
            want[f][lo:hi] = fill
        if out != "none":
            want_w[lo:hi] = fill & 0xFFFF
    got = gl.download()
    for f in want:
        assert np.array_equal(np.concatenate([a.view(np.uint32) for a in got[f]]), want[f]), f
    assert np.array_equal(np.concatenate(got["weight_out"]), want_w)
    assert got["flag"] == 0
    _grads_unchanged(gl, L)
    gl.free()


def test_direction_probe_over_several_launches_with_empty_tensors():
    """40 tensors (some empty) split into several launches: the read part
    changes nothing, the write part sets every element."""
    sizes = [(f"t{k}", 0 if k % 7 == 3 else 1 + (k * 7919) % 20000) for k in range(40)]
    w = synth.Workload(name="direction_forty", seed=4150, tensors=tuple(sizes), replicas=5,
                       grad_dtype="fp16", step=2)
    log(f"case direction forty tensors N={w.numel}")
    L = synth.make_layer(w)
    gl = GpuLayer(L, out="fp16")
    layer = la.Layer(gl.params, gl.grads)
    layer.direction_probe(la.PROBE_READS)
    got = gl.download()
    for i in range(len(w.tensors)):
        assert np.array_equal(got["master"][i].view(np.uint32), L.master[i].view(np.uint32))
    layer.direction_probe(la.PROBE_WRITES, fill=0x40490FDB)
    got = gl.download()
    for i in range(len(w.tensors)):
        for f in ("master", "exp_avg", "exp_avg_sq"):
            assert np.all(got[f][i].view(np.uint32) == 0x40490FDB), (f, i)
        assert np.all(got["weight_out"][i] == 0x0FDB), i
    _grads_unchanged(gl, L)
    gl.free()
