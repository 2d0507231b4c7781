"""The C-ABI library on the host: it loads, exports what include/layeradam.h
declares, accounts bytes as the pages do, and rejects bad arguments before
anything reaches a GPU. No kernel runs here.

The argument-validation cases use made-up device addresses; every one of them
is invalid on purpose and must be refused on the host. They are skipped
where a GPU is visible, so that no such address can ever reach a device.
"""
import ctypes
import json
import os
import re

import pytest
import torch  # noqa: F401  (load torch's HIP runtime before the library)

import optimizer_step_layeradam_amd as la
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "layeradam.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "state_accounting.json")


def declared_functions():
    text = open(HEADER).read()
    return re.findall(r"LA_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(la.EXPORTS)
    lib = ctypes.CDLL(la.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name


def test_version_names_the_target():
    assert "gfx950" in la.version()


def test_header_compiles_as_c():
    import subprocess
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        with open(src, "w") as f:
            f.write('#include "layeradam.h"\nint main(void){ la_layer_desc d = {0};'
                    ' return (int)la_state_bytes(&d); }\n')
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-c", "-I",
                        os.path.join(ROOT, "include"), src, "-o", os.path.join(d, "t.o")],
                       check=True)


# ---------------------------------------------------------------------------
# Byte accounting against the pages' printed values
# ---------------------------------------------------------------------------
def test_state_bytes_match_the_pages():
    g = json.load(open(GOLDEN))
    per = g["bytes_per_param"]
    assert (per["bf16_or_fp16_weights"] + per["bf16_or_fp16_gradients"] + per["fp32_master"]
            + per["fp32_adam_m_and_v"]) == per["total"] == 16
    assert la.state_bytes([1]) == per["total"]
    # master + m + v share of the state: 12 bytes per parameter
    assert per["fp32_master"] + per["fp32_adam_m_and_v"] == g["master_plus_moments_bytes_per_param"]["value"]
    for inst in g["instances"]:
        n = inst["params"]
        # split the count over several tensors, as a real layer list would be
        numels = [n // 4] * 3 + [n - 3 * (n // 4)]
        b = la.state_bytes(numels)
        if "state_bytes_greater_than" in inst:
            assert b > inst["state_bytes_greater_than"]
        if "state_bytes_at_least" in inst:
            assert b >= inst["state_bytes_at_least"]
        assert b == 16 * n


@pytest.mark.parametrize("name", sorted(synth.WORKLOADS))
def test_traffic_bytes_of_each_workload(name):
    w = synth.WORKLOADS[name]
    numels = [n for _, n in w.tensors]
    assert la.traffic_bytes(numels, w.replicas) == (2 * w.replicas + 26) * w.numel
    assert la.traffic_bytes(numels, w.replicas) == w.traffic_bytes


def test_workload_sizes():
    # parameter counts of the layer shapes (tensor list: q, k, v, o, gate, up,
    # down and two norms)
    expect = {"tiny": 274_432, "qwen3_4b_layer": 100_930_560,
              "qwen3_14b_layer": 330_311_680, "flat_800m": 800_000_003,
              "qwen25_72b_layer": 877_674_496}
    for name, n in expect.items():
        assert synth.WORKLOADS[name].numel == n


def test_traffic_without_a_compute_copy():
    assert la.traffic_bytes([1000, 24], 8, la.OUT_NONE) == (2 * 8 + 24) * 1024
    assert la.traffic_bytes([1000, 24], 8, la.OUT_FP16) == (2 * 8 + 26) * 1024


def test_accounting_rejects_bad_descriptors():
    desc, keep = la.make_layer([dict(numel=10)], 0, la.GRAD_BF16)
    assert la.state_bytes_raw(desc) == -1
    desc, keep = la.make_layer([dict(numel=-1)], 1, la.GRAD_BF16)
    assert la.traffic_bytes_raw(desc) == -1


# ---------------------------------------------------------------------------
# Validation, all on the host
# ---------------------------------------------------------------------------
host_only = pytest.mark.skipif(torch.cuda.is_available(),
                               reason="uses made-up device addresses; host-only check")

BASE = 0x7F0000000000  # made-up, 16-byte aligned; never dereferenced
HP = dict(lr=1e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01, step=1)


def fake_tensor(k, n=1024, R=2):
    base = BASE + k * 0x100000000
    return dict(master=base, exp_avg=base + 0x10000000, exp_avg_sq=base + 0x20000000,
                weight_out=base + 0x30000000,
                grads=[base + 0x40000000 + r * 0x1000000 for r in range(R)], numel=n)


def expect_status(tensors, R, dtype, hp, status, flag=0):
    desc, keep = la.make_layer(tensors, R, dtype)
    with pytest.raises(la.LayerAdamError) as e:
        la.step_raw(desc, la.make_params(**hp), flag)
    assert e.value.status == status, str(e.value)
    assert la.last_error() != ""


@host_only
@pytest.mark.parametrize("R", [0, 9, -1])
def test_replica_count_out_of_range(R):
    expect_status([fake_tensor(0)], R, la.GRAD_BF16, HP, 1)


@host_only
def test_unknown_gradient_dtype():
    expect_status([fake_tensor(0)], 2, 7, HP, 4)


@host_only
@pytest.mark.parametrize("bad", [dict(step=0), dict(step=-5), dict(beta1=1.0), dict(beta1=-0.1),
                                 dict(beta2=1.0), dict(lr=-1e-3), dict(lr=float("inf")),
                                 dict(eps=float("nan")), dict(weight_decay=-0.1),
                                 dict(grad_unscale=0.0), dict(grad_unscale=float("inf")),
                                 dict(grad_unscale=-1.0)])
def test_hyperparameters_outside_their_domain(bad):
    hp = dict(HP, grad_unscale=1.0)
    hp.update(bad)
    expect_status([fake_tensor(0)], 2, la.GRAD_BF16, hp, 1)


@host_only
@pytest.mark.parametrize("field", ["master", "exp_avg", "exp_avg_sq", "weight_out", "grad1"])
def test_null_buffer(field):
    t = fake_tensor(0)
    if field == "grad1":
        t["grads"][1] = 0
    else:
        t[field] = 0
    expect_status([t], 2, la.GRAD_BF16, HP, 1)


@host_only
@pytest.mark.parametrize("field", ["master", "exp_avg", "exp_avg_sq", "weight_out", "grad0"])
def test_misaligned_buffer(field):
    t = fake_tensor(0)
    if field == "grad0":
        t["grads"][0] += 8
    else:
        t[field] += 4
    expect_status([t], 2, la.GRAD_BF16, HP, 2)


@host_only
def test_misaligned_flag():
    expect_status([fake_tensor(0)], 2, la.GRAD_BF16, HP, 2, flag=BASE + 0x50000002)


@host_only
@pytest.mark.parametrize("case", ["m_on_master", "w_inside_v", "across_tensors", "grad_on_w",
                                  "flag_in_master"])
def test_overlapping_buffers(case):
    a, b = fake_tensor(0), fake_tensor(1)
    flag = 0
    if case == "m_on_master":
        a["exp_avg"] = a["master"] + 16
    elif case == "w_inside_v":
        a["weight_out"] = a["exp_avg_sq"] + 2048
    elif case == "across_tensors":
        b["master"] = a["exp_avg"] + 1024
    elif case == "grad_on_w":
        b["grads"][1] = a["weight_out"]
    elif case == "flag_in_master":
        flag = a["master"] + 64
    expect_status([a, b], 2, la.GRAD_BF16, HP, 3, flag=flag)


@host_only
def test_unknown_output_format():
    desc, keep = la.make_layer([fake_tensor(0)], 2, la.GRAD_BF16, 3)
    with pytest.raises(la.LayerAdamError) as e:
        la.step_raw(desc, la.make_params(**HP))
    assert e.value.status == 4


@host_only
@pytest.mark.parametrize("rng_", [(-1, 10), (5, 4), (0, 2049), (2049, 2049)])
def test_element_range_outside_the_layer(rng_):
    desc, keep = la.make_layer([fake_tensor(0, n=1024), fake_tensor(1, n=1024)], 2,
                               la.GRAD_BF16)
    with pytest.raises(la.LayerAdamError) as e:
        la.step_range_raw(desc, la.make_params(**HP), *rng_)
    assert e.value.status == 1


@host_only
@pytest.mark.parametrize("case", ["null", "misaligned", "on_master", "on_weight"])
def test_bad_skip_flag(case):
    t = fake_tensor(0)
    skip = {"null": 0, "misaligned": BASE + 0x50000002, "on_master": t["master"] + 128,
            "on_weight": t["weight_out"]}[case]
    desc, keep = la.make_layer([t], 2, la.GRAD_BF16)
    with pytest.raises(la.LayerAdamError) as e:
        la.step_gated_raw(desc, la.make_params(**HP), skip)
    assert e.value.status == {"null": 1, "misaligned": 2, "on_master": 3, "on_weight": 3}[case]


@host_only
@pytest.mark.parametrize("case", ["null", "misaligned", "on_grad", "unscale0", "null_grad"])
def test_bad_gradient_check(case):
    t = fake_tensor(0)
    flag, unscale = BASE + 0x50000000, 1.0
    if case == "null":
        flag = 0
    elif case == "misaligned":
        flag += 2
    elif case == "on_grad":
        flag = t["grads"][1] + 64
    elif case == "unscale0":
        unscale = 0.0
    elif case == "null_grad":
        t["grads"][0] = 0
    desc, keep = la.make_layer([t], 2, la.GRAD_BF16)
    with pytest.raises(la.LayerAdamError) as e:
        la.check_gradients_raw(desc, unscale, flag)
    assert e.value.status == {"null": 1, "misaligned": 2, "on_grad": 3, "unscale0": 1,
                              "null_grad": 1}[case]


@host_only
def test_buffers_a_mode_does_not_touch_are_not_required():
    # the gradient check reads gradients only; without a compute copy the
    # output pointer is ignored. Both pass validation and reach the (absent)
    # device here.
    t = fake_tensor(0)
    t.update(master=0, exp_avg=0, exp_avg_sq=0, weight_out=0)
    desc, keep = la.make_layer([t], 2, la.GRAD_BF16)
    with pytest.raises(la.LayerAdamError) as e:
        la.check_gradients_raw(desc, 1.0, BASE + 0x50000000)
    assert e.value.status == 5
    t = fake_tensor(0)
    t["weight_out"] = 0
    desc, keep = la.make_layer([t], 2, la.GRAD_BF16, la.OUT_NONE)
    with pytest.raises(la.LayerAdamError) as e:
        la.step_raw(desc, la.make_params(**HP))
    assert e.value.status == 5


@host_only
def test_too_many_tensors():
    expect_status([fake_tensor(k % 4, n=0) for k in range(la.MAX_TENSORS + 1)], 2,
                  la.GRAD_BF16, HP, 1)


@host_only
def test_negative_numel():
    t = fake_tensor(0)
    t["numel"] = -3
    expect_status([t], 2, la.GRAD_BF16, HP, 1)


def test_no_tensors_or_only_empty_tensors_enqueue_nothing():
    # nothing to launch: succeeds without touching the device
    desc, keep = la.make_layer([], 3, la.GRAD_BF16)
    la.step_raw(desc, la.make_params(**HP))
    desc, keep = la.make_layer([dict(numel=0), dict(numel=0)], 3, la.GRAD_FP16)
    la.step_raw(desc, la.make_params(**HP))
    assert la.last_error() == ""


@host_only
def test_error_messages_are_per_thread():
    import threading
    barrier = threading.Barrier(8)
    seen = {}

    def worker(k):
        lib = la.load()
        bad_r = k % 2 == 0
        desc, keep = la.make_layer([fake_tensor(0)], 0 if bad_r else 2, la.GRAD_BF16)
        hp = la.make_params(**dict(HP, step=1 if bad_r else 0))
        msgs = set()
        for _ in range(200):
            barrier.wait() if _ == 0 else None
            rc = lib.layer_adam_step(ctypes.byref(desc), ctypes.byref(hp), None, None)
            msgs.add((rc, lib.la_last_error().decode().split(",")[0]))
        seen[k] = msgs

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    for k, msgs in seen.items():
        assert len(msgs) == 1, msgs
        rc, msg = next(iter(msgs))
        assert rc == 1
        assert msg.startswith("num_replicas" if k % 2 == 0 else "step"), msg


@host_only
@pytest.mark.parametrize("case", ["null", "misaligned", "on_master"])
def test_bad_device_step_pointer(case):
    t = fake_tensor(0)
    step = {"null": 0, "misaligned": BASE + 0x50000004, "on_master": t["master"] + 64}[case]
    desc, keep = la.make_layer([t], 2, la.GRAD_BF16)
    with pytest.raises(la.LayerAdamError) as e:
        la.step_device_step_raw(desc, la.make_params(**HP), step)
    assert e.value.status == {"null": 1, "misaligned": 2, "on_master": 3}[case]


@host_only
def test_device_step_still_checks_the_other_hyperparameters():
    desc, keep = la.make_layer([fake_tensor(0)], 2, la.GRAD_BF16)
    with pytest.raises(la.LayerAdamError) as e:
        la.step_device_step_raw(desc, la.make_params(**dict(HP, beta2=1.5)), BASE + 0x50000000)
    assert e.value.status == 1


def test_binding_refuses_host_flags_and_step_counts_before_any_call():
    """Flags and the device step count must be device scalars of the right
    type; a host tensor is refused in the binding, before the library runs."""
    import torch
    with pytest.raises(TypeError):
        la._flag_ptr(torch.zeros(1, dtype=torch.int32))
    with pytest.raises(TypeError):
        la._step_ptr(torch.ones(1, dtype=torch.int64))


def test_binding_refuses_more_than_eight_replicas():
    import torch
    p = torch.zeros(8)
    grads = [[torch.zeros(8, dtype=torch.bfloat16)] * (la.MAX_REPLICAS + 1)]
    with pytest.raises(ValueError, match="at most 8"):
        la._describe([(p, p, p, None)], grads)


@host_only
def test_copy_reference_refusals():
    """Every call here is invalid (or empty), so nothing is ever enqueued."""
    lib = la.load()
    a, b = 0x7F0000000000, 0x7F0100000000
    cases = [(a, b, 24, 1), (a, b, -16, 1), (0, b, 1024, 1), (a, 0, 1024, 1),
             (a + 8, b, 1024, 2), (a, b + 4, 1024, 2), (a, a + 512, 1024, 3),
             (a + 1008, a, 1024, 3)]
    for dst, src, n, want in cases:
        rc = lib.la_copy_reference(ctypes.c_void_p(dst), ctypes.c_void_p(src), n, None)
        assert rc == want, (hex(dst), hex(src), n, rc, la.last_error())
        assert la.last_error()
    assert lib.la_copy_reference(ctypes.c_void_p(a), ctypes.c_void_p(b), 0, None) == 0


@host_only
@pytest.mark.parametrize("case", ["null_master", "null_grad", "misaligned_v", "m_on_master",
                                  "grad_on_copy", "bad_out", "R9"])
def test_stream_probe_refusals(case):
    """The stream probe checks its buffers as the update does (it writes
    master, m, v and the copy); nothing reaches the device on a refusal."""
    t, R, out = fake_tensor(0), 2, la.OUT_BF16
    if case == "null_master":
        t["master"] = 0
    elif case == "null_grad":
        t["grads"][1] = 0
    elif case == "misaligned_v":
        t["exp_avg_sq"] += 4
    elif case == "m_on_master":
        t["exp_avg"] = t["master"] + 256
    elif case == "grad_on_copy":
        t["grads"][0] = t["weight_out"] + 32
    elif case == "bad_out":
        out = 7
    elif case == "R9":
        R = 9
    desc, keep = la.make_layer([t], R, la.GRAD_BF16, out)
    with pytest.raises(la.LayerAdamError) as e:
        la.stream_probe_raw(desc)
    assert e.value.status == {"null_master": 1, "null_grad": 1, "misaligned_v": 2,
                              "m_on_master": 3, "grad_on_copy": 3, "bad_out": 4,
                              "R9": 1}[case]


def test_stream_probe_of_an_empty_layer_enqueues_nothing():
    desc, keep = la.make_layer([dict(numel=0)], 2, la.GRAD_BF16)
    la.stream_probe_raw(desc)
    assert la.last_error() == ""


@host_only
@pytest.mark.parametrize("case", ["bad_part", "wg_low", "wg_high", "range_past_end",
                                  "range_reversed", "range_negative", "null_master",
                                  "misaligned_m", "grad_on_v", "R0"])
def test_direction_probe_refusals(case):
    """The direction probe checks its buffers as the stream probe does, plus
    its part, residency and element range; nothing is enqueued on a refusal."""
    t, R = fake_tensor(0), 2
    part, lo, hi, wg = la.PROBE_READS, 0, t["numel"], -1
    if case == "bad_part":
        part = 2
    elif case == "wg_low":
        wg = -2
    elif case == "wg_high":
        wg = 65
    elif case == "range_past_end":
        hi = t["numel"] + 1
    elif case == "range_reversed":
        lo, hi = 8, 4
    elif case == "range_negative":
        lo = -1
    elif case == "null_master":
        t["master"] = 0
    elif case == "misaligned_m":
        t["exp_avg"] += 8
    elif case == "grad_on_v":
        t["grads"][1] = t["exp_avg_sq"] + 64
    elif case == "R0":
        R = 0
    desc, keep = la.make_layer([t], R, la.GRAD_BF16)
    with pytest.raises(la.LayerAdamError) as e:
        la.direction_probe_raw(desc, part, lo, hi, workgroups_per_cu=wg)
    assert e.value.status == {"null_master": 1, "misaligned_m": 2, "grad_on_v": 3}.get(case, 1)
    assert la.last_error()


@pytest.mark.parametrize("part", [0, 1])
def test_direction_probe_of_an_empty_layer_enqueues_nothing(part):
    desc, keep = la.make_layer([dict(numel=0)], 2, la.GRAD_BF16)
    la.direction_probe_raw(desc, part, 0, 0)
    assert la.last_error() == ""


@host_only
@pytest.mark.parametrize("part", [0, 1])
def test_direction_probe_of_an_empty_range_enqueues_nothing(part):
    """An empty range of a non-empty layer launches nothing, so it succeeds
    without a GPU."""
    desc, keep = la.make_layer([fake_tensor(0)], 2, la.GRAD_BF16)
    la.direction_probe_raw(desc, part, 40, 40)
    assert la.last_error() == ""


@host_only
@pytest.mark.parametrize("case", ["use_range_2", "range_past_end", "range_reversed",
                                  "skip_misaligned", "skip_on_master", "step_misaligned",
                                  "step_on_copy", "flag_misaligned", "bad_beta2_with_step",
                                  "no_hyperparameters"])
def test_step_ex_refusals(case):
    """layer_adam_step_ex checks each option as its own entry point does, plus
    use_range; nothing is enqueued on a refusal."""
    t = fake_tensor(0)
    desc, keep = la.make_layer([t], 2, la.GRAD_BF16)
    hp = la.make_params(**HP)
    opts = la.StepOptions(0, 0, 0, None, None, None)
    if case == "use_range_2":
        opts.use_range = 2
    elif case == "range_past_end":
        opts.use_range, opts.elem_begin, opts.elem_end = 1, 0, t["numel"] + 1
    elif case == "range_reversed":
        opts.use_range, opts.elem_begin, opts.elem_end = 1, 9, 8
    elif case == "skip_misaligned":
        opts.skip_if_nonzero = BASE + 0x50000002
    elif case == "skip_on_master":
        opts.skip_if_nonzero = t["master"] + 64
    elif case == "step_misaligned":
        opts.step_on_device = BASE + 0x50000004
    elif case == "step_on_copy":
        opts.step_on_device = t["weight_out"] + 16
    elif case == "flag_misaligned":
        opts.overflow_flag = BASE + 0x50000001
    elif case == "bad_beta2_with_step":
        opts.step_on_device = BASE + 0x50000000
        hp = la.make_params(**dict(HP, beta2=1.0))
    lib = la.load()
    rc = lib.layer_adam_step_ex(ctypes.byref(desc),
                                None if case == "no_hyperparameters" else ctypes.byref(hp),
                                ctypes.byref(opts), None)
    want = {"skip_misaligned": 2, "step_misaligned": 2, "flag_misaligned": 2,
            "skip_on_master": 3, "step_on_copy": 3}.get(case, 1)
    assert rc == want, (case, rc, la.last_error())
    assert la.last_error()


@host_only
def test_step_ex_defaults_and_empty_range_enqueue_nothing_when_refused_or_empty():
    """NULL options mean layer_adam_step (here refused for t = 0, the same
    message as layer_adam_step); an empty element range launches nothing."""
    desc, keep = la.make_layer([fake_tensor(0)], 2, la.GRAD_BF16)
    lib = la.load()
    bad = la.make_params(**dict(HP, step=0))
    assert lib.layer_adam_step_ex(ctypes.byref(desc), ctypes.byref(bad), None, None) == 1
    msg = la.last_error()
    assert lib.layer_adam_step(ctypes.byref(desc), ctypes.byref(bad), None, None) == 1
    assert la.last_error() == msg
    la.step_ex_raw(desc, la.make_params(**HP), 100, 100)
    assert la.last_error() == ""


def test_binding_step_ex_needs_both_range_ends_and_a_step():
    desc, keep = la.make_layer([dict(numel=0)], 2, la.GRAD_BF16)
    with pytest.raises(ValueError):
        la.step_ex_raw(desc, la.make_params(**HP), 0, None)
    with pytest.raises(ValueError):
        la._ex_params(1e-5, 0.9, 0.999, 1e-8, 0.0, None, 1.0, None)
