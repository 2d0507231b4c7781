"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

- The oracle built with -fsanitize=address,undefined runs its whole pin suite.
- The library's host side (argument checks, aliasing sort, range clipping),
  built with the sanitizers on the host pass only, runs every refusal path
  with made-up addresses. Every call is invalid by construction, so nothing
  is ever enqueued; the test is skipped where a GPU is visible.
"""
import os
import subprocess
import sys
import tempfile

import pytest
import torch

import oracle
from optimizer_step_layeradam_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _gcc_runtime(name):
    return subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True,
                          check=True).stdout.strip()


def test_oracle_pins_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "liboracle_san.so")
        subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                        "-fPIC", "-shared", "-fsanitize=address,undefined",
                        "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-o", lib,
                        os.path.join(ROOT, "oracle", "la_oracle.c"), "-lm"], check=True)
        env = dict(os.environ, LD_PRELOAD=f"{_gcc_runtime('libasan.so')} {_gcc_runtime('libubsan.so')}",
                   ASAN_OPTIONS="detect_leaks=0", LA_ORACLE_LIB_OVERRIDE=lib)
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                            os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
        assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


DRIVER = r'''
import ctypes, sys
sys.path.insert(0, ROOT)
import optimizer_step_layeradam_amd as la
lib = la.load(LIB)
BASE = 0x7F0000000000          # made up; never dereferenced

def fake(k, n=1024, R=2):
    b = BASE + k * 0x100000000
    return dict(master=b, exp_avg=b + 0x10000000, exp_avg_sq=b + 0x20000000,
                weight_out=b + 0x30000000,
                grads=[b + 0x40000000 + r * 0x1000000 for r in range(R)], numel=n)

hp = la.make_params(1e-5, 0.9, 0.999, 1e-8, 0.01, 1)
bad_hp = la.make_params(1e-5, 0.9, 0.999, 1e-8, 0.01, 0)
calls = 0

def refused(rc):
    global calls
    calls += 1
    assert rc not in (0, 5), (rc, lib.la_last_error())   # refused on the host
    assert lib.la_last_error()

for R in (0, 9):
    d, k = la.make_layer([fake(0)], R, 0)
    refused(lib.layer_adam_step(ctypes.byref(d), ctypes.byref(hp), None, None))
d, k = la.make_layer([fake(0)], 2, 0, 7)
refused(lib.layer_adam_step(ctypes.byref(d), ctypes.byref(hp), None, None))
d, k = la.make_layer([fake(0), fake(1)], 2, 0)
refused(lib.layer_adam_step(ctypes.byref(d), ctypes.byref(bad_hp), None, None))
for lo, hi in ((-1, 5), (7, 3), (0, 99999)):
    refused(lib.layer_adam_step_range(ctypes.byref(d), ctypes.byref(hp), lo, hi, None, None))
refused(lib.layer_adam_step_gated(ctypes.byref(d), ctypes.byref(hp), None, None, None))
refused(lib.layer_adam_step_device_step(ctypes.byref(d), ctypes.byref(hp),
                                        ctypes.c_void_p(BASE + 0x50000004), None, None))
refused(lib.la_check_gradients(ctypes.byref(d), 0.0, ctypes.c_void_p(BASE + 0x50000000), None))
# 256 tensors of every size class, disjoint except one overlap found only
# after sorting more than a thousand written ranges
many = []
for i in range(256):
    t = fake(i % 3, n=(i * 7919) % 3000)
    for key in ("master", "exp_avg", "exp_avg_sq", "weight_out"):
        t[key] += i * 0x10000
    many.append(t)
many[200]["exp_avg"] = many[17]["weight_out"] + 64 if many[17]["numel"] > 64 else many[17]["master"]
d, k = la.make_layer(many, 2, 0)
refused(lib.layer_adam_step(ctypes.byref(d), ctypes.byref(hp), None, None))
assert lib.la_state_bytes(ctypes.byref(d)) > 0 and lib.la_traffic_bytes(ctypes.byref(d)) > 0
# the combined entry point: bad use_range, range, misaligned skip and step
for o in (la.StepOptions(2, 0, 0, None, None, None), la.StepOptions(1, 5, 1 << 40, None, None, None),
          la.StepOptions(0, 0, 0, None, BASE + 0x50000002, None),
          la.StepOptions(0, 0, 0, None, None, BASE + 0x50000004)):
    refused(lib.layer_adam_step_ex(ctypes.byref(d), ctypes.byref(hp), ctypes.byref(o), None))
refused(lib.layer_adam_step_ex(ctypes.byref(d), ctypes.byref(bad_hp), None, None))
# the direction probe: bad part, residency and range
for part, lo, hi, wg in ((2, 0, 1024, -1), (0, 0, 1024, 65), (1, 0, 1024, -2), (0, 9, 3, -1),
                         (1, 0, 1 << 40, -1)):
    refused(lib.la_direction_probe(ctypes.byref(d), part, lo, hi, 0, wg, None))
# the reference copy: odd size, NULL, misaligned, overlapping
for dst, src, n in ((BASE, BASE + 0x10000000, 24), (0, BASE, 1024), (BASE + 8, BASE + 0x10000000, 1024),
                    (BASE, BASE + 512, 1024)):
    refused(lib.la_copy_reference(ctypes.c_void_p(dst), ctypes.c_void_p(src), n, None))
print("refusals", calls)
'''


@pytest.mark.skipif(torch.cuda.is_available(), reason="made-up device addresses; host-only")
def test_library_host_code_under_asan_and_ubsan():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    runtime = subprocess.run(["bash", "-c", f"ls {rocm}/lib/llvm/lib/clang/*/lib/linux/"
                              "libclang_rt.asan-x86_64.so | head -1"],
                             capture_output=True, text=True).stdout.strip()
    if not runtime:
        pytest.skip("clang ASan runtime not found")
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "liblayeradam_san.so")
        sanitize = ["-Xarch_host", "-fsanitize=address",
                    "-Xarch_host", "-fsanitize=undefined",
                    "-Xarch_host", "-fno-sanitize-recover=undefined",
                    "-Xarch_host", "-fno-omit-frame-pointer"]
        hip_build.build(out=lib, extra=["-O1", "-g"] + sanitize)
        script = os.path.join(d, "driver.py")
        with open(script, "w") as f:
            f.write(f"ROOT = {ROOT!r}\nLIB = {lib!r}\n" + DRIVER)
        env = dict(os.environ, LD_PRELOAD=runtime,
                   ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0")
        r = subprocess.run([sys.executable, script], env=env, capture_output=True, text=True,
                           timeout=300)
        assert r.returncode == 0 and "refusals" in r.stdout, r.stdout[-3000:] + r.stderr[-3000:]
