"""The library's own gfx950 build, inspected on the host (hipcc cross-compiles
the device code; nothing runs): what the parity tests rely on, and what the
update's design claims about its instructions, checked in the compiler's
output.

- No packed FP32 instructions (the build switches the feature off).
- No contraction: the device IR of the update and check kernels holds plain
  fadd/fmul/fdiv and sqrt with no fast-math flags and no fused multiply-add
  in single precision (the double-precision fma of the device step's pow
  aside, which only its own instantiations carry).
- IEEE single-precision mode: denormals kept on input and output, round to
  nearest even.
- No scratch memory (no register spills) in any kernel.
- The default update kernels and the stream probe carry no double-precision
  instruction: the device step's pow is compiled only into its own mode.
- Every 16-byte load of the update, the probes and the copy is a
  non-temporal buffer load, every 16-byte store a buffer store written
  through to memory (sc0 sc1 nt).
"""
import os
import re
import subprocess
import tempfile

import pytest

from optimizer_step_layeradam_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "optimizer_step_layeradam_amd", "csrc")
FLAGS = [f for f in hip_build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
UPDATE = re.compile(r"layer_adam_kernelILi(\d)ELb([01])ELb([01])ELi(\d)ELi(\d)E")


def _compile(src, out, ir=False):
    cmd = [hip_build.hipcc(), *FLAGS, "--cuda-device-only", "-S", "-I",
           os.path.join(ROOT, "include"), "-I", CSRC, "-o", out, os.path.join(CSRC, src)]
    if ir:
        cmd.insert(-3, "-emit-llvm")
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)


@pytest.fixture(scope="module")
def build_outputs():
    with tempfile.TemporaryDirectory() as d:
        jobs = {"kernel_s": ("la_kernel.hip", os.path.join(d, "k.s"), False),
                "kernel_ll": ("la_kernel.hip", os.path.join(d, "k.ll"), True),
                "copy_s": ("la_copy.hip", os.path.join(d, "c.s"), False)}
        procs = {k: _compile(*v) for k, v in jobs.items()}
        out = {}
        for k, p in procs.items():
            log, _ = p.communicate(timeout=600)
            assert p.returncode == 0, log[-3000:]
            with open(jobs[k][1]) as f:
                out[k] = f.read()
        yield out


def asm_functions(text):
    """{mangled kernel name: its instructions} from an assembly listing."""
    funcs, name, body = {}, None, []
    for line in text.splitlines():
        m = re.match(r"^(_Z\S+):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name and line.startswith(".Lfunc_end"):
            funcs[name] = "\n".join(body)
            name = None
            continue
        if name:
            body.append(line)
    return funcs


def kernel_descriptors(text):
    """{kernel name: {amdhsa field: value}} from the .amdhsa_kernel blocks."""
    out = {}
    for m in re.finditer(r"\.amdhsa_kernel (\S+)\n(.*?)\.end_amdhsa_kernel", text, re.S):
        out[m.group(1)] = dict(re.findall(r"\.(amdhsa_\w+) (\S+)", m.group(2)))
    return out


def ir_functions(text):
    return {m.group(1): m.group(2) for m in
            re.finditer(r"^define [^@]*@(\S+)\(.*?\{\n(.*?)^\}", text, re.M | re.S)}


def test_every_kernel_was_found(build_outputs):
    k = asm_functions(build_outputs["kernel_s"])
    c = asm_functions(build_outputs["copy_s"])
    updates = [n for n in k if UPDATE.search(n)]
    # R = 1..8 x gradient format x flag x copy format x {host, device step}, plus the probes
    assert len([n for n in updates if UPDATE.search(n).group(5) in "01"]) == 8 * 2 * 2 * 3 * 2
    assert len([n for n in updates if UPDATE.search(n).group(5) == "2"]) == 8 * 2
    assert len([n for n in k if "check_kernel" in n]) == 16
    assert len([n for n in c if "direction_kernel" in n]) == 9
    assert len([n for n in c if "copy_kernel" in n]) == 1


def test_no_packed_fp32_instructions(build_outputs):
    for key in ("kernel_s", "copy_s"):
        found = re.findall(r"\bv_pk_(?:add|mul|fma)_f32\b", build_outputs[key])
        assert not found, (key, found[:5])


def test_no_contraction_or_fast_math_in_single_precision(build_outputs):
    funcs = ir_functions(build_outputs["kernel_ll"])
    assert funcs
    for name, body in funcs.items():
        assert "llvm.fmuladd" not in body, name
        assert "llvm.fma.f32" not in body, name
        flagged = re.findall(r"= (?:fadd|fsub|fmul|fdiv|call) (?:[a-z]+ )*(?:contract|fast|afn|arcp|"
                             r"reassoc|nnan|ninf|nsz)\b", body)
        assert not flagged, (name, flagged[:3])
        assert "!fpmath" not in body, name
        m = UPDATE.search(name)
        if "llvm.fma.f64" in body:
            assert m and m.group(5) == "1", f"double fma outside the device-step mode: {name}"
    # the update's arithmetic is there, correctly rounded: fdiv and sqrt, no approximations
    body = funcs[next(n for n in funcs if UPDATE.search(n) and UPDATE.search(n).group(5) == "0")]
    assert "fdiv float" in body and "llvm.sqrt.f32" in body
    assert "llvm.amdgcn.rcp" not in body and "llvm.amdgcn.rsq" not in body


def test_ieee_single_precision_mode_and_no_scratch(build_outputs):
    for key in ("kernel_s", "copy_s"):
        descs = kernel_descriptors(build_outputs[key])
        assert descs
        for name, d in descs.items():
            assert d["amdhsa_private_segment_fixed_size"] == "0", name   # no spills
            assert d["amdhsa_float_denorm_mode_32"] == "3", name         # denormals kept
            assert d["amdhsa_float_round_mode_32"] == "0", name          # nearest even
            assert d["amdhsa_ieee_mode"] == "1", name


def test_default_update_and_probe_carry_no_double_precision(build_outputs):
    for name, body in asm_functions(build_outputs["kernel_s"]).items():
        m = UPDATE.search(name)
        if m and m.group(5) in "02":
            f64 = re.findall(r"\bv_\w+_f64\b", body)
            assert not f64, (name, f64[:5])
        if m and m.group(5) == "1":
            assert re.search(r"\bv_\w+_f64\b", body), name  # the device step's pow is there


def test_streaming_loads_and_written_through_stores(build_outputs):
    funcs = {**asm_functions(build_outputs["kernel_s"]), **asm_functions(build_outputs["copy_s"])}
    for name, body in funcs.items():
        if "check_kernel" in name:
            continue  # the finite check reads with non-temporal global loads
        loads = [l for l in body.splitlines() if re.search(r"\b(buffer|global)_load_dwordx4\b", l)]
        stores = [l for l in body.splitlines() if re.search(r"\b(buffer|global)_store_dwordx4\b", l)]
        if UPDATE.search(name) or "direction_kernel" in name:
            assert all(l.split()[0] == "buffer_load_dwordx4" for l in loads), name
        for l in loads:
            assert re.search(r"\bnt\b", l), (name, l)
        for l in stores:
            assert l.split()[0] == "buffer_store_dwordx4", (name, l)
            assert re.search(r"\bsc0\b", l) and re.search(r"\bsc1\b", l) and \
                re.search(r"\bnt\b", l), (name, l)
        m = UPDATE.search(name)
        if m:
            # master, m, v: three 16-byte loads and (unless probe/no copy aside) stores
            assert len(loads) >= 3 and len(stores) >= 3, name
