"""The C ABI from plain C (no Python, no torch in the process): build
tests/c/la_c_abi_check.c against include/layeradam.h and run it on the GPU;
it compares one layer_adam_step with the oracle element by element."""
import os
import subprocess
import tempfile

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_c_program_matches_the_oracle():
    libdirs = [os.path.join(ROOT, d) for d in ("optimizer_step_layeradam_amd", "oracle", "synth")]
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "la_c_abi_check")
        cmd = ["gcc", "-std=c11", "-O2", "-D__HIP_PLATFORM_AMD__",
               os.path.join(ROOT, "tests", "c", "la_c_abi_check.c"),
               "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"),
               "-I", os.path.join(ROCM, "include"), "-o", exe]
        cmd += [f"-L{p}" for p in libdirs] + [f"-Wl,-rpath,{p}" for p in libdirs]
        cmd += ["-llayeradam", "-lla_oracle", "-lla_synth", f"-L{ROCM}/lib", "-lamdhip64"]
        subprocess.run(cmd, check=True)
        r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
        print(r.stdout, r.stderr, flush=True)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "max 0 ulp" in r.stdout
