"""The pins must catch plausible mistakes in the oracle.

Each mutant is la_oracle.c with one deliberate slip (a transposed operand, a
flipped sign, a wrong bias-correction index, a dropped term, another rounding
or summation order, a wrong format constant). Every mutant is compiled on the
CPU and the pin suite (test_oracle_pins.py) is run against it in a
subprocess; the test passes only if every mutant fails at least one pin.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "la_oracle.c")

MUTANTS = {
    "m uses beta1 for the new term": ("s->c1 * g", "s->b1 * g"),
    "v uses g instead of g^2": ("s->c2 * g_squared", "s->c2 * g"),
    "v keeps beta1": ("s->b2 * v", "s->b1 * v"),
    "step sign flipped": ("p = decayed - step", "p = decayed + step"),
    "weight decay dropped": ("float decayed = p * s->d", "float decayed = p"),
    "decay coupled to lr twice": ("(float)(1.0 - lr * weight_decay)",
                                  "(float)(1.0 - lr * lr * weight_decay)"),
    "bias correction 1 at t+1": ("pow(beta1, t)", "pow(beta1, t + 1.0)"),
    "bias correction 2 at t-1": ("pow(beta2, t)", "pow(beta2, t - 1.0)"),
    "bias correction 2 without sqrt": ("(float)sqrt(bias_correction2)",
                                       "(float)bias_correction2"),
    "bias correction 1 dropped": ("(float)(lr / bias_correction1)", "(float)lr"),
    "eps inside the sqrt": ("float root = sqrtf(v);", "float root = sqrtf(v + s->e);"),
    "eps dropped": ("float denominator = root_corrected + s->e;",
                    "float denominator = root_corrected;"),
    "ratio transposed": ("float ratio = m / denominator;",
                         "float ratio = denominator / m;"),
    "old moment used in the step": ("float ratio = m / denominator;",
                                    "float ratio = *exp_avg / denominator;"),
    "unscale dropped": ("  g = g * u;\n", "\n"),
    "unscale divides": ("  g = g * u;\n", "  g = g / u;\n"),
    "summation starts from the last replica": (
        "float g = lao_decode(grad[0][j], dtype);\n  for (int r = 1; r < replicas; ++r) {\n    float next = lao_decode(grad[r][j], dtype);",
        "float g = lao_decode(grad[replicas - 1][j], dtype);\n  for (int r = replicas - 2; r >= 0; --r) {\n    float next = lao_decode(grad[r][j], dtype);"),
    "last replica skipped": ("for (int r = 1; r < replicas; ++r)",
                             "for (int r = 1; r < replicas - 1; ++r)"),
    "cast truncates": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;",
                       ""),
    "cast ties away from zero": ("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)"),
    "cast NaN not canonical": ("if (isnan(x)) return 0x7FC0;", ""),
    "fp16 exponent bias off by one": ("exponent - 25", "exponent - 24"),
    "fp16 subnormal scale wrong": ("ldexpf((float)fraction, -24)", "ldexpf((float)fraction, -25)"),
    "flag never raised": ("if (flag != NULL && !isfinite(g)) *flag = 1;", ""),
    "fp16 cast truncates": ("double significand = nearbyint(ldexp(a, 10 - unbiased));",
                            "double significand = floor(ldexp(a, 10 - unbiased));"),
    "fp16 cast overflows one binade late": ("if (biased >= 31) return sign | 0x7C00;",
                                            "if (biased > 31) return sign | 0x7C00;"),
    "fp16 subnormals flushed": ("double units = nearbyint(ldexp(a, 24));", "double units = 0.0;"),
    "gradient check ignores the unscale": ("  float u = (float)unscale;\n  int found = 0;",
                                           "  float u = 1.0f;\n  int found = 0;"),
    "gradient check misses NaN": ("if (!isfinite(g)) found = 1;", "if (isinf(g)) found = 1;"),
    "fp16 copy takes the bf16 cast": ("*weight_out = lao_round_fp16(p);",
                                      "*weight_out = lao_round_bf16(p);"),
    "copy cast before the step": ("if (out_dtype == LAO_OUT_BF16) *weight_out = lao_round_bf16(p);",
                                  "if (out_dtype == LAO_OUT_BF16) *weight_out = lao_round_bf16(decayed);"),
    "L2 decay instead of decoupled": (
        "float g = lao_aggregate(x->grad, replicas, dtype, j, s.u);",
        "float g = lao_aggregate(x->grad, replicas, dtype, j, s.u) + (float)weight_decay * x->master[j];"),
}


def _build_mutant(name, old, new, outdir):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutant {name!r}: anchor not found exactly once"
    path = os.path.join(outdir, f"m{abs(hash(name)) % 10**8}.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = path[:-2] + ".so"
    subprocess.run(["gcc", *oracle.CFLAGS, "-I", os.path.dirname(SRC), "-o", lib, path, "-lm"],
                   check=True, capture_output=True)
    return lib


def _pins_fail(lib):
    env = dict(os.environ, LA_ORACLE_LIB_OVERRIDE=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode != 0


def test_every_mutant_is_caught():
    with tempfile.TemporaryDirectory() as d:
        libs = {n: _build_mutant(n, o, w, d) for n, (o, w) in MUTANTS.items()}
        with ThreadPoolExecutor(max_workers=max(1, min(8, os.cpu_count() or 1))) as ex:
            caught = dict(zip(libs, ex.map(_pins_fail, libs.values())))
    survivors = [n for n, c in caught.items() if not c]
    assert not survivors, f"mutants not caught by any pin: {survivors}"


def test_unmutated_oracle_passes_the_pins_through_the_override():
    with tempfile.TemporaryDirectory() as d:
        lib = os.path.join(d, "same.so")
        subprocess.run(["gcc", *oracle.CFLAGS, "-o", lib, SRC, "-lm"], check=True)
        assert not _pins_fail(lib)
