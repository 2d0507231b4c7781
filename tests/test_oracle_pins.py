"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against a definition of a number format, a
library routine (numpy, torch), a closed form, an invariant of exact
arithmetic, or an error bound against a float64 evaluation, chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign, a wrong index of
the bias correction, a transposed operand, a different summation order)
fails at least one of them. No GPU is involved.
"""
import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

F32_EPS = 2.0 ** -24  # unit roundoff of binary32


def ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


def bf16_value(bits):
    """Value of BF16 bit patterns by the format's definition (float64)."""
    bits = np.asarray(bits, np.int64)
    s = (bits >> 15) & 1
    e = (bits >> 7) & 0xFF
    f = (bits & 0x7F).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(f, -133), np.ldexp(128.0 + f, (e - 134).astype(np.int64)))
    mag = np.where(e == 255, np.where(f == 0, np.inf, np.nan), mag)
    return np.where(s == 1, -mag, mag)


def bits_f32(x):
    return np.asarray(x, np.float32).view(np.uint32)


def f32_from_bits(b):
    return np.asarray(b, np.uint32).view(np.float32)


def torch_bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def make_tensor(p, m, v, grads):
    n = p.size
    return oracle.Tensor(np.array(p, np.float32), np.array(m, np.float32),
                         np.array(v, np.float32), np.zeros(n, np.uint16),
                         [np.ascontiguousarray(g, np.uint16) for g in grads])


def random_bf16(rng, n, scale=1e-3):
    x = (rng.standard_normal(n) * scale).astype(np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


HP = dict(lr=1e-5, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------
def test_decode_bf16_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(bits, "bf16").astype(np.float64)
    want = bf16_value(bits)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(want[~nan]))
    # library routine: torch's bfloat16 -> float32
    lib = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(bits_f32(got.astype(np.float32))[~nan], bits_f32(lib)[~nan])


def test_decode_fp16_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    got = oracle.decode(bits, "fp16")
    lib = bits.view(np.float16).astype(np.float32)  # numpy's exact widening
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(bits_f32(got)[~nan], bits_f32(lib)[~nan])
    # subnormal binary16 survive (smallest is 2^-24)
    assert got[1] == 2.0 ** -24 and got[0x03FF] == 1023 * 2.0 ** -24


def _nearest_bf16_reference(x32):
    """BF16 nearest to x by comparing real distances (float64 is exact here),
    ties to the even pattern; beyond the largest finite the next pattern up is
    Inf, taken at magnitude 2^128 as IEEE overflow rounding prescribes."""
    x = x32.astype(np.float64)
    lo = (bits_f32(x32) >> 16).astype(np.int64)
    hi = lo + 1
    lo_v = bf16_value(lo)
    hi_mag = np.where((hi & 0x7FFF) == 0x7F80, 2.0 ** 128, np.abs(bf16_value(hi)))
    hi_v = np.where(x < 0, -hi_mag, hi_mag)
    d_lo = np.abs(x - lo_v)
    d_hi = np.abs(hi_v - x)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    out = np.where(pick_hi, hi, lo)
    out = np.where(np.isinf(x), lo, out)
    return out.astype(np.uint16)


def _structured_f32_patterns():
    highs = np.arange(65536, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x3FFF, 0x4000, 0x7FFE, 0x7FFF, 0x8000,
                     0x8001, 0xBFFF, 0xC000, 0xFFFE, 0xFFFF, 0x1234, 0x9ABC],
                    dtype=np.uint32)
    return (highs[:, None] | lows[None, :]).ravel()


def test_round_bf16_against_nearest_value_definition():
    rng = np.random.default_rng(7)
    pats = np.concatenate([_structured_f32_patterns(),
                           rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32)])
    x = f32_from_bits(pats)
    got = oracle.round_bf16(x)
    nan = np.isnan(x)
    assert np.all(got[nan] == 0x7FC0)
    want = _nearest_bf16_reference(x[~nan])
    bad = np.nonzero(got[~nan] != want)[0]
    assert bad.size == 0, f"first mismatch at pattern {hex(int(pats[~nan][bad[0]]))}"
    # library routine: torch's float32 -> bfloat16 (round to nearest even)
    assert np.array_equal(got[~nan], torch_bf16_bits(x[~nan]))


def test_round_bf16_special_values():
    cases = [
        (0.0, 0x0000), (-0.0, 0x8000), (1.0, 0x3F80), (float("inf"), 0x7F80),
        (float("-inf"), 0xFF80),
        # largest finite float32 lies above the midpoint past 0x7F7F
        (float(np.finfo(np.float32).max), 0x7F80),
        (-float(np.finfo(np.float32).max), 0xFF80),
    ]
    for x, want in cases:
        assert oracle.round_bf16(np.array([x], np.float32))[0] == want
    # exactly half way between 1.0 (even) and the next BF16: stays at 1.0
    assert oracle.round_bf16(f32_from_bits(np.array([0x3F808000], np.uint32)))[0] == 0x3F80
    # half way between 0x3F81 (odd) and 0x3F82: goes to the even one
    assert oracle.round_bf16(f32_from_bits(np.array([0x3F818000], np.uint32)))[0] == 0x3F82


def test_round_fp16_against_numpy():
    """numpy's float32 -> float16 is IEEE round-to-nearest-even with
    subnormals and overflow to Inf."""
    rng = np.random.default_rng(17)
    pats = np.concatenate([_structured_f32_patterns(),
                           rng.integers(0, 2 ** 32, 4_000_000, dtype=np.uint64).astype(np.uint32)])
    x = f32_from_bits(pats)
    got = oracle.round_fp16(x)
    nan = np.isnan(x)
    assert np.all(got[nan] == 0x7E00)
    with np.errstate(over="ignore"):
        lib = x[~nan].astype(np.float16).view(np.uint16)
    bad = np.nonzero(got[~nan] != lib)[0]
    assert bad.size == 0, f"first mismatch at pattern {hex(int(pats[~nan][bad[0]]))}"


def test_round_fp16_special_values():
    cases = [(1.0, 0x3C00), (-2.0, 0xC000), (65504.0, 0x7BFF), (65519.99, 0x7BFF),
             (65520.0, 0x7C00), (-65520.0, 0xFC00), (2.0 ** -24, 0x0001),
             (2.0 ** -25, 0x0000),            # tie between 0 and 2^-24: even
             (3 * 2.0 ** -25, 0x0002),        # tie between 1 and 2 units: even
             (2.0 ** -14, 0x0400), (float("inf"), 0x7C00), (-0.0, 0x8000),
             (1.0 + 2.0 ** -11, 0x3C00),      # tie: even significand
             (1.0 + 3 * 2.0 ** -11, 0x3C02)]  # tie: even significand
    for x, want in cases:
        assert oracle.round_fp16(np.array([x], np.float32))[0] == want, x


# --------------------------------------------------------------------------
# Aggregation of the R replicas
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("R", range(1, 9))
def test_identical_replicas_sum_exactly_to_R_times_g(R, dtype):
    rng = np.random.default_rng(R)
    if dtype == "bf16":
        g = random_bf16(rng, 4096, scale=1.0)
    else:
        g = np.asarray(rng.standard_normal(4096) * 100, np.float16).view(np.uint16)
    dec = (oracle.decode(g, dtype).astype(np.float64))
    got = oracle.aggregate([g] * R, dtype, 1.0)
    # an 8- or 11-bit significand times R <= 8 fits in binary32 exactly
    assert np.array_equal(got.astype(np.float64), R * dec)
    # and equals one replica with unscale R
    assert np.array_equal(got, oracle.aggregate([g], dtype, float(R)))


def test_aggregation_is_a_left_fold_in_replica_order():
    one = np.array([0x3F80], np.uint16)            # 1.0
    tiny = np.array([(127 - 24) << 7], np.uint16)  # 2^-24
    # (1 + 2^-24) + 2^-24 rounds to 1 twice; any other order gives 1 + 2^-23
    assert oracle.aggregate([one, tiny, tiny], "bf16")[0] == np.float32(1.0)
    assert oracle.aggregate([tiny, tiny, one], "bf16")[0] == np.float32(1.0 + 2.0 ** -23)


@pytest.mark.parametrize("R", [2, 3, 5, 8])
def test_aggregation_error_bound(R):
    rng = np.random.default_rng(100 + R)
    grads = []
    for _ in range(R):
        x = rng.standard_normal(20000) * 1e-3
        x = np.where(rng.random(20000) < 0.01, x * 100, x).astype(np.float32)
        grads.append((x.view(np.uint32) >> 16).astype(np.uint16))
    vals = np.stack([bf16_value(g) for g in grads])
    exact = vals.sum(axis=0)
    got = oracle.aggregate(grads, "bf16").astype(np.float64)
    bound = (R - 1) * F32_EPS * np.abs(vals).sum(axis=0)
    assert np.all(np.abs(got - exact) <= bound)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_power_of_two_unscale_is_invisible(dtype):
    """oracle(G * 2^10, u = 2^-10) equals oracle(G, u = 1) bit for bit when the
    scaled gradients stay normal: the unscale multiplies the aggregated
    gradient and nothing else."""
    rng = np.random.default_rng(3)
    n, R = 5000, 3
    if dtype == "fp16":
        exp = rng.integers(1, 21, (R, n))
        G = ((rng.integers(0, 2, (R, n)) << 15) | (exp << 10) | rng.integers(0, 1024, (R, n)))
        G_scaled = G + (10 << 10)
    else:
        exp = rng.integers(60, 120, (R, n))
        G = ((rng.integers(0, 2, (R, n)) << 15) | (exp << 7) | rng.integers(0, 128, (R, n)))
        G_scaled = G + (10 << 7)
    G = G.astype(np.uint16)
    G_scaled = G_scaled.astype(np.uint16)
    p = rng.standard_normal(n).astype(np.float32) * 0.02
    m = rng.standard_normal(n).astype(np.float32) * 1e-4
    v = rng.random(n).astype(np.float32) * 1e-6
    a = make_tensor(p, m, v, list(G))
    b = make_tensor(p, m, v, list(G_scaled))
    oracle.step([a], dtype=dtype, step=7, unscale=1.0, **HP)
    oracle.step([b], dtype=dtype, step=7, unscale=2.0 ** -10, **HP)
    for f in ("master", "exp_avg", "exp_avg_sq", "weight_out"):
        assert np.array_equal(getattr(a, f).view(np.uint8), getattr(b, f).view(np.uint8)), f


# --------------------------------------------------------------------------
# The update: closed forms
# --------------------------------------------------------------------------
def test_zero_gradient_gives_decay_only():
    rng = np.random.default_rng(11)
    n = 10000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    zeros = np.where(rng.random(n) < 0.5, 0x0000, 0x8000).astype(np.uint16)  # +0 / -0
    hp = dict(HP, lr=1e-3, weight_decay=0.1)
    for t in (1, 2, 1000):
        x = make_tensor(p, np.zeros(n), np.zeros(n), [zeros, zeros])
        oracle.step([x], dtype="bf16", step=t, **hp)
        assert np.all(x.exp_avg == 0) and np.all(x.exp_avg_sq == 0)
        d = np.float32(1.0 - hp["lr"] * hp["weight_decay"])
        assert np.array_equal(x.master, p * d)  # one FP32 product
        real = p.astype(np.float64) * (1.0 - hp["lr"] * hp["weight_decay"])
        assert np.all(np.abs(x.master - real) <= ulp32(real) + np.abs(real) * F32_EPS)


def test_zero_learning_rate_keeps_master_and_still_moves_moments():
    rng = np.random.default_rng(12)
    n = 4096
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32)
    g = random_bf16(rng, n)
    x = make_tensor(p, m, v, [g])
    oracle.step([x], dtype="bf16", step=5, **dict(HP, lr=0.0))
    assert np.array_equal(x.master, p)
    assert np.array_equal(x.weight_out, torch_bf16_bits(p))
    assert np.mean(x.exp_avg != m) > 0.99 and np.mean(x.exp_avg_sq != v) > 0.99


def test_first_step_from_zero_moments_is_lr_times_sign():
    """At t = 1 with m = v = 0 the bias corrections cancel: m_hat = g,
    v_hat = g^2, so p' = p*(1 - lr*wd) - lr*g/(|g| + eps) ~ -lr*sign(g)."""
    rng = np.random.default_rng(13)
    n = 50000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    g = random_bf16(rng, n)
    gv = bf16_value(g)
    keep = np.abs(gv) > 1e-6
    lr, wd, eps = 1e-3, 0.01, 1e-8
    x = make_tensor(p, np.zeros(n), np.zeros(n), [g])
    oracle.step([x], dtype="bf16", step=1, **dict(HP, lr=lr, weight_decay=wd))
    delta = x.master.astype(np.float64) - p.astype(np.float64) * (1 - lr * wd)
    tol = lr * (eps / np.abs(gv) + 2.0 ** -20) + 2 * ulp32(p) + np.abs(p) * F32_EPS
    assert np.all(np.abs(delta + lr * np.sign(gv))[keep] <= tol[keep])
    assert np.all(np.sign(delta[keep]) == -np.sign(gv[keep]))


def test_constant_gradient_steps_are_lr_times_sign_at_every_t():
    """With a constant g from zero moments, m_hat_t = g and v_hat_t = g^2 at
    every step t in exact arithmetic, so every step moves p by ~lr; a wrong
    index in either bias correction breaks this from t = 2 on."""
    rng = np.random.default_rng(14)
    n = 4096
    g = random_bf16(rng, n)
    gv = bf16_value(g)
    keep = np.abs(gv) > 1e-5
    lr, wd, eps = 1e-3, 0.0, 1e-8
    x = make_tensor((rng.standard_normal(n) * 0.02).astype(np.float32),
                    np.zeros(n), np.zeros(n), [g])
    for t in range(1, 31):
        before = x.master.astype(np.float64)
        oracle.step([x], dtype="bf16", step=t, **dict(HP, lr=lr, weight_decay=wd))
        delta = x.master.astype(np.float64) - before
        tol = lr * (eps / np.abs(gv) + 1e-5) + 2 * ulp32(before)
        assert np.all(np.abs(delta + lr * np.sign(gv))[keep] <= tol[keep]), t


# --------------------------------------------------------------------------
# The update: library routine and float64 brute force
# --------------------------------------------------------------------------
@pytest.mark.parametrize("t0", [1, 10, 1000])
def test_matches_torch_adamw_single_tensor(t0):
    """R = 1, u = 1: torch.optim.AdamW (single-tensor CPU FP32 path). torch
    orders a few FP32 operations differently (lerp for m, (c2*g)*g for v), so
    agreement is to a few roundings of the terms, not bitwise."""
    rng = np.random.default_rng(t0)
    n = 30000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32)
    x = make_tensor(p, m, v, [random_bf16(rng, n)])
    param = torch.nn.Parameter(torch.from_numpy(p.copy()))
    opt = torch.optim.AdamW([param], lr=HP["lr"], betas=(HP["beta1"], HP["beta2"]),
                            eps=HP["eps"], weight_decay=HP["weight_decay"],
                            foreach=False, fused=False)
    for t in range(t0, t0 + 3):
        g = random_bf16(rng, n)
        x.grads = [g]
        m_old, v_old, p_old = x.exp_avg.copy(), x.exp_avg_sq.copy(), x.master.copy()
        with torch.no_grad():
            param.copy_(torch.from_numpy(p_old))
        opt.state[param] = {"step": torch.tensor(float(t - 1)),
                            "exp_avg": torch.from_numpy(m_old.copy()),
                            "exp_avg_sq": torch.from_numpy(v_old.copy())}
        gf = oracle.decode(g, "bf16")
        param.grad = torch.from_numpy(gf.copy())
        opt.step()
        oracle.step([x], dtype="bf16", step=t, **HP)
        tm = opt.state[param]["exp_avg"].numpy().astype(np.float64)
        tv = opt.state[param]["exp_avg_sq"].numpy().astype(np.float64)
        tp = param.detach().numpy().astype(np.float64)
        gd = gf.astype(np.float64)
        tol_m = 8 * F32_EPS * (np.abs(m_old) + 0.1 * np.abs(gd) + np.abs(gd - m_old) * 0.1)
        tol_v = 8 * F32_EPS * (np.abs(v_old) + 1e-3 * gd * gd)
        assert np.all(np.abs(x.exp_avg - tm) <= tol_m)
        assert np.all(np.abs(x.exp_avg_sq - tv) <= tol_v)
        alpha = HP["lr"] / (1 - HP["beta1"] ** t)
        den = np.sqrt(tv) / math.sqrt(1 - HP["beta2"] ** t) + HP["eps"]
        tol_p = 2 * ulp32(tp) + alpha * (tol_m / den + np.abs(tm / den) * 1e-5)
        assert np.all(np.abs(x.master - tp) <= tol_p)


def _adamw_float64(p, m, v, grads, t, lr, beta1, beta2, eps, weight_decay, unscale):
    g = sum(grads) * unscale
    m1 = beta1 * m + (1 - beta1) * g
    v1 = beta2 * v + (1 - beta2) * g * g
    den = np.sqrt(v1) / math.sqrt(1 - beta2 ** t) + eps
    p1 = p * (1 - lr * weight_decay) - lr / (1 - beta1 ** t) * m1 / den
    return p1, m1, v1, g, den


@pytest.mark.parametrize("case", range(6))
def test_within_fp32_rounding_of_exact_adamw(case):
    """Brute force: the same inputs through AdamW in float64; the FP32 oracle
    must sit within a few roundings of each term."""
    rng = np.random.default_rng(1000 + case)
    n = 20000
    R = 1 + case % 4
    t = [1, 2, 10, 100, 1000, 12345][case]
    hp = dict(lr=[1e-5, 1e-3, 3e-4, 1e-5, 2e-5, 1e-4][case], beta1=[0.9, 0.8, 0.95, 0.9, 0.0, 0.5][case],
              beta2=[0.999, 0.99, 0.95, 0.9999, 0.999, 0.0][case], eps=[1e-8, 1e-6, 1e-8, 0.0, 1e-8, 1e-3][case],
              weight_decay=[0.01, 0.1, 0.0, 0.05, 1.0, 0.01][case])
    unscale = [1.0, 0.5, 1.0 / 3.0, 1.0, 2.0, 0.125][case]
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32) + 1e-12
    grads = [random_bf16(rng, n) for _ in range(R)]
    x = make_tensor(p, m, v, grads)
    oracle.step([x], dtype="bf16", step=t, unscale=unscale, **hp)
    gv = [bf16_value(g) for g in grads]
    p1, m1, v1, g, den = _adamw_float64(p.astype(np.float64), m.astype(np.float64),
                                        v.astype(np.float64), gv, t, unscale=unscale, **hp)
    gabs = (sum(np.abs(a) for a in gv)) * unscale
    k = 16 * F32_EPS
    tm = k * (hp["beta1"] * np.abs(m) + (1 - hp["beta1"]) * gabs)
    tv = k * (hp["beta2"] * v + (1 - hp["beta2"]) * gabs * gabs)
    assert np.all(np.abs(x.exp_avg - m1) <= tm)
    assert np.all(np.abs(x.exp_avg_sq - v1) <= tv)
    alpha = hp["lr"] / (1 - hp["beta1"] ** t)
    tp = k * np.abs(p) + alpha * (tm / den + k * np.abs(m1 / den) + np.abs(m1) * tv / (2 * den * den * np.sqrt(v1) * math.sqrt(1 - hp["beta2"] ** t) + 1e-300))
    assert np.all(np.abs(x.master - p1) <= tp + ulp32(p1))


# --------------------------------------------------------------------------
# Overflow flag and propagation
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("bad", ["+inf", "-inf", "nan"])
def test_flag_and_propagation_of_non_finite_gradients(dtype, bad):
    rng = np.random.default_rng(5)
    n, R = 1000, 3
    codes = {"bf16": {"+inf": 0x7F80, "-inf": 0xFF80, "nan": 0x7FC1},
             "fp16": {"+inf": 0x7C00, "-inf": 0xFC00, "nan": 0x7E01}}[dtype]
    if dtype == "bf16":
        grads = [random_bf16(rng, n) for _ in range(R)]
    else:
        grads = [np.asarray(rng.standard_normal(n), np.float16).view(np.uint16) for _ in range(R)]
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    clean = make_tensor(p, np.zeros(n), np.zeros(n), grads)
    assert oracle.step([clean], dtype=dtype, step=1, with_flag=True, **HP) == 0
    hit = [0, n - 1, 517]
    for j, r in zip(hit, [0, R - 1, 1]):
        grads[r] = grads[r].copy()
        grads[r][j] = codes[bad]
    x = make_tensor(p, np.zeros(n), np.zeros(n), grads)
    assert oracle.step([x], dtype=dtype, step=1, with_flag=True, **HP) == 1
    others = np.setdiff1d(np.arange(n), hit)
    assert np.all(np.isnan(x.master[hit])) and np.all(x.weight_out[hit] == 0x7FC0)
    if bad == "nan":
        assert np.all(np.isnan(x.exp_avg[hit]))
    else:
        assert np.all(np.isinf(x.exp_avg[hit])) and np.all(np.isinf(x.exp_avg_sq[hit]))
    for f in ("master", "exp_avg", "exp_avg_sq", "weight_out"):
        assert np.array_equal(getattr(x, f)[others], getattr(clean, f)[others])


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_gradient_check_finds_exactly_the_non_finite_aggregates(dtype):
    rng = np.random.default_rng(21)
    n, R = 3000, 3
    big = {"bf16": 0x7F7F, "fp16": 0x7BFF}[dtype]      # largest finite
    inf = {"bf16": 0x7F80, "fp16": 0x7C00}[dtype]
    ninf = {"bf16": 0xFF80, "fp16": 0xFC00}[dtype]
    nan = {"bf16": 0x7FC1, "fp16": 0x7E01}[dtype]
    base = [random_bf16(rng, n) if dtype == "bf16" else
            np.asarray(rng.standard_normal(n), np.float16).view(np.uint16) for _ in range(R)]
    x = make_tensor(np.zeros(n), np.zeros(n), np.zeros(n), base)
    assert oracle.check_finite([x], dtype=dtype) == 0
    for code in (inf, ninf, nan):
        g = [b.copy() for b in base]
        g[1][n // 2] = code
        assert oracle.check_finite([make_tensor(np.zeros(n), np.zeros(n), np.zeros(n), g)],
                                   dtype=dtype) == 1
    # +Inf + -Inf in two replicas sums to NaN
    g = [b.copy() for b in base]
    g[0][7], g[2][7] = inf, ninf
    assert oracle.check_finite([make_tensor(np.zeros(n), np.zeros(n), np.zeros(n), g)],
                               dtype=dtype) == 1
    # finite replicas whose sum overflows FP32 only for BF16 (FP16's max is far below)
    g = [np.full(n, big, np.uint16) for _ in range(R)]
    want = 1 if dtype == "bf16" else 0
    assert oracle.check_finite([make_tensor(np.zeros(n), np.zeros(n), np.zeros(n), g)],
                               dtype=dtype) == want
    # the unscale factor enters: 3 * 65504 * 2^112 ~ 2^129.6 overflows FP32
    g = [np.full(n, 0x7BFF, np.uint16) for _ in range(R)]
    if dtype == "fp16":
        assert oracle.check_finite([make_tensor(np.zeros(n), np.zeros(n), np.zeros(n), g)],
                                   dtype=dtype, unscale=2.0 ** 112) == 1


def test_output_format_only_changes_the_compute_copy():
    rng = np.random.default_rng(22)
    n = 5000
    p = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m = (rng.standard_normal(n) * 1e-4).astype(np.float32)
    v = (rng.random(n) * 1e-6).astype(np.float32)
    g = [random_bf16(rng, n), random_bf16(rng, n)]
    outs = {}
    for fmt in ("bf16", "fp16", "none"):
        x = make_tensor(p, m, v, g)
        x.weight_out[:] = 0x7FAA
        oracle.step([x], dtype="bf16", step=4, out_dtype=fmt, **HP)
        outs[fmt] = x
    for f in ("master", "exp_avg", "exp_avg_sq"):
        assert np.array_equal(getattr(outs["bf16"], f), getattr(outs["fp16"], f))
        assert np.array_equal(getattr(outs["bf16"], f), getattr(outs["none"], f))
    assert np.array_equal(outs["bf16"].weight_out, torch_bf16_bits(outs["bf16"].master))
    assert np.array_equal(outs["fp16"].weight_out,
                          outs["fp16"].master.astype(np.float16).view(np.uint16))
    assert np.all(outs["none"].weight_out == 0x7FAA)


def test_large_finite_fp16_sum_does_not_raise_the_flag():
    big = np.full(16, 0x7BFF, np.uint16)  # 65504, largest finite binary16
    x = make_tensor(np.zeros(16), np.zeros(16), np.zeros(16), [big] * 8)
    assert oracle.step([x], dtype="fp16", step=1, with_flag=True, **HP) == 0


def test_every_output_element_is_written():
    rng = np.random.default_rng(8)
    sizes = [1, 2, 3, 7, 8, 9, 1000, 4097]
    ts = []
    for n in sizes:
        x = make_tensor((rng.standard_normal(n) * 0.02).astype(np.float32), np.zeros(n),
                        np.zeros(n), [random_bf16(rng, n), random_bf16(rng, n)])
        x.weight_out[:] = 0x7FAA  # a NaN payload the cast never produces
        ts.append(x)
    oracle.step(ts, dtype="bf16", step=1, **HP)
    for x in ts:
        assert not np.any(x.weight_out == 0x7FAA)
        assert np.array_equal(x.weight_out, torch_bf16_bits(x.master))


def test_invalid_hyperparameters_are_rejected():
    x = make_tensor(np.zeros(4), np.zeros(4), np.zeros(4), [np.zeros(4, np.uint16)])
    for bad in (dict(step=0), dict(beta1=1.0), dict(beta2=-0.1), dict(lr=-1.0),
                dict(eps=-1e-8), dict(weight_decay=float("nan")), dict(unscale=0.0),
                dict(unscale=float("inf"))):
        kw = dict(HP, step=1, unscale=1.0)
        kw.update(bad)
        with pytest.raises(ValueError):
            oracle.step([x], dtype="bf16", **kw)
