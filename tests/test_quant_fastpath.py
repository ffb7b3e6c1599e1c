"""The quantizer kernels' multiply-by-reciprocal fast path, checked on the CPU.

The kernels decide q = rint(fl(fl(x * 127) / eta)) ([P1] "2. Absmax Dynamic
Activation Quantization" and the ActivationQuantizerSTE listing) without the
division wherever p = fl(fl(x * 127) * fl(1 / eta)) is farther than 2^-12
from every half-integer, and with the IEEE division otherwise (also when p is
not finite, or 1 / eta would be subnormal).  This test replays that rule in
float32 numpy and compares it with the plain definition on random,
heavy-tailed, near-tie and extreme-magnitude rows; the GPU parity tests
compare the kernels themselves with the oracle.
"""
import numpy as np
import pytest

f32 = np.float32


def plain(x, eta):
    a = (x * f32(127)).astype(f32)
    return np.clip(np.rint((a / eta).astype(f32)), -128, 127)


def fast_rule(x, eta):
    a = (x * f32(127)).astype(f32)
    rcp = (f32(1) / eta).astype(f32) if eta < f32(2.0 ** 125) else f32(np.nan)
    p = (a * rcp).astype(f32)
    n = np.rint(p)
    with np.errstate(invalid="ignore"):
        ok = np.abs((p - n).astype(f32)) < f32(0.5 - 2.0 ** -12)
    return np.clip(np.where(ok, n, np.rint((a / eta).astype(f32))), -128, 127), ok


@pytest.mark.parametrize("kind", ["normal", "student_t_scaled", "near_ties", "wide_range", "huge"])
def test_fast_path_matches_division(kind):
    rng = np.random.default_rng(["normal", "student_t_scaled", "near_ties", "wide_range", "huge"].index(kind))
    for _ in range(20):
        n = 100_000
        if kind == "normal":
            x = rng.standard_normal(n).astype(f32)
        elif kind == "student_t_scaled":
            x = (rng.standard_t(3, n) * 10.0 ** rng.uniform(-6, 6)).astype(f32)
        elif kind == "near_ties":
            # x * 127 / eta within a few float32 ulps of k + 1/2
            eta = f32(rng.uniform(0.5, 5))
            k = rng.integers(-127, 127, n) + 0.5
            x = (k * float(eta) / 127 * (1 + rng.uniform(-3e-7, 3e-7, n))).astype(f32)
            x[0] = eta
        elif kind == "wide_range":
            x = (rng.uniform(-1, 1, n) * 10.0 ** rng.uniform(-30, 30)).astype(f32)
        else:   # x * 127 overflows, or 1 / eta is subnormal
            s = 10.0 ** rng.uniform(36, 38.5)
            x = (rng.uniform(-1, 1, n) * s).astype(f32)
            x[0] = f32(s)
        eta = f32(max(np.abs(x).max(), f32(1e-5)))
        with np.errstate(over="ignore", invalid="ignore"):
            want = plain(x, eta)
            got, ok = fast_rule(x, eta)
        assert np.array_equal(want, got)
        if kind == "near_ties":
            assert not ok[1:].any()   # every near tie takes the division


def test_zero_and_subnormal_inputs():
    x = np.array([0.0, -0.0, 1e-45, -1e-45, 1e-40, 3e-39], dtype=f32)
    eta = f32(1e-5)
    assert np.array_equal(plain(x, eta), fast_rule(x, eta)[0])
