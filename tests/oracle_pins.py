"""Pins for the CPU oracle: checks against what the BitNet b1.58 pages and the
mathematics fix, none of which re-types the oracle's own formula.

Each ``pin_*`` takes an oracle handle (``oracle.Oracle``) and raises
AssertionError when the oracle disagrees.  ``test_oracle_pins.py`` runs them on
the oracle as built; ``test_oracle_pin_strength.py`` runs them on copies of the
oracle with a planted mistake and requires that each copy fails at least one.

Kinds of pin used (no page prints a numeric worked example):
* facts the pages print (``golden/page_constants.txt``),
* hand-derived examples whose every step is exact,
* exact rational arithmetic (``fractions.Fraction``) for the mean,
* a library routine the method reduces to (integer matrix product),
* brute force over every ternary row of a tiny width,
* invariants and metamorphic relations, and closed-form statistics.
"""
from __future__ import annotations

import os
from fractions import Fraction
from math import erf, sqrt, pi

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def page_constants():
    facts = {}
    with open(os.path.join(GOLDEN, "page_constants.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, *vals = line.split()
            facts.setdefault(name, []).append(vals)
    return facts


def f32(v) -> np.float32:
    return np.float32(v)


def nearest_f32(fr: Fraction) -> np.float32:
    """The float32 nearest to a positive rational, ties to even, found by exact
    comparison among the neighbours of a first guess."""
    guess = np.float32(float(fr))
    cands = {guess, np.nextafter(guess, np.float32(0)), np.nextafter(guess, np.float32(np.inf))}
    best = None
    for c in sorted(cands):
        d = abs(Fraction(float(c)) - fr)
        if best is None or d < best[0]:
            best = (d, c)
        elif d == best[0]:
            # tie: keep the one with an even significand
            if int(np.float32(c).view(np.uint32)) % 2 == 0:
                best = (d, c)
    return np.float32(best[1])


def exact_mean_abs(W: np.ndarray) -> Fraction:
    total = Fraction(0)
    for v in np.asarray(W, np.float32).ravel():
        total += Fraction(abs(float(v)))
    return total / W.size


# ------------------------------------------------------------------ gamma
def pin_gamma_hand(O):
    # mean(|0.5|, |-0.5|, |1.5|, |-1.5|) = 1 exactly
    W = np.array([[0.5, -0.5, 1.5, -1.5]], np.float32)
    assert O.absmean_gamma(W) == f32(1.0)
    # 2x4 matrix: mean of |.| = (1+2+3+4+5+6+7+8)/8 = 4.5
    W = np.arange(1, 9, dtype=np.float32).reshape(2, 4) * np.array([1, -1, 1, -1], np.float32)
    assert O.absmean_gamma(W) == f32(4.5)


def pin_gamma_exact_rational(O):
    rng = np.random.default_rng(1234)
    cases = [
        rng.standard_normal((7, 13), dtype=np.float32) * f32(0.02),
        rng.standard_normal((1, 257), dtype=np.float32),
        rng.uniform(-3, 3, (33, 5)).astype(np.float32),
        # magnitudes spanning 2^-140 .. 2^120: any finite-precision running sum loses them
        (np.float32(2.0) ** rng.integers(-140, 120, (9, 11)).astype(np.float32)
         * rng.uniform(1, 2, (9, 11)).astype(np.float32)),
        np.array([[3e38, 1.0, 1e-30, 2.5e-45]], np.float32),
    ]
    for W in cases:
        want = max(nearest_f32(exact_mean_abs(W)), f32(1e-5))
        got = O.absmean_gamma(W)
        assert got == want, (W.shape, got, want)


def pin_gamma_ties(O):
    one = 1.0
    u = 2.0 ** -23
    # exact mean 1 + 2^-24 lies halfway between 1 and 1 + 2^-23: ties to even -> 1
    W = np.array([[one, one + u]], np.float32)
    assert O.absmean_gamma(W) == f32(1.0)
    # mean 1 + 3*2^-24 is halfway between 1 + 2^-23 (odd) and 1 + 2^-22 (even)
    W = np.array([[one + u, one + 2 * u]], np.float32)
    assert O.absmean_gamma(W) == f32(one + 2 * u)
    # just above the first midpoint: rounds up
    W = np.array([[one, one + u, one, one + 2 * u]], np.float32)  # mean = 1 + 3u/4
    assert O.absmean_gamma(W) == f32(one + u)
    # 1 + 2^-24 + 2^-41: a tie only in its first 25 bits; the far tail decides
    W = np.array([[2.0, u + 2.0 ** -40]], np.float32)
    assert O.absmean_gamma(W) == f32(one + u)


def pin_gamma_clamp(O):
    floor = f32(float(page_constants()["scale_floor"][0][0]))
    assert O.absmean_gamma(np.zeros((3, 5), np.float32)) == floor
    assert O.absmean_gamma(np.full((2, 2), 1e-7, np.float32)) == floor
    tiny = np.full((4, 4), 2.0 ** -149, np.float32)  # subnormal inputs
    assert O.absmean_gamma(tiny) == floor


def pin_gamma_metamorphic(O):
    rng = np.random.default_rng(7)
    W = rng.standard_normal((31, 17), dtype=np.float32) * f32(0.02)
    g = O.absmean_gamma(W)
    for e in (-8, 5, 20):
        assert O.absmean_gamma(W * f32(2.0 ** e)) == g * f32(2.0 ** e)
    assert O.absmean_gamma(-W) == g
    P = rng.permutation(W.ravel()).reshape(17, 31)  # order and shape free
    assert O.absmean_gamma(P) == g


def pin_gamma_statistics(O):
    # E|Z| = sigma * sqrt(2/pi) for Z ~ N(0, sigma^2); sd of |Z| is sigma*sqrt(1-2/pi)
    sigma = 0.02
    n = 1 << 20
    W = np.random.default_rng(99).standard_normal((1024, n // 1024), dtype=np.float32) * f32(sigma)
    g = float(O.absmean_gamma(W))
    mu = sigma * sqrt(2 / pi)
    se = sigma * sqrt(1 - 2 / pi) / sqrt(n)
    assert abs(g - mu) < 5 * se, (g, mu, se)


# ------------------------------------------------------------------ ternarize
def pin_ternarize_range_and_threshold(O):
    lo, hi = (int(v) for v in page_constants()["weight_clip"][0])
    rng = np.random.default_rng(5)
    W = rng.standard_normal((64, 96), dtype=np.float32) * f32(0.02)
    g = O.absmean_gamma(W)
    Wt = O.ternarize(W, g)
    assert set(np.unique(Wt)).issubset({lo, 0, hi})
    # Round-then-clip to [-1, 1] is a threshold at 1/2 on the float32 quotient:
    # +-1 exactly when |W/gamma| > 1/2 (round-half-even sends 0.5 to 0).
    t = W / g
    expect = np.where(np.abs(t) > f32(0.5), np.sign(t), 0).astype(np.int8)
    assert np.array_equal(Wt, expect)


def pin_ternarize_ties(O):
    g = f32(0.25)
    W = np.array([[0.125, -0.125, 0.1250001, 0.375, -0.375, 1.0, -7.0, 0.0]], np.float32)
    # quotients 0.5, -0.5, just above 0.5, 1.5, -1.5, 4, -28, 0
    assert O.ternarize(W, g).tolist() == [[0, 0, 1, 1, -1, 1, -1, 0]]


def pin_ternarize_division(O):
    # The weight quantizer listing divides W by gamma.  For these (gamma, W)
    # pairs the IEEE quotient lands just above 1/2 (so W~ = +1), while a
    # multiply by a rounded reciprocal of gamma would land at or below 1/2.
    # The quotient is rounded to float32 in exact rational arithmetic here.
    cases = [(0.028031973, 0.0140159875), (0.0059057022, 0.0029528514),
             (0.0062154713, 0.003107736), (0.013053724, 0.0065268623)]
    for g, w in cases:
        g, w = f32(g), f32(w)
        q = Fraction(float(nearest_f32(Fraction(float(w)) / Fraction(float(g)))))
        assert q > Fraction(1, 2)
        recip = nearest_f32(1 / Fraction(float(g)))
        assert Fraction(float(nearest_f32(Fraction(float(w)) * Fraction(float(recip))))) <= Fraction(1, 2)
        W = np.array([[w, -w]], np.float32)
        assert O.ternarize(W, g).tolist() == [[1, -1]], (g, w)


def pin_ternarize_symmetry(O):
    rng = np.random.default_rng(6)
    W = rng.standard_normal((16, 40), dtype=np.float32)
    g = O.absmean_gamma(W)
    assert np.array_equal(O.ternarize(-W, g), -O.ternarize(W, g))
    assert np.array_equal(O.ternarize(W * f32(8.0), g * f32(8.0)), O.ternarize(W, g))


def pin_ternarize_statistics(O):
    # gamma -> sigma*sqrt(2/pi), so P(w~ = 0) = P(|Z| <= sqrt(2/pi)/2) = erf(sqrt(1/pi)/2)
    n_rows, K = 1024, 1024
    W = np.random.default_rng(11).standard_normal((n_rows, K), dtype=np.float32) * f32(0.02)
    Wt, g = O.quantize_weights(W)
    p0 = erf(sqrt(2 / pi) / 2 / sqrt(2))
    n = Wt.size
    se = sqrt(p0 * (1 - p0) / n)
    z = float((Wt == 0).mean())
    assert abs(z - p0) < 5 * se, (z, p0)
    assert abs(p0 - 0.31006) < 1e-4
    assert abs(float((Wt == 1).mean()) - (1 - p0) / 2) < 5 * se
    # the pages report about a third of weights at zero for trained models
    assert abs(z - float(page_constants()["reported_zero_share"][0][0])) < 0.03


# ------------------------------------------------------------------ packing
def _code_of():
    return {int(w): int(c) for w, c in page_constants()["code"]}


def _shift_of():
    return {int(j): int(s) for j, s in page_constants()["field_shift"]}


def pin_pack_page_bytes(O):
    code, shift = _code_of(), _shift_of()

    def byte_of(ws):
        return sum(code[w] << shift[j] for j, w in enumerate(ws))

    for ws in ([-1, 0, 1, 0], [1, 1, 1, 1], [0, 0, 0, 0], [-1, -1, -1, -1], [1, -1, 0, 1]):
        got = O.pack(np.array([ws], np.int8))
        assert got.shape == (1, 1) and int(got[0, 0]) == byte_of(ws), (ws, got)
    assert int(O.pack(np.array([[-1, 0, 1, 0]], np.int8))[0, 0]) == 0x64
    assert int(O.pack(np.array([[1, 1, 1, 1]], np.int8))[0, 0]) == 0xAA
    assert int(O.pack(np.array([[0, 0, 0, 0]], np.int8))[0, 0]) == 0x55
    assert int(O.pack(np.array([[-1, -1, -1, -1]], np.int8))[0, 0]) == 0x00


def pin_pack_layout_and_padding(O):
    # K = 6: two bytes per row; the second byte holds k = 4, 5 and two pad fields (code 01)
    Wt = np.array([[1, 0, -1, 1, -1, 1], [0, 0, 0, 0, 1, -1]], np.int8)
    P = O.pack(Wt)
    assert P.shape == (2, 2)
    assert P.tolist() == [[0b10_00_01_10, 0b01_01_10_00], [0x55, 0b01_01_00_10]]


def pin_pack_roundtrip(O):
    rng = np.random.default_rng(3)
    for K in (1, 3, 4, 5, 63, 64, 130):
        Wt = rng.integers(-1, 2, (9, K)).astype(np.int8)
        P = O.pack(Wt)
        assert P.shape == (9, (K + 3) // 4)
        assert np.array_equal(O.unpack(P, K), Wt)
        # code 11 never appears
        fields = np.stack([(P >> s) & 3 for s in (0, 2, 4, 6)])
        assert not np.any(fields == 3)


def pin_pack_rejects(O):
    import oracle
    try:
        O.unpack(np.array([[0xFF]], np.uint8), 4)
    except oracle.OracleError:
        pass
    else:
        raise AssertionError("code 11 accepted")
    try:
        O.pack(np.array([[2, 0, 0, 0]], np.int8))
    except oracle.OracleError:
        pass
    else:
        raise AssertionError("non-ternary weight accepted")


# ------------------------------------------------------------------ activation quant
def pin_quant_hand(O):
    # eta = 127 so every quotient x*127/127 = x is exact: this isolates the
    # rounding rule (half to even) from the division.
    x = np.array([[127, 62.5, 63.5, -0.5, 0.5, 1.5, 2.5, -2.5]], np.float32)
    xq, eta = O.quantize_act(x)
    assert eta.tolist() == [127.0]
    assert xq.tolist() == [[127, 62, 64, 0, 0, 2, 2, -2]]
    # eta = 2: quotients (x*127)/2 = 127, -63.5 (-> -64, even), 31.75, -15.875, 0
    x = np.array([[2.0, -1.0, 0.5, -0.25, 0.0]], np.float32)
    xq, eta = O.quantize_act(x)
    assert eta.tolist() == [2.0]
    assert xq.tolist() == [[127, -64, 32, -16, 0]]


def _fl32(fr: Fraction) -> Fraction:
    """Round a rational to the nearest float32 (ties to even), exactly."""
    if fr == 0:
        return Fraction(0)
    r = nearest_f32(abs(fr))
    return Fraction(float(r)) if fr > 0 else -Fraction(float(r))


def pin_quant_op_order(O):
    # Both page listings write round(x * 127.0 / eta): multiply first, then an
    # IEEE division.  For these inputs the other order, (x / eta) * 127,
    # rounds to a different integer.  Each float step below is carried out in
    # exact rational arithmetic and rounded to float32 explicitly.
    cases = [(5.2772126, -4.466932), (7.6121526, 4.2855816), (2.7765708, 2.1316192),
             (1.1328796, 0.084742956), (3.7839653, -3.5307078)]
    for eta, xv in cases:
        eta, xv = f32(eta), f32(xv)
        x = np.array([[eta, xv]], np.float32)
        xq, e = O.quantize_act(x)
        assert e[0] == eta
        mul_first = round(_fl32(_fl32(Fraction(float(xv)) * 127) / Fraction(float(eta))))
        div_first = round(_fl32(_fl32(Fraction(float(xv)) / Fraction(float(eta))) * 127))
        assert mul_first != div_first
        assert int(xq[0, 1]) == mul_first, (eta, xv, int(xq[0, 1]), mul_first)


def pin_quant_invariants(O):
    qb = int(page_constants()["qb"][0][0])
    rng = np.random.default_rng(8)
    x = np.concatenate([rng.standard_normal((5, 300), dtype=np.float32),
                        rng.standard_t(3, (5, 300)).astype(np.float32)])
    xq, eta = O.quantize_act(x)
    assert np.array_equal(eta, np.abs(x).max(axis=1))
    assert xq.min() >= -qb and xq.max() <= qb
    arg = np.abs(x).argmax(axis=1)
    assert np.array_equal(np.abs(xq[np.arange(len(x)), arg]), np.full(len(x), qb))
    assert np.all((np.sign(xq) == np.sign(x)) | (xq == 0))
    # within a rounding step of the real-valued x*127/eta (two float roundings
    # add at most 2^-17 on a quotient of magnitude <= 127)
    real = x.astype(np.float64) * qb / eta.astype(np.float64)[:, None]
    assert np.max(np.abs(xq - real)) <= 0.5 + 2.0 ** -16
    # monotone within a row
    for m in range(len(x)):
        o = np.argsort(x[m], kind="stable")
        assert np.all(np.diff(xq[m][o].astype(int)) >= 0)


def pin_quant_metamorphic(O):
    rng = np.random.default_rng(9)
    x = rng.standard_normal((4, 77), dtype=np.float32)
    xq, eta = O.quantize_act(x)
    for e in (-10, 3, 30):
        xq2, eta2 = O.quantize_act(x * f32(2.0 ** e))
        assert np.array_equal(xq2, xq)
        assert np.array_equal(eta2, eta * f32(2.0 ** e))
    xqn, etan = O.quantize_act(-x)
    assert np.array_equal(xqn, -xq) and np.array_equal(etan, eta)
    # per token: each row is quantized on its own
    for m in range(4):
        r, e = O.quantize_act(x[m:m + 1])
        assert np.array_equal(r[0], xq[m]) and e[0] == eta[m]


def pin_quant_floor(O):
    floor = f32(float(page_constants()["scale_floor"][0][0]))
    xq, eta = O.quantize_act(np.zeros((2, 9), np.float32))
    assert np.all(xq == 0) and np.all(eta == floor)
    x = np.array([[5e-6, -2.5e-6, 0.0, 1e-6]], np.float32)  # |x| below the floor
    xq, eta = O.quantize_act(x)
    assert eta[0] == floor
    # 5e-6*127/1e-5 = 63.5 -> 64 or 63 depending on float rounding of the
    # operands; the magnitude is bounded by 127 * 5e-6 / 1e-5 = 63.5
    assert abs(int(xq[0, 0])) in (63, 64) and int(xq[0, 2]) == 0


# ------------------------------------------------------------------ contraction
def pin_contract_hand(O):
    xq = np.array([[127, 62, 64, 0, 0, 2, 2, -2]], np.int8)
    Wt = np.array([[1, -1, 0, 1, -1, 1, 1, -1]], np.int8)
    # +1 at k=0,3,5,6: 127+0+2+2 = 131; -1 at k=1,4,7: 62+0-2 = 60 -> 71
    assert O.ternary_contract(xq, Wt).tolist() == [[71]]


def pin_contract_bruteforce(O):
    # every ternary row of width 5 (3^5 = 243 rows) against random int8 rows,
    # including the extremes; compared with numpy's integer and float64 matmul
    import itertools
    Wt = np.array(list(itertools.product((-1, 0, 1), repeat=5)), np.int8)
    rng = np.random.default_rng(12)
    xq = np.concatenate([rng.integers(-128, 128, (6, 5)),
                         [[127] * 5, [-128] * 5, [0] * 5, [127, -128, 1, -1, 0]]]).astype(np.int8)
    y = O.ternary_contract(xq, Wt)
    assert y.shape == (10, 243)
    assert np.array_equal(y, xq.astype(np.int64) @ Wt.astype(np.int64).T)
    assert np.array_equal(y, (xq.astype(np.float64) @ Wt.astype(np.float64).T).astype(np.int64))


def pin_contract_library(O):
    rng = np.random.default_rng(13)
    M, N, K = 3, 37, 211  # all distinct, so a transposed operand cannot pass
    xq = rng.integers(-127, 128, (M, K)).astype(np.int8)
    Wt = rng.integers(-1, 2, (N, K)).astype(np.int8)
    ref = xq.astype(np.int64) @ Wt.astype(np.int64).T
    assert np.array_equal(O.ternary_contract(xq, Wt), ref)
    assert np.array_equal(O.ternary_contract(xq, Wt, threads=4), ref)
    # a consistent permutation of the reduction index changes nothing
    p = rng.permutation(K)
    assert np.array_equal(O.ternary_contract(xq[:, p], Wt[:, p]), ref)


def pin_contract_extremes(O):
    K = 28672
    xq = np.full((2, K), 127, np.int8)
    xq[1] = -127
    Wt = np.ones((2, K), np.int8)
    Wt[1] = -1
    y = O.ternary_contract(xq, Wt)
    assert y.tolist() == [[127 * K, -127 * K], [-127 * K, 127 * K]]


# ------------------------------------------------------------------ dequant and chain
def pin_dequant(O):
    qb = int(page_constants()["qb"][0][0])
    rng = np.random.default_rng(14)
    y_int = rng.integers(-3_600_000, 3_600_000, (4, 50)).astype(np.int32)
    y_int[0, 0] = 0
    eta = rng.uniform(0.5, 40, 4).astype(np.float32)
    g = f32(0.0173)
    y = O.dequant(y_int, eta, g)
    real = y_int.astype(np.float64) * eta.astype(np.float64)[:, None] * float(g) / qb
    nz = real != 0
    # three float32 roundings: relative error below 2^-22
    assert np.all(np.abs(y[nz] - real[nz]) <= 2.0 ** -22 * np.abs(real[nz]))
    assert y[0, 0] == 0.0
    # exact case: eta*gamma = 127 -> scale 1
    assert O.dequant(np.array([[5, -9]], np.int32), np.array([127.0], np.float32),
                     f32(1.0)).tolist() == [[5.0, -9.0]]


def _signed_nearest_f32(fr: Fraction) -> np.float32:
    if fr == 0:
        return f32(0.0)
    v = nearest_f32(abs(fr))
    return v if fr > 0 else -v


def pin_dequant_association(O):
    # The scale is (eta * gamma) / 127 in this order, each step rounded to
    # float32 (BitLinear158.forward step 5 of the first page's production
    # listing; the fifth page's bitlinear_forward listing).  Pairs are chosen
    # where the other two associations, eta * (gamma / 127) and
    # gamma * (eta / 127), give three different float32 scales; the expected
    # bits come from exact rational arithmetic, rounded once per step.
    qb = int(page_constants()["qb"][0][0])
    rng = np.random.default_rng(2024)
    etas, gammas = [], []
    for _ in range(40000):
        eta = f32(rng.uniform(0.5, 40.0))
        g = f32(rng.uniform(0.005, 0.05))
        a = f32(f32(eta * g) / f32(qb))
        b = f32(eta * f32(g / f32(qb)))
        c = f32(g * f32(eta / f32(qb)))
        if len({float(a), float(b), float(c)}) == 3:
            etas.append(eta)
            gammas.append(g)
        if len(etas) == 8:
            break
    assert len(etas) == 8
    y_int = np.array([1, -1, 7, 1 << 20, -3_641_344, 2_000_001], np.int32)
    for eta, g in zip(etas, gammas):
        eg = nearest_f32(Fraction(float(eta)) * Fraction(float(g)))
        s = nearest_f32(Fraction(float(eg)) / qb)
        want = [_signed_nearest_f32(int(v) * Fraction(float(s))) for v in y_int]
        got = O.dequant(y_int[None, :], np.array([eta], np.float32), g)[0]
        assert got.tolist() == [float(w) for w in want], (eta, g, got, want)


def pin_chain_hand(O):
    # W = [1,-1,0,1,-1,1,1,-1]: gamma = 7/8; W/gamma = +-8/7 or 0 -> W~ = W
    W = np.array([[1, -1, 0, 1, -1, 1, 1, -1]], np.float32)
    Wt, g = O.quantize_weights(W)
    assert g == f32(0.875) and Wt.tolist() == [[1, -1, 0, 1, -1, 1, 1, -1]]
    x = np.array([[127, 62.5, 63.5, -0.5, 0.5, 1.5, 2.5, -2.5]], np.float32)
    y, xq, eta, y_int = O.forward(x, Wt, g)
    # y_int = 71; scale = (127 * 0.875) / 127 = 0.875 exactly; y = 62.125
    assert y_int.tolist() == [[71]] and y.tolist() == [[62.125]]


def pin_demo_shapes(O):
    # the first page's demonstration: batch 2 x seq 64 tokens, 1024 -> 2048
    rng = np.random.default_rng(42)
    x = rng.standard_normal((2 * 64, 1024), dtype=np.float32)
    W = rng.standard_normal((2048, 1024), dtype=np.float32) * f32(0.02)
    Wt, g = O.quantize_weights(W)
    y, xq, eta, y_int = O.forward(x, Wt, g, threads=4)
    assert y.shape == (128, 2048) and set(np.unique(Wt)) == {-1, 0, 1}
    assert np.array_equal(y_int, xq.astype(np.int64) @ Wt.astype(np.int64).T)


# ------------------------------------------------------------ absmedian gamma
# The median of |W| in place of the mean (second page: BitNet b1.58 Reloaded's
# absmedian baseline); an even count takes the mean of the two middle values.

def pin_absmedian_hand(O):
    assert O.absmedian_gamma(np.array([[3, -1, 2]], np.float32)) == f32(2)
    # even count: (2 + 3) / 2, where the mean of |W| would be 4
    assert O.absmedian_gamma(np.array([[1, -2, 3, -10]], np.float32)) == f32(2.5)
    assert O.absmedian_gamma(np.array([[-7.0]], np.float32)) == f32(7)
    assert O.absmedian_gamma(np.zeros((3, 4), np.float32)) == f32(1e-5)   # clamp


def pin_absmedian_library(O):
    # numpy's median of the magnitudes in float64 is the mean of the two middle
    # values rounded once in float64; rounding that to float32 is the correctly
    # rounded mean (53 >= 2 * 24 + 2 bits), so it must equal the oracle's.
    rng = np.random.default_rng(41)
    for N, K in ((1, 1), (1, 2), (3, 5), (4, 6), (17, 33), (64, 64), (101, 7)):
        W = (rng.standard_normal((N, K)) * np.exp2(rng.integers(-20, 20, (N, K)))).astype(np.float32)
        W[rng.random((N, K)) < 0.2] = 0
        want = np.float32(np.median(np.abs(W).astype(np.float64)))
        want = max(want, f32(1e-5))
        assert O.absmedian_gamma(W) == want, (N, K)


def pin_absmedian_ties(O):
    one = f32(1)
    u = np.float32(2.0 ** -23)
    # middle pair 1 and 1 + 2^-23: mean 1 + 2^-24, a tie, to the even 1
    W = np.array([[0.5, 1, 1 + u, 3]], np.float32)
    assert O.absmedian_gamma(W) == one
    # middle pair 1 + 2^-23 and 1 + 2^-22: tie, to the even 1 + 2^-22
    W = np.array([[0.5, -(1 + u), 1 + 2 * u, 3]], np.float32)
    assert O.absmedian_gamma(W) == np.float32(1 + 2 * u)


def pin_absmedian_invariants(O):
    rng = np.random.default_rng(42)
    W = rng.standard_normal((37, 53)).astype(np.float32)
    g = O.absmedian_gamma(W)
    P = rng.permutation(W.size)
    assert O.absmedian_gamma(W.ravel()[P].reshape(53, 37)) == g
    assert O.absmedian_gamma(-W) == g
    assert O.absmedian_gamma(W * np.float32(2 ** 7)) == g * np.float32(2 ** 7)


def pin_absmedian_statistics(O):
    # |N(0, s^2)| has median s * Phi^-1(3/4) = 0.67449 s, and the ternarizer
    # then zeroes |W| < gamma / 2: a fraction 2 Phi(0.33724) - 1 = 0.26406.
    rng = np.random.default_rng(43)
    W = (rng.standard_normal((700, 1000)) * 0.02).astype(np.float32)
    Wt, g = O.quantize_weights_absmedian(W)
    assert abs(float(g) / (0.02 * 0.6744897501960817) - 1) < 0.005
    zero = float((Wt == 0).mean())
    assert abs(zero - (erf(0.33724487509804085 / sqrt(2)))) < 0.003


# ------------------------------------------------------------ base-3 packing
# Five ternary weights per byte (second page: 1.58 bits per weight under
# compact ternary packing; third page: log2(3) bits of information).  Reading
# of the layout: digit w + 1, weight k = 5b + j at 3^j, pad digit 1.

def _base3_value(ws) -> int:
    """Value of the digits w+1 read as a base-3 numeral, least significant
    first, by Python's own base conversion."""
    return int("".join(str(int(w) + 1) for w in reversed(ws)), 3)


def pin_pack3_closed_forms(O):
    W = np.array([[-1] * 5, [1] * 5, [0] * 5, [1, -1, 0, -1, -1]], np.int8)
    assert O.pack3(W).ravel().tolist() == [0, 242, 121, 11]
    # a partial last byte pads with zero weights (digit 1)
    assert O.pack3(np.array([[1, 0, 0, 0, 0, -1, 1]], np.int8)).tolist() == [[122, 123]]
    assert O.pack3(np.zeros((3, 11), np.int8)).shape == (3, 3)


def pin_pack3_exhaustive(O):
    # every ternary 5-vector: the byte is its base-3 numeral, and the map is a
    # bijection onto 0..242
    vecs = np.array(np.meshgrid(*[[-1, 0, 1]] * 5, indexing="ij")).reshape(5, -1).T.astype(np.int8)
    b = O.pack3(vecs).ravel()
    assert sorted(b.tolist()) == list(range(243))
    for v, byte in zip(vecs, b):
        assert int(byte) == _base3_value(v)
    assert np.array_equal(O.unpack3(b.reshape(-1, 1), 5), vecs)


def pin_pack3_roundtrip_and_density(O):
    rng = np.random.default_rng(21)
    for N, K in ((1, 1), (3, 7), (17, 80), (5, 1001)):
        Wt = rng.integers(-1, 2, (N, K)).astype(np.int8)
        p3 = O.pack3(Wt)
        assert p3.shape == (N, -(-K // 5)) and int(p3.max()) <= 242
        assert np.array_equal(O.unpack3(p3, K), Wt)
        assert np.array_equal(O.unpack3(p3, K), O.unpack(O.pack(Wt), K))
        if K % 20 == 0:
            assert p3.size * 5 == O.pack(Wt).size * 4   # 1.6 against 2 bits per weight


def pin_pack3_rejects(O):
    import oracle as _o
    for bad in (243, 255):
        try:
            O.unpack3(np.array([[bad]], np.uint8), 5)
        except _o.OracleError:
            pass
        else:
            raise AssertionError(f"byte {bad} accepted")
    try:
        O.pack3(np.array([[2, 0, 0, 0, 0]], np.int8))
    except _o.OracleError:
        pass
    else:
        raise AssertionError("non-ternary weight accepted")


# ------------------------------------------------------------------ RMSNorm
# RMSNorm without affine parameters before the quantizer (first page, step 1 of
# BitLinear158.forward): norm = 1 / sqrt(mean(x^2) + 1e-6), x_norm = x * norm.
# The mean is exact and rounded once; sqrt and 1/s are IEEE float32 steps.

def _rms_eps() -> np.float32:
    return f32(page_constants()["rms_eps"][0][0])


def _sqrt_f32(t: np.float32) -> np.float32:
    """Correctly rounded float32 square root, decided by exact comparison of
    squares (no library square root is trusted)."""
    tf = Fraction(float(t))
    if tf == 0:
        return f32(0)
    c = np.float32(np.sqrt(np.float64(t)))
    cands = sorted({c, np.nextafter(c, f32(0)), np.nextafter(c, f32(np.inf))})
    best = None
    for v in cands:
        # |v - sqrt(t)| compared through (v^2 - t) / (v + sqrt(t)); equivalently
        # compare the candidates' midpoints: sqrt(t) lies above mid iff t > mid^2
        if best is None:
            best = v
            continue
        mid = (Fraction(float(best)) + Fraction(float(v))) / 2
        if tf > mid * mid:
            best = v
        elif tf == mid * mid and int(np.float32(v).view(np.uint32)) % 2 == 0:
            best = v
    return np.float32(best)


def _rms_chain(row: np.ndarray):
    """(ms, norm, x_norm) of one row by exact rational arithmetic."""
    S = sum((Fraction(float(v)) ** 2 for v in row), Fraction(0))
    ms = nearest_f32(S / len(row)) if S else f32(0)
    t = np.float32(_fl32(Fraction(float(ms)) + Fraction(float(_rms_eps()))))
    s = _sqrt_f32(t)
    norm = np.float32(_fl32(1 / Fraction(float(s))))
    xn = np.array([_fl32(Fraction(float(v)) * Fraction(float(norm))) for v in row], np.float32)
    return ms, norm, xn


def pin_rms_hand(O):
    # x = [768, 1024, 0, 0]: sum of squares 1638400, mean 409600 = 640^2, so
    # s = 640 and norm = fl(1/640); x_norm = 768 / 640 and 1024 / 640 up to one
    # rounding: eta = fl(1024 * fl(1/640)) = fl(1.6) since 1024 is a power of
    # two, and round(127 * 1.2 / 1.6) = round(95.25) = 95.
    x = np.array([[768, 1024, 0, 0]], np.float32)
    xq, eta, ms, norm = O.rmsnorm_quantize_act(x)
    assert ms[0] == f32(409600)
    assert Fraction(float(norm[0])) == _fl32(Fraction(1, 640))
    assert Fraction(float(eta[0])) == _fl32(Fraction(8, 5))
    assert xq.tolist() == [[95, 127, 0, 0]]


def pin_rms_constant_rows(O):
    # A row of +-2^j (j >= 4): mean of squares 2^(2j) exactly, 1e-6 is below
    # half an ulp of it, sqrt = 2^j, norm = 2^-j, so x_norm = +-1 exactly.
    rng = np.random.default_rng(11)
    for j in (4, 5, 10, 40):
        for K in (1, 3, 64, 1000):
            sign = np.where(rng.random(K) < 0.5, -1.0, 1.0).astype(np.float32)
            x = (sign * np.float32(2.0 ** j))[None, :]
            xn, ms, norm = O.rmsnorm(x)
            assert ms[0] == f32(2.0 ** (2 * j)) and norm[0] == f32(2.0 ** -j)
            assert np.array_equal(xn[0], sign)
            xq, eta, _, _ = O.rmsnorm_quantize_act(x)
            assert eta[0] == f32(1) and np.array_equal(xq[0], (sign * 127).astype(np.int8))


def pin_rms_exact_sum(O):
    # One large element and many ones: a float32 running sum absorbs every one
    # (2^24 + 1 = 2^24); the exact mean keeps them.  K = 1024, step 2^-9 there.
    big = [4096.0]
    for ones, want in ((1023, 16385.0),                  # 511.5 steps: tie, up to even
                       (1022, 16384 + 511 / 512),        # 511 steps: exact
                       (1021, 16384 + 510 / 512)):       # 510.5 steps: tie, down to even
        row = np.array(big + [1.0] * ones + [0.0] * (1023 - ones), np.float32)
        _, ms, _ = O.rmsnorm(row[None, :])
        assert ms[0] == f32(want), (ones, ms[0], want)
        assert Fraction(float(ms[0])) == Fraction(float(nearest_f32(Fraction(2 ** 24 + ones, 1024))))


def pin_rms_rational(O):
    # Random rows over a wide exponent range, zeros and subnormals included,
    # against the exact rational chain.
    rng = np.random.default_rng(12)
    for K in (1, 2, 5, 17, 64):
        for _ in range(6):
            mant = rng.uniform(1, 2, K) * np.where(rng.random(K) < 0.5, -1, 1)
            expo = rng.integers(-60, 60, K)
            row = (mant * np.exp2(expo)).astype(np.float32)
            row[rng.random(K) < 0.15] = 0
            if K > 2:
                row[0] = np.float32(3e-41)               # a subnormal
            xn, ms, norm = O.rmsnorm(row[None, :])
            ems, enorm, exn = _rms_chain(row)
            assert ms[0] == ems and norm[0] == enorm, (K, ms[0], ems, norm[0], enorm)
            assert np.array_equal(xn[0], exn)
    # Tiny rows whose mean of squares is a float32 subnormal (or rounds to 0).
    for K in (1, 3, 8):
        for lo in (-75, -70, -66):
            row = (rng.uniform(1, 2, K) * np.exp2(rng.integers(lo, lo + 4, K))).astype(np.float32)
            _, ms, _ = O.rmsnorm(row[None, :])
            ems, _, _ = _rms_chain(row)
            assert ms[0] == ems, (K, lo, ms[0], ems)
            assert ms[0] < np.finfo(np.float32).tiny


def pin_rms_extremes(O):
    # Squares beyond float32: the mean rounds to +Inf, norm to 0, the row to 0.
    x = np.full((1, 16), 1e20, np.float32)
    xq, eta, ms, norm = O.rmsnorm_quantize_act(x)
    assert np.isinf(ms[0]) and norm[0] == 0 and not xq.any() and eta[0] == f32(1e-5)
    # All zeros: mean 0, norm = 1 / sqrt(1e-6), nothing to quantize.
    z = np.zeros((1, 16), np.float32)
    xq, eta, ms, norm = O.rmsnorm_quantize_act(z)
    want = np.float32(_fl32(1 / Fraction(float(_sqrt_f32(_rms_eps())))))
    assert ms[0] == 0 and norm[0] == want and not xq.any() and eta[0] == f32(1e-5)


def pin_rms_invariants(O):
    rng = np.random.default_rng(13)
    x = (rng.standard_normal((6, 300)) * np.exp2(rng.integers(-8, 8, (6, 1)))).astype(np.float32)
    x[2, 7] = 3e4                                        # mixed magnitudes
    xn, ms, norm = O.rmsnorm(x)
    xq, eta, ms2, norm2 = O.rmsnorm_quantize_act(x)
    assert np.array_equal(ms, ms2) and np.array_equal(norm, norm2)
    for m in range(x.shape[0]):
        # rounding is monotone, so the largest |x_norm| is fl(max|x| * norm)
        amax = np.float32(np.abs(x[m]).max())
        assert Fraction(float(eta[m])) == _fl32(Fraction(float(amax)) * Fraction(float(norm[m])))
        # the exact mean does not depend on the order of the terms
        p = rng.permutation(x.shape[1])
        _, msp, _ = O.rmsnorm(x[m, p][None, :])
        assert msp[0] == ms[m]
        # scaling by 4 scales the mean by 16 exactly while ms >= 32 (1e-6 then
        # vanishes in the sum), so x_norm is unchanged
        if ms[m] >= 32:
            xn4, ms4, _ = O.rmsnorm((x[m] * 4)[None, :])
            assert ms4[0] == ms[m] * 16 and np.array_equal(xn4[0], xn[m])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
