"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: worked
values from the pages (tests/golden/), closed forms, exact rational
arithmetic, textbook special cases and brute force on tiny inputs.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import tq_inputs as ti

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F32 = np.float32


def _golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = (p.strip() for p in line.split(";"))
            rows.append((a, b))
    return rows


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [line.strip() for line in f if line.strip() and not line.startswith("#")]


def _f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


# ---------------------------------------------------------------- sizes / pack

def test_packed_size_golden():
    for a, b in _golden("sizes.txt"):
        assert oracle.packed_bytes(int(a)) == int(b)


def test_pack_worked_bytes_golden():
    for a, b in _golden("pack_worked_bytes.txt"):
        vals = np.array([int(v) for v in a.split(",")], dtype=np.int8)
        want = np.array([int(h, 16) for h in b.split()], dtype=np.uint8)
        got = oracle.pack_codes(vals)[0]
        np.testing.assert_array_equal(got, want)
        np.testing.assert_array_equal(oracle.unpack_codes(got, vals.size)[0], vals)


def test_pack_roundtrip_64x1536():
    # the pack/unpack identity at the shape Hetman-2b s.8 test 5 uses
    q = ti.random_ternary(5, 64, 1536)
    p = oracle.pack_codes(q)
    assert p.shape == (64, 384)
    np.testing.assert_array_equal(oracle.unpack_codes(p, 1536), q)


def test_pack_bit_positions_exhaustive():
    # every 4-tuple of values maps to the byte whose 2-bit field j holds v_j + 1
    for a in range(-1, 2):
        for b in range(-1, 2):
            for c in range(-1, 2):
                for d in range(-1, 2):
                    byte = oracle.pack_codes(np.array([a, b, c, d]))[0, 0]
                    fields = [(int(byte) >> (2 * j)) & 3 for j in range(4)]
                    assert fields == [a + 1, b + 1, c + 1, d + 1]
                    assert 3 not in fields


def test_unpack_rejects_code_11():
    with pytest.raises(ValueError):
        oracle.unpack_codes(np.array([[0xFF]], dtype=np.uint8), 4)


def test_pack_rejects_non_ternary():
    with pytest.raises(ValueError):
        oracle.pack_codes(np.array([[2, 0, 0, 0]]))


# ------------------------------------------------------------- rational rounding

def test_round_rational_representable_identity():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(2000).astype(np.float32),
        (rng.standard_normal(500) * 1e-30).astype(np.float32),
        np.array([1e-45, 2**-126, 3.4e38, 1.0, 0.5], dtype=np.float32)])
    for v in np.abs(vals):
        fr = Fraction(float(v))
        if fr == 0:
            continue
        assert oracle.round_rational_to_f32(fr.numerator, fr.denominator) == v


def test_round_rational_ties_to_even():
    # midpoints between neighbouring fp32 values go to the even significand
    one = Fraction(1)
    ulp = Fraction(1, 2**23)
    assert oracle.round_rational_to_f32(*_nd(one + ulp / 2)) == F32(1.0)
    assert oracle.round_rational_to_f32(*_nd(one + 3 * ulp / 2)) == _f32(0x3F800002)
    # just above / below a midpoint
    eps = Fraction(1, 2**80)
    assert oracle.round_rational_to_f32(*_nd(one + ulp / 2 + eps)) == _f32(0x3F800001)
    assert oracle.round_rational_to_f32(*_nd(one + 3 * ulp / 2 - eps)) == _f32(0x3F800001)
    # carry into the next binade
    top = Fraction(2) - Fraction(1, 2**24)          # midpoint below 2.0
    assert oracle.round_rational_to_f32(*_nd(top)) == F32(2.0)
    # subnormal midpoint: 1.5 * 2**-149 -> 2 * 2**-149 (even)
    assert oracle.round_rational_to_f32(3, 2**150) == _f32(2)


def test_round_rational_matches_double_off_ties():
    # away from fp32 midpoints, rounding the fp64 nearest value again is exact
    rng = np.random.default_rng(1)
    for _ in range(3000):
        n = int(rng.integers(1, 2**62))
        d = int(rng.integers(1, 2**40))
        want = np.float32(n / d)
        got = oracle.round_rational_to_f32(n, d)
        v = Fraction(n, d)
        lo = Fraction(float(np.nextafter(want, np.float32(0))))
        hi = Fraction(float(np.nextafter(want, np.float32(np.inf))))
        w = Fraction(float(want))
        near_tie = min(abs(v - (w + lo) / 2), abs(v - (w + hi) / 2)) < w * Fraction(1, 2**50)
        if not near_tie:
            assert got == want


def _nd(fr):
    return fr.numerator, fr.denominator


# -------------------------------------------------------------------- absmean

def test_gamma_all_zero_is_eps():
    assert oracle.absmean_scale(np.zeros(1000, np.float32)) == F32(1e-6)


def test_gamma_constant_magnitude_exact():
    for a in [0.02, 1.0, 3.1415927, 1e-3, 123.456]:
        a = F32(a)
        w = np.array([a, -a, a, -a, -a, a, a], dtype=np.float32)
        assert oracle.absmean_scale(w) == a


def test_gamma_small_cases():
    assert oracle.absmean_scale(np.array([1.0, 3.0], np.float32)) == F32(2.0)
    assert oracle.absmean_scale(np.array([-1.0, 3.0, -2.0], np.float32)) == F32(2.0)


def test_gamma_exact_tie_goes_to_even():
    # mean of [1, 1 + 2^-23] is 1 + 2^-24: a midpoint; ties-to-even gives 1.0
    w = np.array([1.0, _f32(0x3F800001)], np.float32)
    assert oracle.absmean_scale(w) == F32(1.0)
    # mean of [1 + 2^-23, 1 + 2^-22] is 1 + 3*2^-24: midpoint; even is 1 + 2^-22
    w = np.array([_f32(0x3F800001), _f32(0x3F800002)], np.float32)
    assert oracle.absmean_scale(w) == _f32(0x3F800002)


def test_gamma_beyond_double_precision():
    # sum = 3 + 2^-23 + 2^-60, mean = 0.75 + 2^-25 + 2^-62: just above the
    # midpoint between 0.75 and 0.75 + 2^-24, so it rounds up.  A sum carried
    # in fp64 loses the 2^-60 term and lands exactly on the midpoint, which
    # would round to the even neighbour 0.75 instead.
    w = np.array([1.0, 1.0, _f32(0x3F800001), F32(2.0**-60)], np.float32)
    assert oracle.absmean_scale(w) == _f32(0x3F400001)
    naive = np.float32(np.sum(np.abs(w).astype(np.float64)) / 4)
    assert naive == F32(0.75)


def test_gamma_matches_fraction_mean_on_random_groups():
    rng = np.random.default_rng(2)
    for trial in range(40):
        n = int(rng.integers(1, 300))
        scale = 10.0 ** rng.integers(-30, 30)
        w = (rng.standard_normal(n) * scale).astype(np.float32)
        fr = oracle.exact_fraction_mean(w)
        want = oracle.round_rational_to_f32(fr.numerator, fr.denominator)
        want = max(want, F32(1e-6))
        assert oracle.absmean_scale(w) == want


def test_exact_abs_sum_against_fraction():
    rng = np.random.default_rng(3)
    w = np.concatenate([rng.standard_normal(500).astype(np.float32),
                        np.array([1e-45, -3e-42, 1e30, -2.5e-38], np.float32)])
    units = oracle.exact_abs_sum_units(w)
    fr = sum((Fraction(float(abs(v))) for v in w), Fraction(0))
    assert Fraction(units, 2**149) == fr


def test_gamma_statistics_normal_weights():
    # E|w| = sigma * sqrt(2/pi) for w ~ N(0, sigma^2)
    W = ti.workload_weights("decode")
    g = oracle.absmean_scales(W, "tensor")[0]
    assert abs(g / (0.02 * np.sqrt(2 / np.pi)) - 1) < 2e-3
    # and it agrees with the fp64 mean rounded to fp32 unless that mean sits
    # within fp64 error of an fp32 midpoint
    m64 = np.mean(np.abs(W).astype(np.float64))
    assert abs(float(g) - m64) <= float(np.spacing(np.float32(g)))


def test_gamma_per_row_uses_each_row():
    W = np.array([[1, -3, 0, 0], [2, 2, -2, 2]], np.float32)
    np.testing.assert_array_equal(oracle.absmean_scales(W, "row"),
                                  np.array([1.0, 2.0], np.float32))
    np.testing.assert_array_equal(oracle.absmean_scales(W, "tensor"),
                                  np.array([1.5], np.float32))


# -------------------------------------------------------------------- ternarize

def test_ternarize_half_even_tie():
    # W = [1, 3]: gamma = 2, w/gamma = [0.5, 1.5] -> [0, 1] (half to even, then
    # clamp), packed with zero-code padding to 0x59
    W = np.array([[1.0, 3.0]], np.float32)
    packed, g = oracle.pack_ternary(W, "tensor")
    assert g[0] == F32(2.0)
    np.testing.assert_array_equal(oracle.ternarize(W, g), [[0, 1]])
    assert packed[0, 0] == 0x59


def test_ternarize_brute_force_grid():
    # every w in {-4..4}/4 against gamma = 1: round half even then clamp
    w = (np.arange(-16, 17, dtype=np.float32) / 4).reshape(1, -1)
    q = oracle.ternarize(w, np.array([1.0], np.float32))[0]
    for wi, qi in zip(w[0], q):
        if abs(wi) <= 0.5:
            assert qi == 0
        else:
            assert qi == (1 if wi > 0 else -1)


def test_ternarize_equals_half_scale_comparison():
    # For normal fp32 w and gamma, fp32(w/gamma) rounds above 0.5 exactly when
    # w > gamma/2: the next fp32 above gamma/2 exceeds it by more than
    # gamma*2^-25, half the spacing of fp32 values just above 0.5.  So the
    # round-and-clamp rule is the comparison |w| > gamma/2, ties giving 0.
    rng = np.random.default_rng(4)
    for _ in range(200):
        g = F32(np.abs(rng.standard_normal()) * 10.0 ** rng.integers(-5, 5) + 1e-6)
        h = F32(g * F32(0.5))
        near = [h, np.nextafter(h, F32(np.inf)), np.nextafter(h, F32(0)),
                F32(1.5) * g, np.nextafter(F32(1.5) * g, F32(np.inf))]
        w = np.array(near + [-v for v in near] +
                     list((rng.standard_normal(20) * g).astype(np.float32)),
                     np.float32).reshape(1, -1)
        q = oracle.ternarize(w, np.array([g], np.float32))[0]
        want = (w[0] > h).astype(np.int8) - (w[0] < -h).astype(np.int8)
        np.testing.assert_array_equal(q, want)


def test_zero_fraction_normal_weights():
    # for N(0, s^2) and gamma = s*sqrt(2/pi): P(|w| <= gamma/2) = erf(sqrt(1/(4 pi)))
    from math import erf, pi, sqrt
    W = ti.workload_weights("tiny")
    packed, g = oracle.pack_ternary(W, "tensor")
    q = oracle.unpack_codes(packed, 256)
    frac0 = np.mean(q == 0)
    assert abs(frac0 - erf(sqrt(1 / (4 * pi)))) < 0.01


def test_binary_mode():
    W = np.array([[0.0, -0.0, 1e-30, -1e-30, 2.0, -3.0, 0.5, -0.5]], np.float32)
    packed, g = oracle.pack_ternary(W, "row", "binary")
    q = oracle.unpack_codes(packed, 8)
    np.testing.assert_array_equal(q, [[1, 1, 1, -1, 1, -1, 1, -1]])
    assert g[0] == oracle.absmean_scale(W[0])
    assert set(np.unique(packed)) <= {b for b in range(256)
                                      if all(((b >> (2 * j)) & 3) in (0, 2) for j in range(4))}


# ----------------------------------------------------------- activation quant

def test_act_quant_golden():
    for a, b in _golden("act_quant_cases.txt"):
        x = np.array([[float(v) for v in a.split(",")]], np.float32)
        want = np.array([[int(v) for v in b.split(",")]], np.int8)
        q, sx = oracle.quant_act_int8(x)
        np.testing.assert_array_equal(q, want)
        assert sx[0] == F32(1.0)


def test_act_quant_scale_is_one_division_golden():
    for a, b in _golden("act_quant_scale_cases.txt"):
        x = np.array([[float.fromhex(v.strip()) for v in a.split(",")]], np.float32)
        want = np.array([[int(v) for v in b.split(",")]], np.int8)
        q, _ = oracle.quant_act_int8(x)
        np.testing.assert_array_equal(q, want)


def test_act_quant_argmax_hits_127_and_bounds():
    X = ti.activations(11, 64, 777)
    q, sx = oracle.quant_act_int8(X)
    assert np.abs(q.astype(int)).max() <= 127
    am = np.argmax(np.abs(X), axis=1)
    np.testing.assert_array_equal(np.abs(q[np.arange(64), am]), 127)
    np.testing.assert_array_equal(np.sign(q[np.arange(64), am]),
                                  np.sign(X[np.arange(64), am]))


def test_act_quant_zero_token():
    q, sx = oracle.quant_act_int8(np.zeros((2, 16), np.float32))
    assert not q.any()
    np.testing.assert_array_equal(sx, np.float32(np.float32(1e-6) / np.float32(127)))


def test_act_quant_power_of_two_invariance():
    X = ti.activations(12, 8, 300, dtype="f32")
    q0, s0 = oracle.quant_act_int8(X)
    for k in (-20, -3, 1, 5, 30):
        q1, s1 = oracle.quant_act_int8(X * np.float32(2.0**k))
        np.testing.assert_array_equal(q0, q1)
        np.testing.assert_array_equal(s1, s0 * np.float32(2.0**k))


def test_act_quant_gain_clamp():
    # Hetman-2b s.8 test 4: a x500 input and a x1e-5 input hit the eta bounds
    rng = np.random.default_rng(42)
    big = (rng.standard_normal((2, 512)) * 500).astype(np.float32)
    tiny = (rng.standard_normal((2, 512)) * 1e-5).astype(np.float32)
    _, sb = oracle.quant_act_int8(big, bounds=(0.05, 40.0))
    _, st = oracle.quant_act_int8(tiny, bounds=(0.05, 40.0))
    np.testing.assert_array_equal(sb, np.float32(np.float32(40.0) / np.float32(127)))
    np.testing.assert_array_equal(st, np.float32(np.float32(0.05) / np.float32(127)))


def test_act_quant_scale_is_single_fp32_division():
    # s = fp32(127/eta), q = rint(fp32(x*s)); check one value by exact rationals
    x = np.array([[0.3, -1.7, 2.9]], np.float32)
    q, sx = oracle.quant_act_int8(x)
    eta = Fraction(float(F32(2.9)))
    s = oracle.round_rational_to_f32(*_nd(Fraction(127) / eta))
    for j in range(3):
        p = Fraction(float(x[0, j])) * Fraction(float(s))
        pr = oracle.round_rational_to_f32(*_nd(abs(p)))
        v = float(pr) * (1 if p >= 0 else -1)
        assert q[0, j] == int(np.rint(v))


# ------------------------------------------------------------------------ FWHT

def _golden_dict(name):
    return {a: b for a, b in _golden(name)}


def test_fwht_normalizer_constant():
    g = _golden_dict("fwht_constants.txt")
    assert abs(float(oracle.FWHT_NORM) - float(g["normalizer"])) < 1e-9
    assert oracle.FWHT_NORM == np.float32(1 / np.sqrt(512))


def test_fwht_basis_vectors_closed_form():
    # H e_j has entries (-1)^popcount(i & j), unnormalised, for every j
    E = np.eye(512, dtype=np.float32)
    Hx = oracle.fwht_block(E, normalize=False)      # row j = H e_j
    for j in range(512):
        i = np.arange(512)
        sign = np.array([(-1) ** bin(int(v)).count("1") for v in (i & j)], np.float32)
        np.testing.assert_array_equal(Hx[j], sign)


def test_fwht_integer_inputs_exact():
    # |x| <= 2^14: every partial sum is an integer below 2^24, so the fp32
    # butterfly equals the integer matrix product with the Sylvester matrix
    rng = np.random.default_rng(7)
    x = rng.integers(-2**14, 2**14 + 1, size=(6, 512)).astype(np.int64)
    H = oracle.hadamard_matrix(512)
    want = x @ H.T
    got = oracle.fwht_block(x.astype(np.float32), normalize=False)
    np.testing.assert_array_equal(got.astype(np.int64), want)


def test_fwht_isometry_involution_spike():
    g = _golden_dict("fwht_constants.txt")
    rng = np.random.default_rng(42)
    x = rng.standard_normal((8, 512)).astype(np.float32)
    y = oracle.fwht_block(x, normalize=True)
    assert np.max(np.abs(np.linalg.norm(x, axis=1) - np.linalg.norm(y, axis=1))) \
        < float(g["isometry_tol"])
    assert np.max(np.abs(oracle.fwht_block(y, normalize=True) - x)) \
        < float(g["involution_tol"])
    spike = np.zeros((1, 512), np.float32)
    spike[0, int(g["spike_index"])] = float(g["spike_value"])
    s = oracle.fwht_block(spike, normalize=True)
    peak = float(np.max(np.abs(s)))
    assert abs(peak - float(g["spike_peak"])) < float(g["spike_tol"])
    assert abs(100.0 / peak - float(g["attenuation"])) < 0.01
    # signs: + for i < 256, - for i >= 256 (popcount of i & 256)
    v = np.float32(np.float32(100.0) * oracle.FWHT_NORM)
    np.testing.assert_array_equal(s[0, :256], v)
    np.testing.assert_array_equal(s[0, 256:], -v)


def test_fwht_blockwise_independent_blocks():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((3, 2048)).astype(np.float32)
    y = oracle.fwht512(x, normalize=True)
    for b in range(4):
        np.testing.assert_array_equal(
            y[:, 512 * b:512 * (b + 1)],
            oracle.fwht_block(x[:, 512 * b:512 * (b + 1)], normalize=True))
    with pytest.raises(ValueError):
        oracle.fwht512(np.zeros((1, 500), np.float32))


# ------------------------------------------------------------ prologue

def _is_nearest_f32(v, exact):
    """v is the fp32 nearest to the rational `exact`, ties to the even
    significand (checked with exact rationals against both neighbours)."""
    v = F32(v)
    up = np.nextafter(v, F32(np.inf))
    dn = np.nextafter(v, F32(0)) if v > 0 else F32(0)
    d0 = abs(Fraction(float(v)) - exact)
    du = abs(Fraction(float(up)) - exact)
    dd = abs(Fraction(float(dn)) - exact)
    if d0 > du or d0 > dd:
        return False
    if d0 == du or (v > 0 and d0 == dd):
        return (int(np.array([v]).view(np.uint32)[0]) & 1) == 0
    return True


def test_mean_of_squares_is_the_nearest_fp32_to_the_exact_mean():
    rng = np.random.default_rng(4)
    rows = [rng.standard_normal(512), rng.standard_t(3, 4096), rng.standard_normal(3) * 1e-3,
            rng.standard_normal(64) * 2.0**-60, rng.standard_normal(7) * 2.0**40,
            np.array([3.0]), rng.standard_t(1, 1000)]
    for x in rows:
        x = np.asarray(x, np.float32)
        sq = [Fraction(float(v)) for v in (x * x).astype(np.float32)]
        exact = sum(sq, Fraction(0)) / len(sq)
        assert _is_nearest_f32(oracle.mean_of_squares(x), exact)
    g = _golden_dict("prologue_cases.txt")
    for key in ("tie_even", "tie_above", "fp64_wrong"):
        xs, want = g[key].split("->")
        x = np.array([float.fromhex(v.strip()) if "p" in v else float(v)
                      for v in xs.split(",")], np.float32)
        assert oracle.mean_of_squares(x) == F32(float.fromhex(want.strip()) if "p" in want
                                                else float(want))


def _decimal_rsqrt(var, eps):
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    return float(1 / (Decimal(float(var)) + Decimal(float(eps))).sqrt())


def test_rms_factor_exact_cases_and_ulp_bound():
    # all |x| = 16: the mean is 256 exactly, fp32(256 + 1e-6) = 256 (1e-6 is
    # below half the spacing 2^-15), sqrt 16, r = 1/16 exactly
    x = np.where(np.arange(512) % 3 == 0, -16.0, 16.0).astype(np.float32)
    assert oracle.rms_factor(x) == F32(0.0625)
    # all x = 2^-10: the mean is 2^-20 and eps is about as large, so it must
    # enter: r = 1/sqrt(2^-20 + fp32(1e-6)), not 1024
    x = np.full(64, 2.0**-10, np.float32)
    r = oracle.rms_factor(x)
    want = _decimal_rsqrt(2.0**-20, F32(1e-6))
    assert abs(float(r) - want) <= 2 * float(np.spacing(F32(want)))
    assert abs(float(r) - 1024.0) > 100
    # random tokens: three roundings after the exact mean, within 2 ulp
    rng = np.random.default_rng(5)
    for scale in (1.0, 1e-3, 30.0):
        x = (rng.standard_t(3, 2048) * scale).astype(np.float32)
        var = sum((Fraction(float(v)) for v in (x * x).astype(np.float32)), Fraction(0)) / x.size
        want = _decimal_rsqrt(float(var), F32(1e-6))
        r = oracle.rms_factor(x)
        assert abs(float(r) - want) <= 2 * float(np.spacing(F32(want)))


def _nearest_f32(exact):
    """fp32 nearest to a non-negative rational or Decimal `exact` (ties to
    even), found by comparing it with the neighbours of a float guess."""
    from decimal import Decimal
    ex = Fraction(exact) if not isinstance(exact, Decimal) else Fraction(str(exact))
    v = F32(float(ex))
    for _ in range(4):
        up, dn = np.nextafter(v, F32(np.inf)), np.nextafter(v, F32(0))
        if abs(Fraction(float(up)) - ex) < abs(Fraction(float(v)) - ex):
            v = up
        elif abs(Fraction(float(dn)) - ex) < abs(Fraction(float(v)) - ex):
            v = dn
        else:
            break
    for w in (np.nextafter(v, F32(np.inf)), np.nextafter(v, F32(0))):
        if abs(Fraction(float(w)) - ex) == abs(Fraction(float(v)) - ex):
            if int(np.array([w]).view(np.uint32)[0]) % 2 == 0:
                v = w
    return v


def _rmsnorm_by_rationals(x, g):
    """Hetman-2b s.4 evaluated on exact rationals, rounding to fp32 after
    each operation the page performs in fp32, left to right:
    var = mean(x^2), rsqrt(var + eps), then x * rsqrt * weight."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    sq = [_nearest_f32(Fraction(float(v)) ** 2) for v in x]
    var = _nearest_f32(sum((Fraction(float(v)) for v in sq), Fraction(0)) / len(sq))
    t = _nearest_f32(Fraction(float(var)) + Fraction(float(F32(1e-6))))
    root = _nearest_f32(Decimal(float(t)).sqrt())
    r = _nearest_f32(1 / Fraction(float(root)))
    out = []
    for v, w in zip(x, g):
        a = _nearest_f32(abs(Fraction(float(v)) * Fraction(float(r))))
        a = a if v >= 0 else -a
        b = _nearest_f32(abs(Fraction(float(a)) * Fraction(float(w))))
        out.append(b if (a >= 0) == (w >= 0) else -b)
    return r, np.array(out, np.float32)


def test_rmsnorm_matches_the_page_expression_on_rationals():
    rng = np.random.default_rng(72)
    for i in range(24):
        K = int(rng.choice([4, 9, 64]))
        x = (rng.standard_t(3, K) * 10.0 ** rng.uniform(-3, 2)).astype(np.float32)
        g = rng.uniform(0.25, 3.0, K).astype(np.float32)
        r, want = _rmsnorm_by_rationals(x, g)
        assert oracle.rms_factor(x) == r, i
        np.testing.assert_array_equal(oracle.rmsnorm(x, g)[0], want)


def test_act_quant_codes_on_rationals_sweep():
    # s = fp32(127 / eta) and q = rint(fp32(x * s)) evaluated on exact
    # rationals for many tokens: a scale formed as 1 / (eta / 127), or a
    # product rounded differently, moves some of these codes
    rng = np.random.default_rng(73)
    X = (rng.standard_normal((120, 48)) * 10.0 ** rng.uniform(-2, 2, (120, 1))).astype(np.float32)
    q, sx = oracle.quant_act_int8(X)
    for i in range(X.shape[0]):
        eta = Fraction(float(np.max(np.abs(X[i]))))
        s = Fraction(float(_nearest_f32(127 / eta)))
        for k in range(X.shape[1]):
            p = Fraction(float(X[i, k])) * s
            a = Fraction(float(_nearest_f32(abs(p))))
            want = _round_half_even(a) * (1 if p >= 0 else -1)
            assert q[i, k] == max(-127, min(127, want)), (i, k)
        assert sx[i] == _nearest_f32(eta / 127)


def test_rmsnorm_weight_is_applied_per_element():
    X = ti.activations(71, 3, 1024, dist="student_t3")
    base = oracle.rmsnorm(X)
    np.testing.assert_array_equal(oracle.rmsnorm(X, -np.ones(1024, np.float32)), -base)
    np.testing.assert_array_equal(oracle.rmsnorm(X, np.full(1024, 8.0, np.float32)), base * 8)
    onehot = np.zeros(1024, np.float32)
    onehot[613] = 1.0
    y = oracle.rmsnorm(X, onehot)
    assert np.count_nonzero(y[:, np.arange(1024) != 613]) == 0
    np.testing.assert_array_equal(y[:, 613], base[:, 613])


def test_prologue_spike_golden():
    g = _golden_dict("prologue_cases.txt")
    x = np.zeros((1, 512), np.float32)
    x[0, int(g["spike_index"])] = float(g["spike_value"])
    assert oracle.mean_of_squares(x[0]) == F32(float(g["spike_var"]))
    q, sx = oracle.bitlinear_prologue(x)
    want = np.concatenate([np.full(256, 127), np.full(256, -127)]).astype(np.int8)
    np.testing.assert_array_equal(q[0], want)
    assert sx[0] == _f32(int(g["spike_sx_bits"], 16))
    assert sx[0] == F32(F32(float(g["spike_eta"])) / F32(127))


def _round_half_even(fr):
    f = fr.numerator // fr.denominator
    rem = fr - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2):
        return f + 1
    return f


def test_prologue_integer_tokens_against_exact_rationals():
    # tokens of +-16: RMSNorm gives r = 1/16 exactly and +-1 values, the
    # unnormalised transform z = H x is the integer Sylvester product, and
    # every code is 127 z / max|z| rounded, up to the fp32 products' few ulp
    # (only codes within 1e-4 of a half-integer may differ, by one)
    rng = np.random.default_rng(61)
    X = (rng.choice([-16.0, 16.0], size=(4, 1024))).astype(np.float32)
    H = oracle.hadamard_matrix(512)
    q, sx = oracle.bitlinear_prologue(X)
    for i in range(4):
        z = np.concatenate([H @ (X[i, b * 512:(b + 1) * 512] / 16).astype(np.int64)
                            for b in range(2)])
        zmax = int(np.max(np.abs(z)))
        exact_eta = zmax / np.sqrt(512.0)
        assert abs(float(sx[i]) - exact_eta / 127) <= 1e-6 * exact_eta / 127
        for k in range(1024):
            v = Fraction(127 * int(z[k]), zmax)
            dist = abs(v - (v.numerator // v.denominator) - Fraction(1, 2))
            if dist > Fraction(1, 10000):
                assert q[i, k] == _round_half_even(v), (i, k)
            else:
                assert abs(int(q[i, k]) - _round_half_even(v)) <= 1


def test_prologue_matches_fp64_chain_up_to_boundaries():
    X = ti.activations(5105, 64, 4096, dist="student_t3")
    q, sx = oracle.bitlinear_prologue(X)
    ql, sxl = oracle.bitlinear_prologue_fp64(X)
    d = np.abs(q.astype(int) - ql.astype(int))
    assert d.max() <= 1
    assert np.mean(d) < 1e-3
    np.testing.assert_allclose(sx, sxl, rtol=1e-6)


def test_prologue_clamp_bound_tokens():
    rng = np.random.default_rng(9)
    K = 4096
    H = oracle.hadamard_matrix(512)
    # (a) upper clamp: one block carries 8 x a Hadamard row, the rest is zero;
    # after RMSNorm and the rotation its energy sits in one value, 64 > 40
    xa = np.zeros(K, np.float32)
    xa[1024:1536] = (H[37] * 2.0**3).astype(np.float32)
    # (b) lower clamp: all |x| = 2^-20, so eps dominates RMSNorm's denominator
    xb = (rng.choice([-1.0, 1.0], size=K) * 2.0**-20).astype(np.float32)
    # (c) zero token
    xc = np.zeros(K, np.float32)
    X = np.stack([xa, xb, xc])
    q, sx = oracle.bitlinear_prologue(X)
    assert sx[0] == F32(F32(40.0) / F32(127))
    assert sx[1] == F32(F32(0.05) / F32(127))
    assert sx[2] == F32(F32(0.05) / F32(127))
    assert not q[2].any()
    nz = np.nonzero(q[0])[0]
    np.testing.assert_array_equal(nz, [1024 + 37])
    assert q[0, 1024 + 37] == 127
    ql, _ = oracle.bitlinear_prologue_fp64(X)
    assert np.abs(q.astype(int) - ql.astype(int)).max() <= 1


def test_prologue_off_reduces_to_plain_quantiser():
    X = ti.activations(91, 6, 1024, dtype="f32")
    X[2] = 0
    q0, s0 = oracle.quant_act_int8(X)
    q1, s1 = oracle.bitlinear_prologue(X, bounds=None, rmsnorm_on=False, fwht=False)
    np.testing.assert_array_equal(q0, q1)
    np.testing.assert_array_equal(s0, s1)
    q2, s2 = oracle.quant_act_int8(X * 100, bounds=(0.05, 40.0))
    q3, s3 = oracle.bitlinear_prologue(X * 100, rmsnorm_on=False, fwht=False)
    np.testing.assert_array_equal(q2, q3)
    np.testing.assert_array_equal(s2, s3)


def test_prologue_rmsnorm_of_power_of_two_magnitudes():
    # every |x| = 2^a (a >= 3): the mean of squares is 4^a exactly, eps is
    # below half its spacing, r = 2^-a exactly, so RMSNorm only rescales by a
    # power of two and the codes are the plain quantiser's codes of x
    rng = np.random.default_rng(93)
    for a in (3, 7):
        X = (rng.choice([-1.0, 1.0], size=(3, 640)) * 2.0**a).astype(np.float32)
        q0, s0 = oracle.quant_act_int8(X)
        q1, s1 = oracle.bitlinear_prologue(X, bounds=None, fwht=False)
        np.testing.assert_array_equal(q0, q1)
        np.testing.assert_array_equal(s1, s0 * F32(2.0**-a))


def test_prologue_fwht_of_integer_tokens_is_exact():
    # without RMSNorm, |x| <= 2^14 integers: the transform is exact and the
    # codes are those of the plain quantiser applied to fp32(z * c)
    rng = np.random.default_rng(94)
    X = rng.integers(-2**10, 2**10, size=(3, 1024)).astype(np.float32)
    H = oracle.hadamard_matrix(512)
    z = np.concatenate([X[:, :512].astype(np.int64) @ H.T,
                        X[:, 512:].astype(np.int64) @ H.T], axis=1)
    xr = (z.astype(np.float32) * oracle.FWHT_NORM).astype(np.float32)
    q0, s0 = oracle.quant_act_int8(xr, bounds=(0.05, 40.0))
    q1, s1 = oracle.bitlinear_prologue(X, rmsnorm_on=False)
    np.testing.assert_array_equal(q0, q1)
    np.testing.assert_array_equal(s0, s1)


# ------------------------------------------------------------ contraction

def _gather_reference(q, w):
    # BitRASP additive_ternary_linear_int8: sum of x where W = +1 minus sum
    # of x where W = -1, written independently here
    M, N = q.shape[0], w.shape[0]
    out = np.zeros((M, N), np.int64)
    for o in range(N):
        pos = np.nonzero(w[o] == 1)[0]
        neg = np.nonzero(w[o] == -1)[0]
        out[:, o] = q[:, pos].astype(np.int64).sum(1) - q[:, neg].astype(np.int64).sum(1)
    return out


def test_contraction_three_references_agree():
    for (M, N, K, seed) in [(1, 3, 4, 1), (3, 17, 60, 2), (5, 33, 260, 3), (2, 64, 1024, 4)]:
        q = ti.random_int8(seed, M, K)
        w = ti.random_ternary(seed + 100, N, K)
        packed = oracle.pack_codes(w)
        acc = oracle.contract(q, packed, K)
        np.testing.assert_array_equal(acc, _gather_reference(q, w))
        if M * N * K <= 3 * 17 * 60:
            for m in range(M):
                for o in range(N):
                    assert acc[m, o] == sum(int(q[m, k]) * int(w[o, k]) for k in range(K))


def test_contraction_equals_int64_product_at_scale():
    # the float64 product is exact for integer operands: check it against
    # numpy's int64 matrix product (integer arithmetic, no rounding) on
    # shapes with several thousand terms per sum and extreme values
    rng = np.random.default_rng(41)
    for (M, N, K) in [(7, 40, 16384), (33, 257, 4096), (2, 5, 6912)]:
        q = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
        q[0] = 127
        if M > 1:
            q[1] = -128
        w = ti.random_ternary(M + N + K, N, K)
        w[0] = 1
        w[-1] = -1
        want = q.astype(np.int64) @ w.astype(np.int64).T
        np.testing.assert_array_equal(oracle.contract(q, oracle.pack_codes(w), K), want)
    b = np.where(rng.standard_normal((9, 1024)) >= 0, 1, -1).astype(np.int8)
    q = rng.integers(-127, 128, size=(3, 1024)).astype(np.int8)
    np.testing.assert_array_equal(oracle.contract_signs(q, oracle.pack_signs(b), 1024),
                                  q.astype(np.int64) @ b.astype(np.int64).T)


def test_bf16_rounding_golden():
    for a, b in _golden("bf16_rounding.txt"):
        got = oracle.bf16_round_from_f64(np.array([float.fromhex(a)]))[0]
        assert float(got) == float.fromhex(b), a


def test_contraction_all_plus_one_and_bounds():
    q = ti.random_int8(20, 4, 512)
    w = np.ones((3, 512), np.int8)
    acc = oracle.contract(q, oracle.pack_codes(w), 512)
    np.testing.assert_array_equal(acc, np.repeat(q.astype(np.int64).sum(1)[:, None], 3, 1))
    q = np.full((1, 6912), 127, np.int8)
    w = -np.ones((1, 6912), np.int8)
    acc = oracle.contract(q, oracle.pack_codes(w), 6912)
    assert acc[0, 0] == -127 * 6912 and abs(acc[0, 0]) < 2**24


def test_epilogue_identity_and_zero():
    q = ti.random_int8(30, 3, 64)
    w = ti.random_ternary(31, 5, 64)
    acc = oracle.contract(q, oracle.pack_codes(w), 64)
    g = np.array([0.0123], np.float32)
    sx = np.array([0.01, 0.02, 0.5], np.float32)
    y = oracle.epilogue(acc, g, sx)
    np.testing.assert_allclose(y / (float(g[0]) * sx.astype(np.float64)[:, None]), acc,
                               rtol=1e-15)
    assert np.all(y[acc == 0] == 0)


def test_whole_layer_tiny_matches_gemv_emulation():
    # Hetman-2b s.7 GEMV semantics: per row, per packed byte, decode four
    # weights, accumulate in integers, scale once.  Written out here with
    # Python integers for a few rows of the tiny workload.
    W = ti.workload_weights("tiny")
    X = ti.workload_activations("tiny")
    r = oracle.ternary_linear(X, W)
    for m in range(X.shape[0]):
        for o in (0, 1, 77, 255):
            acc = 0
            for j, byte in enumerate(r["packed"][o]):
                for s in range(4):
                    code = (int(byte) >> (2 * s)) & 3
                    acc += int(r["q"][m, 4 * j + s]) * (code - 1)
            assert acc == r["acc"][m, o]
            y = float(acc) * float(r["scale"][0]) * float(r["sx"][m])
            assert abs(y - r["y"][m, o]) <= 1e-12 * max(1.0, abs(y))


# ---------------------------------------------------------------- 1-bit signs

def test_sign_pack_golden_sizes_and_bytes():
    for a, b in _golden("sign_pack.txt"):
        kind, *vals = a.split()
        if kind == "size":
            R, C = int(vals[0]), int(vals[1])
            nbytes, sbytes, mb, ratio = b.split()
            packed = oracle.packed1_bytes(R * C)
            assert packed == int(nbytes) == R * C // 8
            assert 4 * R == int(sbytes)
            assert f"{(packed + 4 * R) / 1e6:.2f}" == mb
            assert f"{4 * R * C / (packed + 4 * R):.1f}" == ratio
        else:
            v = np.array([int(x) for x in vals], dtype=np.int8)
            assert int(oracle.pack_signs(v)[0, 0]) == int(b, 16)


def test_sign_pack_roundtrip_and_rejects():
    rng = np.random.default_rng(5)
    b = np.where(rng.random((7, 64)) < 0.5, 1, -1).astype(np.int8)
    assert np.array_equal(oracle.unpack_signs(oracle.pack_signs(b), 64), b)
    with pytest.raises(ValueError):
        oracle.pack_signs(np.ones((1, 12), np.int8))
    with pytest.raises(ValueError):
        oracle.pack_signs(np.zeros((1, 8), np.int8))


def test_binary1_agrees_with_two_bit_binary():
    # the same binary weights and scales as the 2-bit binary mode, only the
    # storage differs
    W = ti.normal_weights(77, 24, 96)
    W[0, :5] = 0.0
    W[1, 3] = -0.0
    p1, s1 = oracle.pack_binary1(W, "row")
    p2, s2 = oracle.pack_ternary(W, "row", mode="binary")
    assert np.array_equal(oracle.unpack_signs(p1, 96), oracle.unpack_codes(p2, 96))
    assert np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    assert oracle.unpack_signs(p1, 96)[0, :5].tolist() == [1] * 5   # sign(0) -> +1
    assert oracle.unpack_signs(p1, 96)[1, 3] == 1                   # -0.0 -> +1


def test_contract_signs_brute_force_and_identity():
    rng = np.random.default_rng(6)
    M, N, K = 3, 5, 40
    q = rng.integers(-127, 128, (M, K)).astype(np.int8)
    b = np.where(rng.random((N, K)) < 0.5, 1, -1).astype(np.int8)
    acc = oracle.contract_signs(q, oracle.pack_signs(b), K)
    for m in range(M):
        for o in range(N):
            ref = 0
            for k in range(K):
                ref += int(q[m, k]) * int(b[o, k])
            assert acc[m, o] == ref
            plus = sum(int(q[m, k]) for k in range(K) if b[o, k] == 1)
            assert acc[m, o] == 2 * plus - int(q[m].astype(np.int64).sum())


# ---------------------------------------------------------------- SwiGLU clamp

def test_swiglu_clamped_closed_forms():
    from scipy.special import expit
    g = np.array([-30.0, -3.0, -0.5, 0.0, 0.5, 3.0, 30.0])
    u = np.array([2.0, -1.5, 4.0, 7.0, -2.0, 0.25, 0.1])
    h = oracle.swiglu_clamped(g, u)
    # silu(g) = g * sigmoid(g) through an independent library sigmoid
    ref = np.clip(g * expit(g) * u, -10.0, 10.0)
    np.testing.assert_allclose(h, ref, rtol=1e-14, atol=0)
    assert h[3] == 0.0                                  # silu(0) = 0
    # silu(g) - silu(-g) = g (odd part of g * sigmoid(g))
    gg = np.linspace(-8, 8, 33)
    one = np.ones_like(gg)
    np.testing.assert_allclose(oracle.swiglu_clamped(gg, one, 1e9) -
                               oracle.swiglu_clamped(-gg, one, 1e9), gg, atol=1e-12)
    # the clamp binds at exactly +-10 and only there
    big = oracle.swiglu_clamped(np.array([20.0, 20.0, 4.0]), np.array([3.0, -3.0, 1.0]))
    assert big[0] == 10.0 and big[1] == -10.0 and abs(big[2] - 4.0 * expit(4.0)) < 1e-14


def test_ffn_swiglu_decode_matches_stepwise_float_reference():
    # the whole FFN against float matrix products of the unpacked weights
    rng = np.random.default_rng(9)
    d, f, M = 64, 96, 3
    X = rng.standard_normal((M, d)).astype(np.float32)
    mats = []
    for (n, k), seed in (((f, d), 1), ((f, d), 2), ((d, f), 3)):
        mats.append(oracle.pack_ternary(ti.normal_weights(50 + seed, n, k), "row"))
    h, g, u, y = oracle.ffn_swiglu_decode(X, *mats)
    q, sx = oracle.quant_act_int8(X)
    wg = oracle.unpack_codes(mats[0][0], d).astype(np.float64) * mats[0][1][:, None]
    wu = oracle.unpack_codes(mats[1][0], d).astype(np.float64) * mats[1][1][:, None]
    xq = q.astype(np.float64) * sx[:, None].astype(np.float64)
    np.testing.assert_allclose(g, xq @ wg.T, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(u, xq @ wu.T, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(h, np.clip(g / (1 + np.exp(-g)) * u, -10, 10), rtol=1e-14)
    hq, hs = oracle.quant_act_int8(h.astype(np.float32))
    wd = oracle.unpack_codes(mats[2][0], f).astype(np.float64) * mats[2][1][:, None]
    np.testing.assert_allclose(y, (hq.astype(np.float64) * hs[:, None]) @ wd.T, rtol=1e-12,
                               atol=1e-15)


# ---------------------------------------------------------------- backward

def test_backward_adjoint_identities():
    # the layer y = gamma * X w^T is linear in X and in W: its gradients are
    # fixed by <dY, y(V)> = <dX, V> and <dY, X U^T> = <dW, U> for any V, U
    rng = np.random.default_rng(11)
    M, N, K = 5, 7, 24
    w = ti.random_ternary(12, N, K)
    packed = oracle.pack_codes(w)
    for gam in (np.array([0.37], np.float32), (rng.random(N) + 0.5).astype(np.float32)):
        dY = rng.standard_normal((M, N))
        V = rng.standard_normal((M, K))
        g = gam.astype(np.float64) if gam.size > 1 else np.full(N, float(gam[0]))
        yV = V @ (w.astype(np.float64) * g[:, None]).T        # y(V) = gamma * V w^T
        dX = oracle.backward_input(dY, packed, gam, K)
        assert abs(np.sum(dY * yV) - np.sum(dX * V)) < 1e-10 * np.sum(np.abs(dY * yV))
    X = rng.standard_normal((M, K))
    U = rng.standard_normal((N, K))
    dW = oracle.backward_weight(X, dY)
    assert dW.shape == (N, K)
    assert abs(np.sum(dY * (X @ U.T)) - np.sum(dW * U)) < 1e-10 * np.sum(np.abs(dY * (X @ U.T)))


def test_backward_brute_force():
    rng = np.random.default_rng(13)
    M, N, K = 2, 3, 8
    w = ti.random_ternary(14, N, K)
    packed = oracle.pack_codes(w)
    gam = np.array([0.5, 2.0, 0.25], np.float32)
    dY = rng.standard_normal((M, N))
    X = rng.standard_normal((M, K))
    dX = oracle.backward_input(dY, packed, gam, K)
    dW = oracle.backward_weight(X, dY)
    for m in range(M):
        for k in range(K):
            ref = 0.0
            for n in range(N):
                ref += dY[m, n] * float(gam[n]) * int(w[n, k])
            assert abs(dX[m, k] - ref) < 1e-12
    for n in range(N):
        for k in range(K):
            ref = sum(dY[m, n] * X[m, k] for m in range(M))
            assert abs(dW[n, k] - ref) < 1e-12


# ----------------------------------------------------- thresholds and formats

def test_code_formats_golden():
    for a, b in _golden("code_formats.txt"):
        kind, *vals = a.split()
        if kind == "enc":
            v = np.array([int(x) for x in vals], dtype=np.int8)
            for fmt, hx in zip(("native", "f0", "f1"), b.split()):
                byte = oracle.encode_format(v, fmt)
                assert int(byte[0, 0]) == int(hx, 16), (vals, fmt)
                assert np.array_equal(oracle.decode_format(byte, fmt)[0], v)
        else:
            fmt, hx = vals
            got = oracle.decode_format(np.array([int(hx, 16)], np.uint8), fmt)[0]
            assert got.tolist() == [int(x) for x in b.split()]


def test_code_formats_roundtrip_and_conversion():
    q = ti.random_ternary(21, 9, 64)
    enc = {f: oracle.encode_format(q, f) for f in oracle.FORMATS}
    assert np.array_equal(enc["native"], oracle.pack_codes(q))
    for f in oracle.FORMATS:
        assert np.array_equal(oracle.decode_format(enc[f], f), q)
        for g in oracle.FORMATS:
            assert np.array_equal(oracle.convert_codes(enc[f], f, g), enc[g])
    # Format 0 is the two's-complement low bits of the value (the page's w & 3)
    for v in (-1, 0, 1):
        assert int(oracle.encode_format(np.full(4, v, np.int8), "f0")[0, 0]) == \
            sum((v & 3) << (2 * i) for i in range(4))
    # every byte decodes to values in {-1, 0, 1}, and re-encoding a decoded
    # byte maps reserved codes to the format's zero code
    allb = np.arange(256, dtype=np.uint8).reshape(1, -1)
    for f in oracle.FORMATS:
        v = oracle.decode_format(allb, f)
        assert set(np.unique(v)) <= {-1, 0, 1}
        again = oracle.encode_format(v, f)
        assert np.array_equal(oracle.decode_format(again, f), v)


def test_thresholds_golden():
    for a, b, c in (line.split(";") for line in _golden_lines("thresholds.txt")):
        kind, value, *w = a.split()
        W = np.array([[float(x) for x in w]], dtype=np.float32)
        q, sc = oracle.ternarize_threshold(W, "tensor", kind, float(value))
        assert q[0].tolist() == [int(x) for x in b.split()], a
        assert float(sc[0]) == float(c)


def test_threshold_half_factor_is_the_rounding_rule():
    # |w| > gamma/2 is round(w/gamma) != 0 (ties to even put 0.5 at 0), and
    # fp32(0.5) * gamma = gamma/2 exactly: the two routes must agree
    for gran in ("tensor", "row"):
        W = ti.normal_weights(22, 64, 256)
        q, sc = oracle.ternarize_threshold(W, gran, "relative", 0.5)
        gam = oracle.absmean_scales(W, gran)
        assert np.array_equal(q, oracle.ternarize(W, gam))
        assert np.array_equal(sc, gam)
    # exact ties at gamma/2 stay zero on both routes
    W = np.array([[0.5, -0.5, 1.5, -1.5]], np.float32)      # gamma = 1
    q, _ = oracle.ternarize_threshold(W, "tensor", "relative", 0.5)
    assert q[0].tolist() == oracle.ternarize(W, np.array([1.0], np.float32))[0].tolist() == [0, 0, 1, -1]


def test_threshold_monotone_and_brute_force():
    W = ti.normal_weights(23, 16, 128)
    prev = None
    for f in (0.0, 0.3, 0.55, 1.0, 2.0):
        q, gam = oracle.ternarize_threshold(W, "row", "relative", f)
        nz = np.count_nonzero(q)
        if prev is not None:
            assert nz <= prev
        prev = nz
        if f == 0.0:
            assert np.array_equal(q, np.sign(W).astype(np.int8))
        for i in range(0, 16, 5):
            h = np.float32(np.float32(f) * gam[i])
            for j in range(0, 128, 7):
                w = W[i, j]
                assert q[i, j] == (1 if w > h else (-1 if w < -h else 0))
    q, sc = oracle.ternarize_threshold(W, "tensor", "absolute", 0.01)
    assert float(sc[0]) == float(np.float32(0.01))
    assert np.array_equal(q, (W > np.float32(0.01)).astype(np.int8) - (W < -np.float32(0.01)).astype(np.int8))
