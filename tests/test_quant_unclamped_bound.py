"""The per-token quantiser's codes need no clamp when eta >= max|x|.

With s = fp32(127 / eta) and |x| <= eta, fp32(x * s) is at most
127 * (1 + 2^-24) before rounding, hence at most 127 + 2^-17 after it, and
rounds half to even to a code in [-127, 127].  The single-token GEMV kernels
rely on this to skip the clamp when no gain clamp is set.  This checks the
bound in float32 arithmetic on many eta (normal, subnormal, extreme) at
x = eta and the neighbouring values below it.
"""
import numpy as np
import pytest

F32 = np.float32


def _codes(x, eta):
    s = F32(127.0) / eta                      # fp32, correctly rounded
    t = (x * s).astype(np.float32)            # fp32 product
    return np.rint(t.astype(np.float64)), t


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_codes_stay_within_127_without_clamp(seed):
    rng = np.random.default_rng(seed)
    # eta across the fp32 range: random bit patterns of positive finite floats
    bits = rng.integers(0x00000001, 0x7F7FFFFF, size=400_000, dtype=np.uint32)
    eta = bits.view(np.float32)
    eta = eta[(eta >= F32(1e-30)) & (eta <= F32(1e30))]
    for x in (eta, np.nextafter(eta, F32(0)), np.nextafter(np.nextafter(eta, F32(0)), F32(0))):
        q, t = _codes(x.astype(np.float32), eta)
        assert np.all(np.abs(t) <= F32(127.0) + F32(2.0 ** -17))
        assert np.all(np.abs(q) <= 127)
        q, _ = _codes(-x.astype(np.float32), eta)
        assert np.all(np.abs(q) <= 127)


def test_codes_at_eta_are_127():
    # x = eta gives the extreme code exactly (the argmax element of a token)
    eta = np.array([1e-6, 0.05, 0.3, 1.0, 3.14159, 40.0, 1e4, 7e20], dtype=np.float32)
    q, _ = _codes(eta, eta)
    np.testing.assert_array_equal(q, 127)
