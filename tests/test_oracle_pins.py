"""The fp64 oracle against its pins (closed forms, exact rational brute force,
invariants and the golden PR's printed geometry).  CPU only."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    return oracle.Oracle()


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def test_round_bf16_matches_definition():
    """Nearest bf16 (8 significant bits, ties to even): 1 + 2^-8 is a tie that
    goes down to 1, 1 + 3*2^-8 goes up to 1 + 2^-6, 1 + 2^-8 + 2^-30 goes up."""
    import numpy as np
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -30, -3.0, 0.0, 255.5])
    want = np.array([1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -3.0, 0.0, 256.0])
    assert np.array_equal(oracle.round_bf16(x), want)


def test_round_bf16_against_significand_form():
    """The bit-level rounding equals rint(m * 256) / 256 * 2^e (x = m 2^e, 1/2 <= |m| < 1)
    on values across 60 binades and on every kind of tie: odd 9-bit significands (exact
    ties, both signs) and their neighbours one fp64 ulp away."""
    import numpy as np
    rng = np.random.default_rng(7)

    def significand_form(x):
        m, e = np.frexp(x)
        return np.ldexp(np.rint(m * 256.0) / 256.0, e)

    x = rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000)
    ties = np.ldexp((2 * rng.integers(128, 256, 4000) + 1) / 512.0, rng.integers(-40, 40, 4000))
    probe = np.concatenate([x, ties, -ties, np.nextafter(ties, np.inf), np.nextafter(ties, -np.inf)])
    assert np.array_equal(oracle.round_bf16(probe), significand_form(probe))
