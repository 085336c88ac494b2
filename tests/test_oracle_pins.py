"""The oracle against its pins (CPU only)."""

import numpy as np
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.FAST_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


@pytest.mark.slow
def test_f32_to_f16_exhaustive(orc):
    """All 2^32 binary32 bit patterns against torch's CPU conversion."""
    step = 1 << 26
    for start in range(0, 1 << 32, step):
        pats = np.arange(start, start + step, dtype=np.uint64).astype(np.uint32)
        P.check_f32_to_f16_chunk(orc, pats)


def test_quantize_rejects_bad_arguments(orc):
    w = np.ones((2, 4), dtype=np.float32)
    for pct in (0.0, -1.0, 100.5, float("nan")):
        with pytest.raises(ValueError):
            orc.quantize(w, pct)
    bad = w.copy()
    bad[1, 2] = np.inf
    with pytest.raises(ValueError):
        orc.quantize(bad, 100.0)


def test_quantize_fixed_rejects_bad_bounds(orc):
    w = np.ones((2, 4), dtype=np.float32)
    for b in ([1.0, -1.0], [1.0, np.inf], [np.nan, 1.0]):
        with pytest.raises(ValueError):
            orc.quantize_fixed(w, np.float32(b))
