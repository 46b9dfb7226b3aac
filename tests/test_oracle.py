"""The CPU oracle against its pins (see oracle_pins.py), and the proof that
the pins catch a planted mistake anywhere in the oracle."""
import numpy as np
import pytest

import oracle
import oracle_pins

N_MUTANTS = 21


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle_lib, pin):
    ok, detail = pin(0)
    assert ok, detail


@pytest.mark.parametrize("mutant", range(1, N_MUTANTS + 1))
def test_planted_mistake_is_caught(mutant):
    oracle.build(mutant, force=False)
    failed = []
    for pin in oracle_pins.PINS:
        try:
            ok, _ = pin(mutant)
        except Exception:  # a crash also counts as caught
            ok = False
        if not ok:
            failed.append(pin.__name__)
    assert failed, f"mutant {mutant} passes every pin"


def test_pool_placement_roundtrip():
    H, P, dh, pages = 2, 4, 3, 6
    pool = np.full(2 * pages * H * P * dh, -1.0)
    pt = np.array([4, 1, 5])
    rows = np.arange(10 * H * dh, dtype=np.float64).reshape(10, H * dh)
    oracle.pool_place(pool, 1, pt, 0, rows[:7], pages, H, P, dh)
    oracle.pool_place(pool, 1, pt, 7, rows[7:], pages, H, P, dh)
    back = oracle.pool_read(pool, 1, pt, 10, pages, H, P, dh)
    assert np.array_equal(back, rows)
    # hand-worked offset: layer 1, page 5, head 1, slot 1 -> position 9, head 1
    off = ((((1 * pages + 5) * H + 1) * P + 1) * dh)
    assert np.array_equal(pool[off:off + dh], rows[9, dh:2 * dh])
    # layer 0 untouched
    assert np.all(pool[:pages * H * P * dh] == -1.0)
