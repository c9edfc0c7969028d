"""The oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins as op


@pytest.fixture(scope="module")
def orc():
    return oracle.load()


@pytest.mark.parametrize("pin", op.FAST_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_align_invariants_on_workloads(orc):
    op.pin_align_invariants_workloads(orc)


def test_align_invariants_stress(orc):
    op.pin_align_invariants_workloads(orc, names=("align_stress", "align_stress_neg"))


def test_capacity_bound_is_tight(orc):
    # one token per expert per slot, each alone in its block: the bound is met
    import numpy as np
    E, B = 8, 16
    out = orc.align(np.arange(E, dtype=np.int32).reshape(1, E), np.zeros(1, np.int32), E, 1, B)
    assert out["num_tokens_post_padded"][0] == E * B == out["cap"]
