"""CPU tests: the oracle against its pins, for all 16 operator variants, and a
check that each planted mistake is caught by at least one pin."""
import pytest

import oracle_pins as OP
from oracle import mutants

IDS = ["-".join(v) for v in OP.VARIANTS]


@pytest.mark.parametrize("variant", OP.VARIANTS, ids=IDS)
@pytest.mark.parametrize("pin", OP.PINS, ids=[p.__name__ for p in OP.PINS])
def test_pin(oracle_mod, variant, pin):
    pin(OP.cfg_of(*variant))


@pytest.mark.parametrize("K", [1, 2, 16, 64])
@pytest.mark.parametrize("variant", [v for v in OP.VARIANTS if v[3] == "full"][::2], ids=lambda v: "-".join(v))
def test_pins_other_K(oracle_mod, variant, K):
    for pin in (OP.pin_autograd_rows, OP.pin_zero_sum, OP.pin_autograd_head):
        pin(OP.cfg_of(*variant, K=K, tau=5.0))


@pytest.mark.parametrize("mutation", sorted(mutants.MUTANTS))
def test_planted_mistake_is_caught(oracle_mod, mutation):
    caught = []
    for variant in OP.VARIANTS:
        cfg = OP.cfg_of(*variant, mutation=mutation)
        for pin in OP.PINS:
            try:
                pin(cfg)
            except (AssertionError, ValueError, FloatingPointError) as e:
                caught.append((variant, pin.__name__, str(e)[:80]))
                break
        if caught:
            break
    assert caught, f"no pin catches the planted mistake {mutation!r}"
