"""The oracle against its pins (brute force, closed forms, page values, library routines, invariants)."""
import pytest

from oracle import moe_ref
from tests import oracle_pins as pins


@pytest.mark.parametrize("name,check", pins.ALL_CHECKS, ids=[n for n, _ in pins.ALL_CHECKS])
def test_oracle_pin(name, check, page_values):
    check(moe_ref, page_values)


def test_brute_select_tie_rule():
    from oracle import brute

    assert brute.select([1.0, 1.0, 1.0], 2) == [0, 1]
    assert brute.select([1.0, 2.0, 1.0], 2) == [1, 0]
    assert brute.select([0.5, 0.5, 0.7, 0.5], 3) == [2, 0, 1]


def test_page_value_arithmetic(page_values):
    """The pages' own arithmetic is consistent (guards the fixture against typos)."""
    import math

    assert round(math.log(128), 2) == page_values["max_entropy_nats_E128"]
    assert round(math.log2(60), 2) == page_values["max_entropy_bits_E60"]
    assert page_values["probe_selections"] / page_values["probe_experts"] == page_values["probe_uniform_per_expert"]
    assert page_values["router_example_batch"] * page_values["router_example_seq"] == page_values["router_example_rows"]
