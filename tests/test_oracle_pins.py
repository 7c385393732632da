"""The oracle against its pins (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.PINS, ids=[p.__name__ for p in pins.PINS])
def test_pin(pin):
    pin()


def test_golden_page_numbers():
    """The closed form and byte arithmetic used by the pins reproduce every
    number the "A2A backends" page prints for them (sections 1.3, 2.3, 4.1)."""
    for kind, E, G, k, rows, value, *_ in pins.read_golden("pages_copies.txt"):
        E, G, k, value = int(E), int(G), int(k), float(value)
        c = float(pins.closed_form_copies(E, G, k))
        row_bytes = 10240  # 5,120 bf16 elements (section 1.1)
        if kind == "copies":
            assert round(c, 2) == value, (E, G, k, c)
        elif kind.startswith("mib_"):
            per_token = {"mib_all": G, "mib_expert": k, "mib_gpu": c}[kind]
            mib = int(rows) * per_token * row_bytes / 2 ** 20
            digits = 0 if value >= 10 else 1
            assert round(mib, digits) == value, (kind, rows, mib)
        elif kind == "pct_more":
            assert round(100 * (G / c - 1)) == value, (G, c)
        elif kind == "pct_expert":
            assert round(100 * (k / c - 1)) == value, (k, c)
        else:
            raise AssertionError(f"unknown golden row kind {kind}")
