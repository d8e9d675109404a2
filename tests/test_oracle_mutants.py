"""The pins of ``test_oracle_pins.py`` are strong enough: each deliberately
broken copy of the Newton-Schulz routine below (a dropped term, a wrong sign,
a transposed operand, a wrong norm, a missing transpose back, ...) must fail
at least one of them.  The mistakes are planted here, in CPU copies of the
oracle's routine; nothing runs on a GPU."""
import numpy as np
import pytest

from tests.test_oracle_pins import ALL_CHECKS


def _make(variant):
    def ns(g, coeffs, steps, eps):
        g = np.asarray(g, dtype=np.float64)
        coeffs = list(coeffs)
        if len(coeffs) == 1:
            coeffs = coeffs * steps
        if variant == "norm_squared":
            x = g / (np.sum(g * g) + eps)
        elif variant == "max_norm":
            x = g / (np.abs(g).max() + eps)
        else:
            x = g / (np.linalg.norm(g) + eps)
        tall = g.shape[0] > g.shape[1]
        if tall and variant != "no_transpose":
            x = x.T
        for a, b, c in coeffs:
            if variant == "gram_wrong_side" and x.shape[0] == x.shape[1]:
                A = x.T @ x
            else:
                A = x @ x.T if not (variant == "no_transpose" and tall) else x.T @ x
            if variant == "drop_c":
                B = b * A
            elif variant == "flip_b":
                B = -b * A + c * (A @ A)
            elif variant == "c_times_A":
                B = b * A + c * A
            else:
                B = b * A + c * (A @ A)
            if variant == "no_transpose" and tall:
                x = a * x + x @ B
            elif variant == "update_wrong_side" and x.shape[0] == x.shape[1]:
                x = a * x + x @ B
            elif variant == "drop_a":
                x = B @ x
            elif variant == "a_on_B":
                x = x + a * (B @ x)
            else:
                x = a * x + B @ x
        if tall and variant not in ("no_transpose", "no_transpose_back"):
            x = x.T
        return x
    return ns


MUTANTS = ["norm_squared", "max_norm", "drop_c", "flip_b", "c_times_A", "drop_a", "a_on_B",
           "no_transpose_back", "gram_wrong_side", "update_wrong_side"]


@pytest.mark.parametrize("variant", MUTANTS)
def test_mutant_is_caught(variant):
    ns = _make(variant)
    caught = []
    for check in ALL_CHECKS:
        try:
            check(ns)
        except (AssertionError, ValueError):
            caught.append(check.__name__)
    assert caught, f"mutant {variant} passed every pin"


def test_unmutated_copy_passes():
    ns = _make("none")
    for check in ALL_CHECKS:
        check(ns)
