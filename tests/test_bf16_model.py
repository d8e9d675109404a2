"""CPU checks of the bf16 rounding model the GPU tests use."""
import numpy as np

from oracle import muon_oracle as O
from tests.bf16_model import bf16, newton_schulz_bf16


def test_bf16_model_matches_the_oracle_on_well_conditioned_inputs():
    """The bf16 rounding model used by the GPU tests stays within the 2e-2
    bar of the fp64 oracle on a well-conditioned matrix, and its rounding is
    round-to-nearest-even (ties to even on exact halves)."""
    assert bf16(1.0 + 2.0 ** -8) == 1.0                 # tie: to even (1.0)
    assert bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # tie: to even (upper)
    assert bf16(1.0 + 2.0 ** -8 + 2.0 ** -12) == 1.0 + 2.0 ** -7
    g = np.random.default_rng(9).standard_normal((64, 160))
    ref = O.newton_schulz(g)
    assert np.linalg.norm(newton_schulz_bf16(g, (O.QUINTIC,), 5) - ref) / np.linalg.norm(ref) <= 2e-2
