"""fp64 CPU oracle of the Muon step and its AdamW branch (test infrastructure
only; see ``oracle.muon_oracle`` and ``oracle.adamw_oracle``).  Imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark, never by the library."""
from .muon_oracle import *  # noqa: F401,F403
from .muon_oracle import (QUINTIC, CUBIC, HYBRID_TAIL, DEFAULT_EPS,  # noqa: F401
                          momentum_lerp, frobenius_norm, normalise,
                          needs_transpose, ns_iteration, newton_schulz,
                          rms_scale, apply_update, muon_step_matrix, muon_step,
                          zero_center, nesterov_input)
from .adamw_oracle import (ADAMW_LR, ADAMW_BETAS, ADAMW_EPS, ADAMW_WD,  # noqa: F401
                           adamw_step_tensor, adamw_step)
