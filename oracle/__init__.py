"""CPU oracle for the Muon step and the AdamW half of the hybrid optimizer
(test infrastructure only; see muon_oracle and adamw_oracle)."""
from .muon_oracle import *  # noqa: F401,F403
from .muon_oracle import (EPS, StepResult, frobenius_norm, momentum, muon_step,  # noqa: F401
                          newton_schulz, nominal_ns_flops, normalise, orient,
                          orthogonalise, orthogonalise_bf16_storage, polar_factor,
                          rel_frobenius, scale_factor, split_bf16x2, to_bf16,
                          write_back)
from .adamw_oracle import adamw, adamw_constants  # noqa: F401
