"""float64 CPU oracle for the Muon / Periodic Row-wise Muon step.

Test infrastructure only: the product path never imports this package.
"""
from .muon_oracle import (  # noqa: F401
    OracleHParams,
    is_refresh_step,
    is_tall,
    momentum,
    muon_step,
    newton_schulz,
    ns5_update_direction,
    row_normalise,
    rownorm_step,
    rownorm_update_direction,
    vanilla_step,
)
