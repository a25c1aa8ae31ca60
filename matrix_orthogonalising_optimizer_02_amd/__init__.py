"""Muon and Periodic Row-wise Muon optimizer steps for 2-D weights on MI355X (gfx950).

The work runs in libmuon_rocm.so (HIP kernels behind a C ABI, include/muon_rocm.h);
`binding` marshals torch tensors to it. `workloads` holds the seeded synthetic
inputs used by the tests and the benchmark.
"""
from .binding import (  # noqa: F401
    SCALE_HIDDEN,
    SCALE_MAX_DIM,
    SCALE_RMS,
    AdamWGroup,
    AdamWHParams,
    MuonError,
    MuonHParams,
    MuonOptimizer,
    adamw_default_hparams,
    adamw_step,
    ceiling_copy,
    ceiling_mfma,
    default_hparams,
    load_library,
    make_workspace,
    muon_step,
    ns5_batched,
    ns5_plan,
    rownorm_shard_apply,
    rownorm_shard_colsq,
    rownorm_shard_workspace_bytes,
    rownorm_update,
    rownorm_update_noalloc,
    svd_entropy,
    svd_entropy_workspace_bytes,
    timing_enable,
    timing_read,
    workspace_bytes,
)
