"""MI355X (gfx950) mHC pre / H-aggregate: forward collapse of the
hyper-connection residual stream and its backward, as hand-written HIP
kernels behind a C ABI (include/mhc_h_aggregate.h).

The torch-facing names live in `hyper_connection_residual_mhc_amd.ops` (and
`.coeff` for the coefficient backward epilogue); they are re-exported here
on first access. Calling them loads the shared libraries (ImportError if
they have not been built).
"""

from __future__ import annotations

_OPS_NAMES = (
    "mhc_h_aggregate_fwd", "mhc_h_aggregate_bwd",
    "mhc_h_aggregate_fwd_timed", "mhc_h_aggregate_bwd_timed", "mhc_h_aggregate_bwd_acc",
    "mhc_h_aggregate_plan_bwd_acc", "mhc_h_aggregate_fwd_n", "mhc_h_aggregate_bwd_n",
    "mhc_h_aggregate_plan_fwd_n", "mhc_h_aggregate_plan_bwd_n",
    "mhc_h_aggregate_plan_fwd", "mhc_h_aggregate_plan_bwd",
    "mhc_h_aggregate_validate_fwd", "mhc_h_aggregate_validate_bwd",
    "h_aggregate", "h_aggregate_backward", "HAggregate", "h_aggregate_autograd",
    "mhc_pre_h_aggregate",
)
_COEFF_NAMES = (
    "mhc_coeff_bwd", "mhc_coeff_bwd_workspace_bytes", "mhc_coeff_bwd_plan",
    "mhc_coeff_bwd_validate", "coeff_columns",
)

__all__ = list(_OPS_NAMES) + list(_COEFF_NAMES)


def __getattr__(name: str):
    if name in _OPS_NAMES:
        from . import ops
        return getattr(ops, name)
    if name in _COEFF_NAMES:
        from . import coeff
        return getattr(coeff, name)
    raise AttributeError(name)
