"""MI355X (gfx950) mHC pre / H-aggregate: forward collapse of the
hyper-connection residual stream and its backward, as hand-written HIP
kernels behind a C ABI (include/mhc_h_aggregate.h).

The torch-facing names live in `hyper_connection_residual_mhc_amd.ops`; they
are re-exported here on first access, which loads the shared library (and
raises ImportError if it has not been built).
"""

from __future__ import annotations

_OPS_NAMES = (
    "mhc_h_aggregate_fwd", "mhc_h_aggregate_bwd", "mhc_bf16_rne_probe",
    "mhc_h_aggregate_fwd_timed", "mhc_h_aggregate_bwd_timed", "mhc_h_aggregate_bwd_acc",
    "mhc_h_aggregate_plan_bwd_acc", "mhc_h_aggregate_fwd_n", "mhc_h_aggregate_bwd_n",
    "mhc_h_aggregate_plan_fwd_n", "mhc_h_aggregate_plan_bwd_n",
    "mhc_h_aggregate_plan_fwd", "mhc_h_aggregate_plan_bwd",
    "mhc_h_aggregate_validate_fwd", "mhc_h_aggregate_validate_bwd",
    "h_aggregate", "h_aggregate_backward", "HAggregate", "h_aggregate_autograd",
)

__all__ = list(_OPS_NAMES)


def __getattr__(name: str):
    if name in _OPS_NAMES:
        from . import ops
        return getattr(ops, name)
    raise AttributeError(name)
