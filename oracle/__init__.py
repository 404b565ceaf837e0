"""fp64 CPU oracle for the per-sample gradient-norm path.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the product package.
"""
from .reference import (  # noqa: F401
    RANK_TAU,
    basis_residuals,
    clip_factors,
    exact_explicit,
    exact_gram,
    exact_trace,
    hutch,
    hutch_sign,
    hutch_trace_form,
    hutchpp,
    hutchpp_head_tail,
    hutchpp_sketch,
    hutchpp_sample,
    hutchpp_split,
    layer_sum,
    norms_routed,
    orthonormal_basis,
    routes_exact,
    to_f64,
    unpack_signs,
)
