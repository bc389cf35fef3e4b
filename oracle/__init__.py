"""CPU oracle for RMM -- test infrastructure, never part of the product path."""

from .rmm_oracle import (  # noqa: F401
    col_energy,
    dense,
    error_bound,
    k_rule,
    kv_head,
    matmul,
    pv,
    qk,
    select,
)
