"""Seeded synthetic input generators (no part of the method lives here)."""

from .workloads import (  # noqa: F401
    FULL,
    GAP_REQUIRED,
    Workload,
    attn_pv,
    decode_attn_qk,
    decode_qkv,
    gqa_qk,
    int8_weights,
    mlp_down,
    mlp_up,
    stored64,
    tiny_projection,
    to_bf16,
    to_f32,
    w8_projection,
)
