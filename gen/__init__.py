"""Seeded synthetic input generators (no method arithmetic)."""
from .workloads import SPECS, Spec, Workload, make_config, make_custom, sps_table, to_bf16_bits, bf16_bits_to_f32  # noqa: F401
