"""Seeded synthetic S5 workloads (inputs only; no forward-path arithmetic)."""
from .s5_workloads import *  # noqa: F401,F403
from .s5_workloads import bf16_to_f32  # noqa: F401
