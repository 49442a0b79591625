"""Seeded synthetic workload shapes and input tensors (no method arithmetic)."""
from .configs import BLOCK, CONFIGS, CONFIG_ORDER, Config  # noqa: F401
