"""Seeded synthetic workloads (shapes and inputs) for the Stable LatentMoE layer."""
from .configs import CONFIGS, LayerConfig  # noqa: F401
