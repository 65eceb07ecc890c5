"""Seeded synthetic workloads (sizes, seeds and input generators)."""
from . import configs, synth  # noqa: F401
from .configs import ALL, HEADLINE, TINY, Dims, TreeSpec, Workload, get  # noqa: F401
