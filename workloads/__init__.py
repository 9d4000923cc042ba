"""Seeded synthetic workloads shaped like the pages' MoE models (inputs only)."""
from .synth import SPECS, Spec, Workload, make, custom, random_ids, content_hash, names  # noqa: F401
