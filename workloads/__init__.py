"""Seeded synthetic workloads (shapes and input tensors) for the eviction path."""
from .configs import FULL, SMALL, ScoreShape, Workload  # noqa: F401
