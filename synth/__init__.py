"""Seeded synthetic workloads (shapes and random draws only)."""

from . import configs, gen  # noqa: F401
