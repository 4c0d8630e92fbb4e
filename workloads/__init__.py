"""Seeded synthetic workloads (shapes, seeds and random draws only)."""
