"""Seeded synthetic inputs and workload shapes (no method arithmetic)."""
