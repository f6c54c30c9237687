"""Seeded synthetic inputs (shared by the oracle harness and the GPU harness)."""
