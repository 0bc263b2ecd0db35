"""Seeded synthetic workloads (inputs only; no arithmetic of the method)."""
