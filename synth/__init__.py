"""Seeded synthetic workloads (shapes + input generator) shared by tests and bench."""
