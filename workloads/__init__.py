"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke check."""
