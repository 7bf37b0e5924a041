"""Seeded synthetic workloads shared by the tests and the benchmark."""
