"""Seeded synthetic inputs and workload shapes for the MoGE layer."""
