"""Seeded synthetic MoE-layer workloads (shapes, hyper-parameters, inputs)."""
