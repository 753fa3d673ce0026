"""Seeded synthetic workloads shared by the tests and the benchmark (no operator arithmetic)."""
from .synth import WORKLOADS, Workload, make_inputs, spike_rows

__all__ = ["WORKLOADS", "Workload", "make_inputs", "spike_rows"]
