"""Seeded synthetic workloads (shapes, position ids, input draws) shared by the
HIP path's tests and benchmark and by the oracle.  Holds none of the method's
arithmetic."""

from .configs import ALL, LLAMA7B, LONG, PACKED, QWEN05, TINY, Workload, get  # noqa: F401
