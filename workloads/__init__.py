"""Verify-step workloads: shapes (configs) and seeded synthetic inputs (gen).

Shared by the oracle's tests and by the HIP path's tests and benchmark; holds no arithmetic of
the method itself.
"""
from .configs import Layer, Workload, WORKLOADS, ORDER, noise_sigma  # noqa: F401
