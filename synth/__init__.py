"""Seeded synthetic inputs for the Pyramid Sparse Attention forward path (shared by tests,
the oracle's calibration script and the benchmark; holds none of the method's arithmetic)."""
from .workloads import WORKLOADS, Workload, get  # noqa: F401
from .video_field import generate, generate_qkv, head_field, random_qkv  # noqa: F401
