"""Seeded synthetic inputs (no arithmetic of the method itself)."""
from .gen import *  # noqa: F401,F403
from .gen import WORKLOADS, LayerShape, Workload  # noqa: F401
