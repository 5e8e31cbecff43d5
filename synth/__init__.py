"""Seeded synthetic inputs shared by the oracle tests and the GPU path (no layer arithmetic)."""
from .inputs import *  # noqa: F401,F403
from .inputs import WORKLOADS, Workload, Layer, make_layer, make_x  # noqa: F401
