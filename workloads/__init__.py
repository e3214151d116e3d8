"""Seeded synthetic workloads (shapes, seeds, value draws) shared by the oracle
and the GPU path.  No part of the method is computed here."""
from . import configs, generate  # noqa: F401
from .configs import ALL, BY_NAME, Workload  # noqa: F401
