"""Partitioned on-chip (LDS) integer histogram for AMD Instinct MI355X (gfx950).

``hist.Plan`` / ``hist.run`` call the C-ABI library libpca_hist.so, whose HIP
kernels do all of the work; ``inputs`` draws the seeded synthetic workloads.
"""
from . import hist  # noqa: F401
from .hist import Plan, run  # noqa: F401
