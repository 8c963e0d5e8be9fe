"""Seeded synthetic workloads for the 4-bit Shampoo preconditioner step.

This package only draws random numbers and reshapes them; it holds none of
the method's arithmetic, so the CPU oracle and the HIP path can both be fed
from it.  ``configs`` defines the five workloads, ``cost`` the algorithmic
flop / byte accounting used to report throughput against the roofline.
"""

from .configs import CONFIGS, Workload, get_workload, split_blocks  # noqa: F401
