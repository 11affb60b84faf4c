"""Seeded synthetic inputs for paged attention.

This package only draws random numbers and lays them out as a paged KV
cache (raw storage bits, block tables, lengths).  It holds none of the
attention arithmetic, so both the fp64 oracle and the HIP path can consume
the same inputs without sharing any of the method's code.
"""
from .gen import (  # noqa: F401
    Spec,
    PagedInputs,
    NAMED_SPECS,
    generate,
    named,
    NAN_BITS,
)
