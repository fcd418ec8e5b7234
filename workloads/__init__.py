"""Seeded synthetic inputs for paged decode attention.

This package only draws random numbers and deals physical blocks out to
block tables.  It computes nothing the attention method itself computes (no
address translation, no scores, no softmax), so both the fp64 oracle and the
HIP path can take their inputs from it without sharing any arithmetic.
"""
from .synth import (  # noqa: F401
    Workload,
    CONFIG_NAMES,
    make_config,
    make_small,
    make_workload,
    raw_numpy,
    normal_storage,
    identity_tables,
    permute_pool,
    poison_unused,
)
