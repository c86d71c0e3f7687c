"""Seeded synthetic workloads shared by the tests, the bench and the oracle
checks.  Produces token batches and attention tensors only; it holds none of
the packing or attention arithmetic."""

from .generators import (  # noqa: F401
    Workload,
    CONFIG_NAMES,
    make_workload,
    sweep_workload,
    worked_example,
    attention_inputs,
    pad_rows,
    small_workload,
    SMALL_KINDS,
    edge_layouts,
    score_ramp_inputs,
    batch_attention_inputs,
    device_attention_inputs,
)
