"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle checks.

This package draws random tensors and lays them out; it holds none of the
attention method's arithmetic (no pooling, scoring, selection, softmax or
combine).  Both the CPU oracle and the HIP path consume what it produces.
"""
from .inputs import (  # noqa: F401
    BLOCK,
    WORKLOADS,
    DenseInputs,
    VarlenInputs,
    dense_inputs,
    varlen_inputs,
    workload,
    bf16_to_f64,
    full_gate,
    output_grad,
    tied_dense_inputs,
    tied_varlen_inputs,
    TIED_Q_UNIT,
    TIED_K_UNIT,
)
