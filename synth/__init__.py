"""Seeded synthetic inputs for the memory-efficient linear GRPO loss.

This package only draws random numbers and lays them out; it holds none of the
loss's arithmetic.  Both the CPU oracle (under ``oracle/``) and the GPU binding
take their inputs from here, so the two sides see bit-identical operands.
"""

from .workloads import WORKLOADS, Workload, workload_by_name  # noqa: F401
from .generate import Inputs, generate, materialized_logits_bytes  # noqa: F401
