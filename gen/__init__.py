"""Seeded synthetic workloads for the selective scan, shared by the oracle and the GPU path."""
from .configs import WORKLOADS, Workload, workload, seed_of  # noqa: F401
from .inputs import (S6Inputs, make_inputs, workload_inputs, bf16_bits, bits_to_f32,  # noqa: F401
                     round_bf16, STREAMS, BlockInputs, make_block_inputs)
