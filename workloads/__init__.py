"""Seeded synthetic workloads shared by the tests, the benchmark and smoke()."""
from .synth import (Workload, gaussian, tiny_single_head, rope_gqa, llama8b_layer, gated, gated_config,  # noqa: F401
                    blocks, block_config,
                    long_batched, long_batched_blind_spot, new_token, random_orthonormal)
