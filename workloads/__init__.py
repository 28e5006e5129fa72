"""Seeded synthetic inputs for batched speculative-sampling verification.

This package draws logits, temperatures, positions and draft tokens shaped like
the workloads the pages benchmark on (vocabularies of 32k to 152k entries, draft
lengths 4 to 8, batches of 1 to 512, one or several draft branches per row).
It holds none of the verification arithmetic; both the oracle and the GPU path
consume the bytes it produces.
"""

from .synth import CONFIGS, Workload, make, round_to_bf16_bits, bf16_bits_to_f32  # noqa: F401
