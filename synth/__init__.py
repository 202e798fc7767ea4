"""Seeded synthetic inputs for tree-attention verification.

This package builds candidate trees, bf16 query/key/value tensors (held as
uint16 bit patterns), paged KV caches and fp32 target/draft logits. Both the
CPU oracle tests and the GPU path draw their inputs from here. It holds none of
the verification arithmetic: no mask construction, attention, softmax,
acceptance test or KV commit.
"""

from .workloads import *  # noqa: F401,F403
