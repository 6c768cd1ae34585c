"""Test-infrastructure oracle for causal GQA / paged decode / MLA latent decode.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s CPU-baseline
leg may import this package. It shares no code with the HIP library.
"""
from . import brute, oracle  # noqa: F401
