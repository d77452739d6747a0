"""Seeded synthetic inputs for token-tree verification.

This package is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only *constructs* inputs (topologies, draft tokens, logits, KV
caches and their storage formats); it holds none of the verification
arithmetic (no masking, attention, argmax, walk or gather).
"""

from .gen import *  # noqa: F401,F403
from .configs import *  # noqa: F401,F403
