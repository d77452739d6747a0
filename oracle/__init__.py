"""CPU oracle for one token-tree verification round.

TEST INFRASTRUCTURE. This package is the plain, slow, obviously-correct
reference the GPU library is checked against. Only the test suite, the
entry point's smoke check and the benchmark's CPU-baseline leg may import it;
the library and its Python binding never do, and nothing here imports them.

Floating point is float64 throughout. Storage formats (bf16 bit patterns,
fp16 scales, int8 codes) are decoded here by the oracle's own code.

Parity status: every function is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_draft.py`` or ``tests/test_oracle_lm_head.py`` against
closed forms, brute force, hand-worked examples, library routines (torch SDPA
in float64, scipy's softmax, math.fsum, Python's list max/index) or the pages'
stated equivalences; no function is parity-unpinned.
"""

from .ttv_oracle import *  # noqa: F401,F403
