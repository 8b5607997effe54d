"""Test infrastructure: the slow, plain fp64 CPU oracle for Kimi Delta Attention (KDA).

Nothing in the product path may import, call or execute anything in this package.
Only the tests, the smoke check in ``__graft_entry__`` and the CPU-baseline leg of
``bench.py`` use it.  It shares no code with the HIP path (no kernels, headers,
helpers, constants or pre/post-processing), and it imports nothing from it.

Sources (pages about the method):

* "Kimi Delta Attention: The Linear Attention Behind Kimi K2 and Qwen3"
  (elsolitario.org), section "How Kimi Delta Attention works step by step": the
  per-token cycle decay -> predict -> error scaled by beta -> correct -> read (its
  prose and flowchart; the order of the steps).
* "Kimi Delta Attention Technical Deep Dive" (mohalkarushikesh.github.io),
  section "From attention to recurrent state" (delta rule and its
  forget-plus-write factorisation) and "Systems and implementation tradeoffs"
  (chunkwise scans whose boundary state seeds the next chunk; one-token decode).

Modules:

* :mod:`oracle.kda_ref`        -- the token-by-token recurrence (the definition).
* :mod:`oracle.kda_chunk_ref`  -- the chunkwise algebra in fp64 (what a chunked
  kernel computes), checked against the recurrence.
* :mod:`oracle.kda_prologue`   -- raw projections to the recurrence's inputs (key
  L2 normalisation, sigmoid write strength, sigmoid retention gate).
* :mod:`oracle.kda_bwd_ref`    -- the gradients of the recurrence (reverse-mode chain
  rule through the token cycle), for training; ``kda_chunk_ref.chunked_backward``
  is the same through the chunk algebra.
* :mod:`oracle.pool`           -- fans independent (sequence, head) units out over
  host cores, for the CPU baseline.

Parity pins (``tests/test_oracle_pins.py``, ``tests/test_oracle_decay_variants.py``,
``tests/test_oracle_prologue.py``, ``tests/test_oracle_backward.py``): every function
here is pinned
by closed forms, special cases that reduce to a library routine, exact rational
brute force, a hand-derived worked example and invariants; none is "parity unpinned".
"""

from .kda_ref import (  # noqa: F401
    default_scale,
    recurrence,
    forward,
    decode_step,
)
from .kda_chunk_ref import chunked, chunked_backward  # noqa: F401
from .kda_prologue import (  # noqa: F401
    BETA_LOGIT,
    GATE_LOGIT,
    NORM_K,
    prologue,
)
from .kda_bwd_ref import backward, recurrence_backward, segmented_backward  # noqa: F401
