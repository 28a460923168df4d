"""CPU oracle for context-parallel blockwise causal attention (forward and
backward).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The GPU product (``long_context_causal_amd``) shares no code with it and
never imports it.

Everything here is fp64 and written from the pages' description of the
method, in the pages' order:

* ``attention``  - the plain definition of causal softmax attention with
  its natural-log LSE, and its derivative (dQ, dK, dV for a given dO)
  (C core in ``attention.c``, OpenMP);
* ``cp``         - the context-parallel emulation: zigzag ("one big, one
  small") partition with global positions, the three step modes and the
  ring source of each step, blockwise step attention, the per-step L
  correction and the final O merge, RoPE at global positions, and the
  backward of each ring step with the rank's final L (the K/V gradient
  contributions a reduce-scatter would sum on their owner);
* ``varlen``     - packed variable-length samples: each sample an
  independent causal sequence, split by the zigzag rule on its own, RoPE at
  in-sample positions (reset at every sample start), and the rank's CP
  share of the packed batch.

Pins (tests marked ``not gpu``) tie both to things other than themselves:
closed forms, a library attention routine, exact integer cover of the
causal triangle, the LSE split identity, RoPE's rotation identities and,
for the backward, central finite differences of the forward oracle.
Nothing is "parity unpinned" except the RoPE convention (base 10000,
rotate-half pairing), which the pages do not fix.
"""
from .attention import (attention_rows, attention_rows_bwd, causal_attention,  # noqa: F401
                        causal_attention_bwd, max_threads)
from . import cp  # noqa: F401
from . import varlen  # noqa: F401
