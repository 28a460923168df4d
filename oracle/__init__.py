"""CPU oracle for context-parallel blockwise causal attention (forward).

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package.
The GPU product (``long_context_causal_amd``) shares no code with it and
never imports it.

Everything here is fp64 and written from the pages' description of the
method, in the pages' order:

* ``attention``  - the plain definition of causal softmax attention with
  its natural-log LSE (C core in ``attention.c``, OpenMP over rows);
* ``cp``         - the context-parallel emulation: zigzag ("one big, one
  small") partition with global positions, the three step modes and the
  ring source of each step, blockwise step attention, the per-step L
  correction and the final O merge, and RoPE at global positions.

Pins (tests marked ``not gpu``) tie both to things other than themselves:
closed forms, a library attention routine, exact integer cover of the
causal triangle, the LSE split identity and RoPE's rotation identities.
Nothing is "parity unpinned" except the RoPE convention (base 10000,
rotate-half pairing), which the pages do not fix.
"""
from .attention import attention_rows, causal_attention, max_threads  # noqa: F401
from . import cp  # noqa: F401
