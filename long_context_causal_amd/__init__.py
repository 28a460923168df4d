"""MI355X-native context-parallel blockwise causal attention (forward).

The compute lives in ``libcpattn.so`` (hand-written HIP for gfx950 behind a
C ABI, declared in ``include/cpattn.h``).  ``long_context_causal_amd.cpattn``
is a thin ctypes binding with the same entry-point names; it loads the
library on first use and raises if it is missing - there is no CPU fallback.
"""
from .inputs import WORKLOADS, Workload, make_inputs  # noqa: F401
