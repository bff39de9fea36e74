"""CPU oracle for block-causal attention.

TEST INFRASTRUCTURE, not product code.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it.  It shares no code with the HIP library in
``block_causal_attention_amd`` and never imports it; the two meet only through the seeded inputs
of ``bca_workloads``.

Parity status of every function is listed in ``bca_oracle``'s module docstring.
"""
from . import bca_oracle  # noqa: F401
