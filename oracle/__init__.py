"""fp64 CPU oracle for the gate-first sparse FFN: TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. It shares no code with the HIP library
(``activation_sparse_gated_amd``) and never imports it.
"""
from .reference import (  # noqa: F401
    ACT_RELU, ACT_RSPLUS, activation, build, ffn_lopa, ffn_standard, num_threads,
    set_threads)
from . import counts  # noqa: F401
