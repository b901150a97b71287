"""fp64 CPU oracle for exact softmax attention -- test infrastructure only.

Imported only by tests/, the smoke check in __graft_entry__.py and the CPU
baseline leg of bench.py.  The HIP library never reaches it.
"""
from .attention import backward, forward, online_forward, row_sample_forward  # noqa: F401
