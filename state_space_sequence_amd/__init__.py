"""libssd: Mamba-2 SSD chunked forward and decode state update for MI355X.

The compute lives in ``libssd.so`` (hand-written HIP for gfx950 behind a
C ABI, declared in ``include/ssd.h``).  ``state_space_sequence_amd.libssd``
is the thin ctypes binding; ``state_space_sequence_amd.inputs`` draws the
seeded synthetic workloads.  Importing the package loads nothing native.
"""

__all__ = ["libssd", "inputs"]
