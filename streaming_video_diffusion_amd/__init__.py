"""libstreamattn: streaming-chunk DiT self-attention for MI355X (gfx950).

The compute lives in the HIP library ``libstreamattn.so`` behind a C ABI
(``include/streamattn.h``); ``binding`` is a thin ctypes layer over it and
``inputs`` builds seeded synthetic workloads. Importing this package does not
load the library; the first call into ``binding`` does, and raises if it is
missing.
"""

__version__ = "0.1.0"
