"""MI355X-native Mamba-2 SSD chunked scan.

``libssd.so`` (built from ``csrc/``) holds every step of the path as HIP
kernels for gfx950 behind a C ABI declared in ``include/ssd.h``; ``ssd`` is a
thin ctypes binding over it (argument marshalling only; the library is loaded
on first use).  ``inputs`` draws seeded synthetic problems.
"""
