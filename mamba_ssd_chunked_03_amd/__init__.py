"""MI355X-native Mamba-2 SSD chunked scan.

``libssd.so`` (built from ``csrc/``) holds every step of the path as HIP
kernels for gfx950 behind a C ABI declared in ``include/ssd.h``; ``ssd`` is a
thin ctypes binding over it (argument marshalling only).  ``inputs`` draws
seeded synthetic problems.  The binding is imported lazily so that the input
generator can be used on machines without the built library.
"""


def __getattr__(name):
    if name == "ssd":
        from . import ssd as _ssd
        return _ssd
    raise AttributeError(name)
