"""MI355X-native decode-time KV-cache compression event (mass-segmented, AMS).

The five steps of one event -- window score, mass, segmentation and quota,
select, gather -- run as hand-written HIP kernels for gfx950 behind the C ABI
declared in ``include/kvc.h`` (``libkvc.so``).  ``eviction_window_qk_amd.kvc``
is the thin ctypes binding over that library; it loads the library on first
use and raises if it is missing.  ``eviction_window_qk_amd.synth`` holds the
seeded synthetic input generators.
"""
__all__ = ["kvc", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
