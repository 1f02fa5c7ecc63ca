"""svgear: SVG-EAR error-aware routed sparse attention for MI355X (gfx950).

The compute lives in ``libsvgear.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/svgear.h``).  ``svgear`` is the thin ctypes binding over
it; ``inputs`` draws the seeded synthetic workloads.  Submodules are imported
lazily so that ``inputs`` can be used without loading the HIP library.
"""
__all__ = ["svgear", "inputs"]
