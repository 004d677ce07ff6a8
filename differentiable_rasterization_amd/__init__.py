"""MI355X-native differentiable tile rasterizer for 3D Gaussian Splatting.

The compute lives in ``libgsraster.so`` (hand-written HIP for gfx950, C ABI
declared in ``include/gsraster.h``); :mod:`.raster` is the thin ctypes binding
with the same entry-point names, and :mod:`.scenes` draws seeded synthetic
inputs.  Importing the package loads nothing; the binding loads the library
on first use and raises if it is missing.
"""
__all__ = ["raster", "scenes"]
