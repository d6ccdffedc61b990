"""MI355X-native tile rasterizer for 2D Gaussians (accumulated-sum and alpha-composited).

The compute path is the HIP library ``libgi.so`` (kernels for gfx950 behind the
C ABI declared in ``include/gi.h``); :mod:`rasterizer_gaussian_raster_amd.gi`
is its thin ctypes binding.  Importing this package loads nothing: the library
is opened on first use and a missing library is an error, never a fallback.
"""
__all__ = ["gi", "synth"]
