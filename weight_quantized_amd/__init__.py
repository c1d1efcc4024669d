"""Weight-only quantized linear layer for AMD MI355X (gfx950).

The compute path lives in the HIP library ``libzq.so`` (sources under
``csrc/``, C-ABI declared in ``include/zq.h``); ``weight_quantized_amd.zq`` is
its thin ctypes binding. ``weight_quantized_amd.synth`` holds the seeded input
generators. Importing the package loads nothing; the binding loads the library
on first use and raises if it has not been built.
"""
