"""MXFP4 quantize-then-contract path for AMD MI355X (gfx950).

The compute lives in the HIP library ``libmx355.so`` (C ABI declared in
``include/mx.h``); ``mxfp4_precision_numerics_amd.mx`` is the thin Python
binding over it.  Importing this package loads nothing; ``synth`` holds the
seeded synthetic inputs.
"""
__all__ = ["mx", "synth"]
