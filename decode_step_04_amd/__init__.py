"""Batch-1 GQA transformer decode step for AMD Instinct MI355X (gfx950).

The compute path is the HIP library ``libqdec.so`` built from ``csrc/`` (C ABI declared in
``include/qdec.h``); ``qdec`` is its ctypes binding and does argument marshalling only.
``synth`` draws the seeded synthetic inputs.  Importing the package loads nothing; the binding
loads the library on first use and raises if it has not been built.
"""
__all__ = ["qdec", "synth"]
