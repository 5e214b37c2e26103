"""Contextual-sparsity decode step for AMD MI355X (gfx950).

``configs`` and ``synth`` are plain Python.  The compute path lives in the HIP
library ``libdv.so``; ``contextual_sparsity_decoding_amd.dv`` binds it and
raises on import when the library has not been built.
"""
__all__ = ["configs", "synth"]
