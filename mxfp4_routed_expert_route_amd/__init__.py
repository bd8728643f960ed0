"""MI355X (gfx950) routed-expert MoE layer with MXFP4 expert weights.

The compute path is the HIP library ``libmoe_mxfp4.so`` built from ``csrc/``;
``binding`` is a thin ctypes layer over its C ABI.  Importing this package does
not load the library: ``binding.load()`` does, and fails loudly if it is absent.
"""
__all__ = ["inputs", "binding"]
