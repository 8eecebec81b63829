"""libjetlong: Dynamic Bifocal RoPE attention (Jet-Long) for MI355X / gfx950.

The compute path is the C-ABI shared library ``libjetlong.so`` built from
``csrc/`` (hand-written HIP kernels); ``jetlong`` is its thin ctypes binding.
Importing this package does not load the library; the first call into
``jetlong`` does, and fails loudly when it is missing.
"""
__all__ = ["jetlong", "inputs"]
