"""MI355X-native Kimi Delta Attention (KDA) layer library.

The compute path is the C-ABI shared library built from ``csrc/`` (HIP for
gfx950).  ``abi`` is the thin ctypes binding over it; importing the package
itself loads nothing, so host-only tools (the seeded input generators in
``inputs``) work without the library.
"""
__all__ = ["abi", "inputs"]
