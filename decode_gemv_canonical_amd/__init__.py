"""Lossless BF16 weight compression (exponent-byte canonical Huffman) with the
decode fused into the decode-time matrix-vector and small-batch products, for
AMD Instinct MI355X (gfx950).

The work happens in libuw.so (include/uw.h); this package is its thin Python
binding.  Importing it fails if the library has not been built.
"""
from .uw import *  # noqa: F401,F403
from .uw import CompressedMatrix, PaletteMatrix, UwError, header_symbols, library  # noqa: F401
