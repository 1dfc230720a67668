"""libbsga: block-sparse global attention for VGGT-style multi-view geometry
transformers, as hand-written HIP kernels for gfx950 behind a C ABI.

Importing the package does not load the native library; ``from
block_sparse_global_bsga_amd import bsga`` does, and raises if it is missing.
"""
__all__ = ["synth"]
