"""Grammar-compressed right product y = M x on AMD MI355X (gfx950).

The native library (``libgcs.so``) holds the host builder and the HIP sweep;
``grammar_compressed_sparse_amd.gcs`` is its Python binding.  The seeded input
generators live in ``grammar_compressed_sparse_amd.synth``.  Submodules are
imported on demand so that the generators work without the native library.
"""
__all__ = ["gcs", "synth"]
