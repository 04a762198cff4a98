"""Sparse MLA attention over top-k selected KV for AMD MI355X (gfx950).

The compute lives in a HIP/C++ shared library behind a C ABI
(include/sparse_mla.h); `binding` is its thin ctypes wrapper and `inputs`
holds the seeded synthetic input generators.  Importing the package loads
nothing: the library is opened on first use of `binding`.
"""
