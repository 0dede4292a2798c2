"""Clustered block-sparse attention for MI355X (gfx950).

The compute path is the C-ABI library ``libsa.so`` built from ``csrc/``; the
Python binding in ``_lib`` only marshals arguments.  Importing this package
does not load the library: the first call does, and it raises if the library
is missing.
"""

__all__ = ["workloads"]
