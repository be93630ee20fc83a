"""Paged attention for AMD MI355X (gfx950): HIP kernels behind a C ABI.

``binding`` is the Python face of ``libpa.so`` (include/pa.h);
``workloads`` draws the seeded synthetic inputs; ``build`` compiles the
library in-tree.
"""
