"""libfuse for MI355X (gfx950): single-pass fused row kernels behind a C ABI.

The package holds the HIP sources and the C-ABI library (``csrc/``, built into ``libfuse.so``),
the Python binding, the seeded synthetic inputs (``synth``) and the roofline arithmetic
(``roofline``).
"""
