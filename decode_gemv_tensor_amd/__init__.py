"""Binade on MI355X: BF16 weights with rank-coded exponents, decoded inside
HIP kernels for gfx950.

The compute path is the C-ABI library ``libbinade.so`` (built from
``csrc/`` by ``build.py``); ``binade`` is its Python binding and loads the
library on first use. ``synth`` draws the seeded synthetic inputs used by the
tests and the benchmark.
"""
__all__ = ["binade", "synth", "build"]
