"""Binade on MI355X: BF16 weights with rank-coded exponents, decoded inside
HIP kernels for gfx950.

The compute path is the C-ABI library ``libbinade.so`` (built from
``csrc/``); ``binade`` is its Python binding. ``synth`` draws the seeded
synthetic inputs used by the tests and the benchmark.
"""
__all__ = ["binade", "synth"]


def __getattr__(name):
    if name == "binade":
        from . import binade as _b
        return _b
    raise AttributeError(name)
