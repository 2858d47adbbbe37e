"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the bench.

This package draws random numbers and lays them out; it performs none of the
attention arithmetic.  See ``synth.gen`` for the recipes.
"""
