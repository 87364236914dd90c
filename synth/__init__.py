"""Seeded synthetic inputs for the tree-verify tests and benchmark.

This package only draws inputs (trees, paged KV, logits, GDN tensors); it
holds none of the verify arithmetic, so both the library's tests and the
oracle can take their inputs from it.
"""
from . import configs, trees, workloads  # noqa: F401
