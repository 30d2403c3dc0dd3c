"""Seeded synthetic inputs (model shapes, weights, KV cache, batch state).

Shared by the oracle side (tests) and the HIP side (binding, tests, bench);
holds no arithmetic of the decode step itself.
"""
from . import configs, gen  # noqa: F401
