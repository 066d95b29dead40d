"""LatentIndex sparse-attention indexer hot path for MI355X (gfx950).

The compute lives in ``liblatentindex.so`` (hand-written HIP kernels behind a
C ABI declared in ``include/latentindex.h``).  ``binding`` marshals torch
tensors into that ABI; ``synth`` draws the seeded synthetic workloads.
Importing the package does not load the library; ``binding.lib()`` does, and
fails loudly when it has not been built.
"""
__all__ = ["binding", "synth", "build"]
