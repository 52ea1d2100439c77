"""MI355X (gfx950) sparse Mixture-of-Experts MLP block.

The compute path is the HIP library built from csrc/ (C ABI in include/moe.h); ``binding`` is its
ctypes binding and ``inputs`` the seeded synthetic input recipe. Importing this package does not
load the library; the first call through ``binding`` does, and raises if it is missing.
"""
__all__ = ["binding", "inputs", "build"]
