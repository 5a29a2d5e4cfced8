"""MI355X-native forward pass of a Mixture-of-Experts FFN layer.

libmoe.so (HIP kernels for gfx950 behind the C ABI in include/moe.h) does all
the work; `_lib` is its ctypes binding (same function names as the C entry
points), `layer.MoeLayer` allocates device buffers and calls the stages, and
`inputs` draws seeded synthetic layers. Importing the package loads nothing;
the library is loaded on first use and raises if it was not built.
"""
__all__ = ["inputs", "layer", "_lib", "build"]
