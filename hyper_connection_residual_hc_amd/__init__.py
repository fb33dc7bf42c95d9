"""MI355X (gfx950) implementation of the manifold hyper-connection (mHC) pre/post path.

The compute lives in the HIP library libhc_mi355x.so (C ABI: include/hc_mi355x.h); this
package holds its build script, the ctypes binding (``ops``) and the seeded input generators
(``inputs``). Importing the package does not load the library; the first op call does, and
fails if the library is not built.
"""
from . import inputs, ops  # noqa: F401

__all__ = ["inputs", "ops"]
