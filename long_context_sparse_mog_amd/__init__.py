"""Mixture-of-Gaussians (Iceberg) decode attention for AMD MI355X (gfx950).

The compute lives in libmog (``csrc/``, C ABI in ``include/mog.h``); this
package holds its ctypes binding (``capi``), torch-facing wrappers (``ops``),
the library build step (``build_lib``) and the seeded workload generator
(``synth``).  Importing the package loads nothing; the first library call
loads ``_lib/libmog.so`` and fails loudly if it has not been built.
"""

__all__ = ["capi", "ops", "synth", "build_lib"]
