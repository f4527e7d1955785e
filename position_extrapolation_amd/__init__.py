"""DCA (Dual Chunk Attention) prefill attention for AMD Instinct MI355X.

The compute path is libdca.so (HIP kernels for gfx950 behind the C ABI in
include/dca.h); `api` is its thin ctypes binding, `workloads` the named
problem shapes, `synth` the seeded input generators.
"""

from . import api, synth, workloads  # noqa: F401
from .api import prefill  # noqa: F401
