"""MI355X-native lookahead sparse-KV decode step (OasisKV hot path).

liboasiskv.so (HIP kernels for gfx950 behind a C ABI, include/oasiskv.h) does
all the work; `_lib` is its ctypes binding and `runtime` the per-layer step
chain over it.
"""
from . import _lib  # noqa: F401
