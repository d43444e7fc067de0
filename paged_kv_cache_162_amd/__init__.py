"""pagedkv for MI355X: paged KV cache and paged decode attention.

The product is the C ABI library libpagedkv.so (include/pagedkv.h) built from
csrc/ with hipcc for gfx950. `binding` exposes its functions under the same
names; `session` drives one decode step (slot mapping, cache write, decode)
over device buffers for benchmarks and tests.
"""
from .binding import *  # noqa: F401,F403
from .binding import KVError, lib, LIB_PATH, EXPORTED  # noqa: F401
