"""MI355X-native int8-state Gated DeltaNet / Kimi Delta Attention decode path.

The hot path (decode step, window flush, state codec) is hand-written HIP for
gfx950 behind a C ABI (``liblq.so``, declared in ``include/lq.h``); this
package holds the kernels' sources, the build step, a thin ctypes binding and
the seeded synthetic-input generator.
"""
