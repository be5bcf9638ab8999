"""MI355X-native predictor-gated, neuron-aware sparse FFN (PowerInfer-style decode).

The compute lives in libpi.so (hand-written HIP for gfx950, C ABI in
include/pi.h).  ``_lib`` is its ctypes binding and ``layer.DeviceLayer`` holds a
layer's device buffers.  Importing this package loads nothing; ``_lib.lib()``
loads the library and raises if it has not been built.
"""
__version__ = "0.1.0"
