"""MI355X-native quantized decode / routed-expert library (HIP, gfx950).

The compute lives in ``libqmoe.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/qmoe.h``).  ``decode_moe_mul_amd.qmoe`` is the thin
Python binding: argument marshalling only; every step runs in the kernels.
Importing this package does not load the library; the first call does, and
raises if the library is missing.
"""

__all__ = ["qmoe", "synth", "configs"]
