"""MI355X (gfx950) group-wise fake-quantised linear of EfficientQAT.

The compute path is the HIP library libqat.so behind the C ABI in
include/qat.h; `_lib` is its ctypes binding. `synth` draws the seeded
synthetic inputs. Importing this package loads nothing; the library is
loaded on first use of a binding function.
"""
__all__ = ["_lib", "synth"]
