"""MI355X-native OmniMoE routed atomic-expert layer (forward pass).

The compute lives in libomni.so (hand-written HIP for gfx950, C ABI declared
in include/omni.h); `binding` is its thin ctypes wrapper.  Importing this
package loads nothing; `binding.lib()` loads the library on first use.
"""
__all__ = ["binding", "build"]
