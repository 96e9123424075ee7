"""MI355X-native Kimi Delta Attention (KDA) chunked forward.

The compute path is the C-ABI library ``libkda.so`` (hand-written HIP kernels
for gfx950) declared in ``include/kda.h``; ``chunked_gated_delta_07_amd.kda``
is a thin ctypes binding with the same entry-point names.  Importing this
package loads nothing; the binding loads the library on first use and raises
if it is missing.
"""
__all__ = ["kda", "synth"]
