"""MI355X-native SeKV mixed-resolution decode.

The compute path lives in ``libsekv.so`` (HIP kernels for gfx950 behind a C
ABI declared in ``include/sekv.h``); :mod:`.binding` marshals torch tensors to
it.  :mod:`.synth` draws seeded synthetic inputs.
"""
__all__ = ["binding", "synth"]
