"""MI355X-native CRISP sparse-prefill hot path.

The compute path is the HIP library ``_lib/libcrisp.so`` (C ABI declared in
``include/crisp.h``); :mod:`.crisp` is its thin ctypes binding and
:mod:`.synth` the seeded synthetic input generator.  Submodules are imported
on demand so that loading the generator does not load the GPU library.
"""
__all__ = ["crisp", "synth"]
