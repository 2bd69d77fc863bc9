"""MI355X-native two-sided (Kronecker-factored) GPTQ rounding: BaKron.

The compute path lives in ``libbakron.so`` (HIP kernels for gfx950 behind a
C ABI, declared in ``include/bakron.h``).  ``two_sided_gptq_amd.bakron`` is the
thin ctypes binding; importing this package does not load the library, so the
seeded input generators in ``two_sided_gptq_amd.synth`` work without a GPU.
"""
__all__ = ["bakron", "synth"]
