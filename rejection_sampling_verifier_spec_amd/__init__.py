"""MI355X-native batched speculative-sampling verifier.

The compute path is the HIP library ``libspecverify.so`` (C ABI declared in
``include/specverify.h``); ``rejection_sampling_verifier_spec_amd.api`` is a
thin ctypes binding over it. ``workloads`` makes seeded synthetic inputs.
"""

__all__ = ["api", "workloads"]
