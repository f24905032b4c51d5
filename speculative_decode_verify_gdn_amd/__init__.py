"""MI355X-native speculative verification through GatedDeltaNet layers.

The compute path is the C-ABI shared library ``libgdnverify.so`` built from
``csrc/`` (hand-written HIP for gfx950).  ``binding`` marshals torch tensors to
it; ``workload`` draws seeded synthetic inputs.  Nothing here falls back to a
CPU implementation: if the library is missing, the binding raises.
"""
__all__ = ["binding", "workload"]
