"""MI355X-native draft-tree verification: ancestor-masked tree attention,
the canonical exit law and Tree Exit Verification (TEV), as hand-written HIP
kernels for gfx950 behind a C ABI (``include/tev.h``).

The binding lives in :mod:`draft_tree_verification_amd.tev`; importing this
package does not load the native library.
"""
__all__ = ["tev"]
