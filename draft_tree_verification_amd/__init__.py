"""Draft-tree verification for speculative decoding, as hand-written HIP kernels for MI355X (gfx950).

The compute path lives in ``libev.so`` (built from ``csrc/``) behind a C ABI declared in
``include/ev.h``; :mod:`draft_tree_verification_amd.ev` is its thin ctypes binding.
"""
