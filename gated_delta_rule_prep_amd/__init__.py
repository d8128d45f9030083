"""MI355X-native chunked Kimi Delta Attention (KDA) forward pass.

The compute path is a C-ABI shared library (``libkda.so``, built from
``csrc/`` with hipcc for gfx950) declared in ``include/kda.h``; ``kda.py``
is the thin ctypes binding that marshals torch tensors into it.  Importing
this package loads nothing: ``from gated_delta_rule_prep_amd import kda``
loads the library and fails loudly if it has not been built.
"""
__all__ = ["kda", "inputs", "chunk_kda"]
