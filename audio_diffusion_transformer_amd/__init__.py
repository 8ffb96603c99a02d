"""MI355X-native fused Q/K RMSNorm + RoPE + non-causal attention (libh3attn).

The compute path is the HIP library ``libh3attn.so`` (C ABI in
``include/h3attn.h``); ``h3attn`` is its ctypes binding and ``synth`` draws the
seeded synthetic inputs.  Importing the package does not load the library.
"""
__all__ = ["h3attn", "synth"]
