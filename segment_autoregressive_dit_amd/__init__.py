"""MI355X-native segment-attention hot path (3D RoPE, ring KV-cache append,
block-causal segment attention) behind the C-ABI library ``libnomas.so``.

Importing the package does not load the HIP library; the first call into
``segment_autoregressive_dit_amd.nomas`` does, and fails loudly if it is missing.
"""

__version__ = "0.1.0"
