"""MI355X-native Multi-Head Latent Attention over a latent KV cache.

The compute path lives in a C-ABI shared library of hand-written HIP kernels
for gfx950 (``csrc/``); ``mla_latent_kv_decode_amd.lib`` is a thin ctypes
binding over it.  Importing this package does not load the library; the
binding loads it on first use and raises if it is missing.
"""

__all__ = ["lib", "synth"]
