"""Plain fp64 CPU oracle for Multi-Head Latent Attention (MLA) over a latent KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no kernels, headers, helpers or constant tables) and imports
nothing from it.  Every function computes the method's plain definition in
float64 NumPy, in the NON-absorbed form (K and V are expanded from the latent
rows through kv_b_proj), with one separate absorbed-form function kept only to
check the absorption identity and to provide staged intermediates.

Sources (cited by page title and section in each docstring):
  * "Multi-Head Latent Attention" post in the liorsinai.github.io feed
    (sections 2 KV Caching, 3.1 C cache, 3.3 Absorption, 3.6 Decoupled RoPE,
    3.7 Code) -- the layer, absorption identity, RoPE and decoupled RoPE.
  * "Deepseek V2 Lite Inference Engine in C" (MLA notes) -- kv_a_proj /
    kv_b_proj fusion and the per-head K/V interleave of kv_b_proj.
  * "Transformer and KV Cache Basics" (KV Cache section) -- prefill vs decode
    and the offset causal mask for multi-token steps.

Two storage modules sit beside the layer: ``oracle.fp8`` (an FP8 E4M3 latent
cache with one scale per row, read back as the cache would hand it out) and
``oracle.paged`` (the row lookup of a cache kept in pages named by a block
table).

YaRN (``rope_theta`` with a context-extension factor > 1, and
``yarn_attention_factor``) is named on the pages without a formula; its branch
follows YaRN's NTK-by-parts interpolation in the form DeepSeek's layers run it
(outside the pages).  It is pinned against an independent implementation of
that form (the ``transformers`` library's YaRN initialisation and DeepSeek
attention scaling, importable in the test image) and against the method's
defining properties.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests in
``tests/test_oracle_pins.py`` (brute force, identities, closed forms, special
cases, the independent YaRN implementation); no function is "parity
unpinned".
"""

from .mla import (  # noqa: F401
    MLAShape,
    rms_norm,
    rope,
    latent_rows,
    query_heads,
    expand_kv,
    split_kv_b,
    causal_attention,
    output_projection,
    mla_step,
    absorbed_step,
    decode_batch,
    prefill_batch,
)
