"""Slow, plain fp64 CPU oracle for the segment-attention hot path.

THIS PACKAGE IS TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it. The product path
(``segment_autoregressive_dit_amd``) never imports, calls or links anything here,
and nothing here imports the product path: the two share no code. The only shared
module is the seeded input generator ``segment_autoregressive_dit_amd/synth.py``,
which holds no arithmetic of the method.

What is computed, and where the pages state it:

* 3D rotary position embedding over (frame, row, col) of Q and K -- the model
  card's architecture list ("3D RoPE") as quoted in "Hy-Nomas auf einer RTX 4090"
  (inferencekey.com), section "Modell und Dateien"; the orcarouter.ai article
  "Hy-Nomas: Was Tencent mit seinem frei formbaren interaktiven Weltmodell
  tatsaechlich macht", section "Die Schleife"; and the blog.authon.dev article on
  running Hy-Nomas on an RTX 4090, section "What Hy-Nomas is".   -> ``rope``
* INT8 KV cache ("stored INT8, computed BF16") -- inferencekey.com,
  section "Das Single-GPU-Preset"; blog.authon.dev config excerpt
  ``kv_cache_quantization: int8``.                               -> ``quant``
* the cache of earlier latents' keys and values, carried across segments, of
  which only the last 18 latent frames stay on the GPU -- orcarouter.ai,
  section "Die Schleife"; blog.authon.dev, "What Hy-Nomas is" and the
  ``sliding_window: past_frames: 18`` excerpt under "Hardware tiers".  -> ``ring``
* segment-wise causal joint attention -- madebyagents.com model page "Hy-Nomas",
  component list ("Segment-Autoregressive DiT").                -> ``attention``

Readings of what the pages leave open are listed in each module's docstring.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, invariants, library routines, exact rational arithmetic or
brute force; none is "parity unpinned".
"""

from . import formats, rope, quant, ring, attention  # noqa: F401

__all__ = ["formats", "rope", "quant", "ring", "attention"]
