"""CPU oracle for WIDE's masked dynamic-width execution (test infrastructure).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``sparse_wide_mask_amd``) never imports, links or calls it, and this package
imports nothing from the GPU library.  The two share only ``synth`` (seeded
inputs, no method arithmetic).

The oracle is plain and slow on purpose: NumPy, float64 by default, no
blocking, no sparsity exploitation.  Every layer is computed densely, then the
groups a token's mask drops are zeroed.  See ``oracle/wide_oracle.py`` for what
each function follows on the pages, and for the readings taken where the pages
are silent.
"""
from .wide_oracle import (attn_masked, ffn_masked, layer_masked, mask_reorder,
                          paged_to_contiguous, rmsnorm, rope, router_topk)

__all__ = ["mask_reorder", "ffn_masked", "attn_masked", "layer_masked", "rmsnorm", "rope",
           "router_topk", "paged_to_contiguous"]
