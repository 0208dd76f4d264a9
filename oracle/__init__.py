"""fp64 CPU oracle for attention over a resident, shared KV-cache prefix.

TEST INFRASTRUCTURE ONLY. It is the plain, slow definition the HIP path is checked
against; only ``tests/``, ``__graft_entry__.smoke()`` and the bench's CPU-baseline
leg may import it. It shares no code with ``kv_cache_prefix_amd`` and imports
nothing from it; both sides take their inputs from ``synth`` only.

Parity pins (what each function is checked against, besides itself) live in
``tests/test_oracle_*.py``. Where the pages leave a point open the oracle follows one
reading and is pinned to that reading, not to the pages (parity with the pages is
unpinned there): the LSE base (natural log: ln N at q = 0 and a two-key hand case),
the causal alignment for M < S_suf (bottom-right: torch's masked SDPA with a shifted
lower triangle, at M < S_suf too). ``top_k`` and ``fa_window`` are not implemented.
"""
from .cold_tier import ColdTier
from . import vstore
from .attention import (attend, combine, f64, merge, prefix_query, prefix_query_fused,
                        resolve_head_map, softmax_scale, suffix_visible)
from .mlx4g32 import dequantize, quantize, record_bytes, unpack_codes
from .sparse import (block_means, block_scores, n_blocks, prefix_query_blocks,
                     prefix_query_sparse, prefix_query_sparse_auto, select_blocks)

__all__ = [
    "ColdTier", "vstore",
    "attend", "combine", "f64", "merge", "prefix_query", "prefix_query_fused",
    "resolve_head_map", "softmax_scale", "suffix_visible", "dequantize", "quantize",
    "record_bytes", "unpack_codes", "block_means", "block_scores", "n_blocks", "prefix_query_blocks",
    "prefix_query_sparse", "prefix_query_sparse_auto", "select_blocks",
]
