"""CPU oracle for cross-model reuse of causal attention maps.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports this package: only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
may import or call it. It shares no code with the HIP library (no kernels,
headers, helpers, tables or constant generators) and imports nothing from it.

Plain, slow, obviously-correct float64 numpy, written from the definitions on the
source pages. Each function cites the page and section it follows:

* "IAM: Efficient Inference through Attention Mapping between Different-scale
  LLMs" (paper notes, ACL 2025) -- sections Method 1 (similarity metric on
  flattened maps), Method 2 (mapped-layer order), Method 4 (mapping and
  inference: per-head argmax at prefill, decode reuse, tau thresholds).
* "MapFlow: attention maps reused across models" (news article on "Accelerating
  Cross-Model LLM Inference via Attention Map Reuse") -- the approach section
  (layer mapping, heads combined by learned linear weights, receiver keeps its
  own V) and the storage-and-execution section (block-sparse retention by
  cumulative probability with regular 2-D blocks, two phases: block statistics
  then extraction; fused kernel that mixes heads on chip and multiplies by V).
* "GLIDE: Guided Layerwise Hybrid Attention" -- sections II-A/II-B (causal
  scaled dot-product softmax attention over all earlier keys).

Readings where the pages are silent are stated in the functions' docstrings.
Every function here is pinned by ``tests/test_oracle_*.py`` against closed
forms, invariants, library special cases or brute force.
"""
from .numerics import round_bf16, round_f32
from .attention import causal_map, attn_maps, pack_rows, packed_size, seq_lengths
from .cosine import cosine_matrix, head_map
from .compress import (BLOCK, block_masses, select_blocks, selection_margin, compress_head,
                       compress_block_row, block_compress, row_stats)
from .mapped_av import dense_from_bsr_rows, mapped_av_dense, mapped_av_bsr_rows, mix_maps
from .layers import mapped_layers, mapping_plan, onehot_mix
from .prefix import fnv1a64, prefix_hashes, PrefixIndexModel

__all__ = [
    "round_bf16", "round_f32", "causal_map", "attn_maps", "pack_rows", "packed_size",
    "seq_lengths", "cosine_matrix", "head_map", "BLOCK", "block_masses", "select_blocks",
    "selection_margin", "compress_head", "compress_block_row", "block_compress", "row_stats", "dense_from_bsr_rows",
    "mapped_av_dense", "mapped_av_bsr_rows", "mix_maps", "mapped_layers", "mapping_plan", "onehot_mix",
    "fnv1a64", "prefix_hashes", "PrefixIndexModel",
]
