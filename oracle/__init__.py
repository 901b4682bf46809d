"""CPU oracle of the CSA decode path — TEST INFRASTRUCTURE, not product code.

A plain, slow float64 NumPy restatement of what the pages define for the five
steps (compressor reduce, lightning-indexer score, top-k, gather, sparse
attention with a sink) and their composition into one decode step.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import it.  The HIP library and its Python binding
never do, and the two share no code.  Parity pins: ``tests/test_oracle_pins.py``.
"""

from . import numfmt
from .csa import (
    LayerState,
    SwaRing,
    compress,
    decode_step,
    gather,
    hca_decode_step,
    index_score,
    index_score_fp4,
    index_score_fp8,
    kv_norm,
    mixed_kv_row,
    prefill_chunk,
    rescored_topk,
    rope_rotate,
    sparse_attn,
    topk,
)

__all__ = [
    "numfmt",
    "compress",
    "kv_norm",
    "rope_rotate",
    "mixed_kv_row",
    "index_score",
    "index_score_fp4",
    "index_score_fp8",
    "topk",
    "rescored_topk",
    "gather",
    "sparse_attn",
    "SwaRing",
    "LayerState",
    "decode_step",
    "hca_decode_step",
    "prefill_chunk",
]
