"""Plain float64 CPU oracle of the CSA decode path — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never imports, links or
calls it, and it shares no code, table or helper with the HIP sources.

Sources are the three web pages (git compare views of the
``nvfp4-megamoe-kernel`` repository, a DeepSeek-V4 inference bring-up):

* page 1 — compare ``v0.1-e2e-working...v-c1-c2-c3-20260602``
* page 2 — compare ``master..pure-nvfp4``
* page 3 — compare ``v-precision-floor-fix-20260603..pure-nvfp4``

Each function cites the file and section on those pages that it follows.
Everything is computed in float64 from inputs that were already decoded
exactly (see :mod:`oracle.numfmt`); output rounding to a storage format is
applied once, at the end, by the caller or by an explicit helper.

Parity pins for every function here live in ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "rescored_topk",
    "index_score_fp4",
    "compress",
    "kv_norm",
    "index_score",
    "topk",
    "gather",
    "sparse_attn",
    "SwaRing",
    "LayerState",
    "decode_step",
    "hca_decode_step",
    "prefill_chunk",
]


# ---------------------------------------------------------------------------
# (1) compressor reduce
# ---------------------------------------------------------------------------

def _softmax_weighted_sum(logits: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Per column: softmax over the rows of ``logits``, then the weighted sum of ``values``.

    The max is subtracted before ``exp`` as in the two-pass kernel (pass 1 the
    column max, pass 2 the exp-sum and the weighted sum).
    """
    mx = logits.max(axis=0)
    e = np.exp(logits - mx)
    return (e * values).sum(axis=0) / e.sum(axis=0)


def compress(Z, C, B, m: int, overlap: bool = False) -> np.ndarray:
    """Compress every complete block of ``m`` token rows into one entry.

    Page 1, ``dsv4/kernels/cuda/compressor_reduce.cu``, file header (paper
    eq. 9–12) and the two kernels ``hca_compress_reduce_kernel`` /
    ``csa_compress_reduce_kernel``; with the fix published on page 2 and page 3
    (commit "Fix two correctness bugs: compressor pos bias on KV"): the
    positional bias ``B`` is added to the softmax logits ``Z`` only and never to
    the content ``C``.  Compression is softmax(Z + B) over the block's token
    rows, per channel, followed by the weighted sum of ``C``.

    ``overlap=False`` (ratio-m blocks, no overlap — the HCA form, and the 4xD
    blocks of the decode workloads): ``Z``, ``C`` are ``[T, D]`` and ``B`` is
    ``[m, D]``.  Block ``i`` uses rows ``i*m .. i*m+m-1`` with bias row ``t``
    for its ``t``-th token.

    ``overlap=True`` (the overlapped CSA form): ``Z``, ``C`` are ``[T, 2D]``
    holding an "a" half (columns ``0..D-1``) and a "b" half (``D..2D-1``), and
    ``B`` is ``[m, 2D]``.  Block 0 uses its own ``m`` rows of the b half.  Block
    ``i > 0`` forms one joint softmax over ``2m`` rows: the ``m`` rows of block
    ``i-1`` from the a half (bias rows ``0..m-1`` of the a half) followed by its
    own ``m`` rows from the b half (bias rows ``0..m-1`` of the b half).

    Tail rows (``T mod m``) are ignored: ``n_blocks = T // m``
    (page 1, ``production_compress.py``, ``csa_compress_production``).
    Returns float64 ``[n_blocks, D]``.
    """
    Z = np.asarray(Z, dtype=np.float64)
    C = np.asarray(C, dtype=np.float64)
    B = np.asarray(B, dtype=np.float64)
    if Z.shape != C.shape or Z.ndim != 2:
        raise ValueError("Z and C must be 2-D arrays of the same shape")
    T, width = Z.shape
    if B.shape != (m, width):
        raise ValueError(f"B must be [{m}, {width}], got {B.shape}")
    n_blocks = T // m
    if not overlap:
        D = width
        out = np.empty((n_blocks, D), dtype=np.float64)
        for i in range(n_blocks):
            rows = slice(i * m, (i + 1) * m)
            out[i] = _softmax_weighted_sum(Z[rows] + B, C[rows])
        return out
    if width % 2:
        raise ValueError("overlapped inputs need an even width (a half | b half)")
    D = width // 2
    out = np.empty((n_blocks, D), dtype=np.float64)
    a, b = slice(0, D), slice(D, 2 * D)
    for i in range(n_blocks):
        cur = slice(i * m, (i + 1) * m)
        if i == 0:
            logits = Z[cur, b] + B[:, b]
            values = C[cur, b]
        else:
            prev = slice((i - 1) * m, i * m)
            logits = np.concatenate([Z[prev, a] + B[:, a], Z[cur, b] + B[:, b]], axis=0)
            values = np.concatenate([C[prev, a], C[cur, b]], axis=0)
        out[i] = _softmax_weighted_sum(logits, values)
    return out


def kv_norm(y, weight, eps: float = 1e-6) -> np.ndarray:
    """Weighted RMSNorm applied to each compressed row.

    Page 1, ``compressor_reduce.cu``, ``apply_kv_norm_kernel``:
    ``x * rsqrt(mean(x^2) + 1e-6) * w`` over the row's channels.
    """
    y = np.asarray(y, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    ms = (y * y).mean(axis=-1, keepdims=True)
    return y / np.sqrt(ms + eps) * w


# ---------------------------------------------------------------------------
# (2) lightning-indexer score
# ---------------------------------------------------------------------------

def index_score(q, w, K, q_pos=None, ratio: int = 4) -> np.ndarray:
    """Lightning-indexer score of every compressed block for every query row.

    Page 1, ``ARCHITECTURE_AND_MEMORY_AUDIT.md``, finding F3 (paper §2.3.1,
    eq. 16): ``I[t,s] = sum_h w[t,h] * ReLU(q[t,h] . K[s])`` where ``K[s]`` is
    ONE key per compressed block shared by every indexer head (MQA; einsum
    ``'tnd,cd->tnc'``, then ReLU, then the head-weighted sum).  No extra scale.

    ``q``: ``[T, H, d]``, ``w``: ``[T, H]``, ``K``: ``[N, d]``.

    Causal variant (page 1, ``archived_plans/NEXT_STEPS.md``, Issue 2 and
    "Immediate Next Steps" 1): a query at position ``p`` may only use blocks
    whose window ends at or before ``p``.  Block ``s`` covers positions
    ``ratio*s .. ratio*s + ratio - 1``, so it is visible iff
    ``ratio*s + ratio - 1 <= p``; hidden blocks score ``-inf``.
    Returns float64 ``[T, N]``.
    """
    q = np.asarray(q, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    if q.ndim != 3 or w.shape != q.shape[:2] or K.ndim != 2 or K.shape[1] != q.shape[2]:
        raise ValueError(f"bad shapes q{q.shape} w{w.shape} K{K.shape}")
    T, H, _ = q.shape
    N = K.shape[0]
    out = np.empty((T, N), dtype=np.float64)
    for t in range(T):
        dots = q[t] @ K.T                      # [H, N]: q[t,h] . K[s]
        relu = np.maximum(dots, 0.0)
        out[t] = (w[t][:, None] * relu).sum(axis=0)
    if q_pos is not None:
        pos = np.asarray(q_pos, dtype=np.int64).reshape(T)
        block_end = ratio * np.arange(N, dtype=np.int64) + (ratio - 1)
        hidden = block_end[None, :] > pos[:, None]
        out[hidden] = -np.inf
    return out


def index_score_fp8(q_codes, w, k_codes, k_scale, q_pos=None, ratio: int = 4) -> np.ndarray:
    """The index score with FP8 E4M3 query and keys (the pages' FP8 scoring
    path: keys stored as FP8_E4M3, page 1, ``single_shot_inference.py``, "B2").

    Key s decodes to ``e4m3(k_codes[s]) * k_scale[s]``; the query decodes to
    ``e4m3(q_codes)`` with any per-head scale already folded into ``w`` (for a
    positive scale c, ``ReLU(c * x) = c * ReLU(x)``).  So
    ``I[t,s] = sum_h w[t,h] * ReLU(k_scale[s] * (e4m3(q[t,h]) . e4m3(K[s])))``,
    computed exactly in float64 from the decoded values.  ``q_codes``
    ``[T, H, d]`` uint8, ``w`` ``[T, H]``, ``k_codes`` ``[N, d]`` uint8,
    ``k_scale`` ``[N]``.  Returns float64 ``[T, N]`` (causal mask as in
    :func:`index_score`).
    """
    from .numfmt import e4m3_decode

    qd = e4m3_decode(np.asarray(q_codes, dtype=np.uint8))
    kd = e4m3_decode(np.asarray(k_codes, dtype=np.uint8))
    ks = np.asarray(k_scale, dtype=np.float64)
    if kd.ndim != 2 or ks.shape != (kd.shape[0],):
        raise ValueError(f"bad key shapes {kd.shape} {ks.shape}")
    w = np.asarray(w, dtype=np.float64)
    T, H, _ = qd.shape
    out = np.empty((T, kd.shape[0]), dtype=np.float64)
    for t in range(T):
        dots = (qd[t] @ kd.T) * ks[None, :]    # [H, N]: k_scale[s] * (q[t,h] . K[s])
        out[t] = (w[t][:, None] * np.maximum(dots, 0.0)).sum(axis=0)
    if q_pos is not None:
        pos = np.asarray(q_pos, dtype=np.int64).reshape(T)
        block_end = ratio * np.arange(kd.shape[0], dtype=np.int64) + (ratio - 1)
        out[block_end[None, :] > pos[:, None]] = -np.inf
    return out


def index_score_fp4(q_codes, w, k_codes, k_scales, q_pos=None, ratio: int = 4) -> np.ndarray:
    """The index score with an FP8 E4M3 query and FP4 E2M1 keys with E8M0
    block scales (the FP4 indexer cache of page 1,
    ``ARCHITECTURE_AND_MEMORY_AUDIT.md``, C4, paired with FP4 tensor-core
    scoring; block layout per reading R30).

    Key s decodes to ``e2m1(k_codes[s, j]) * 2^(k_scales[s, j // 32] - 127)``
    (:func:`numfmt.mxfp4_decode_rows`); the query decodes to ``e4m3(q_codes)``
    with any per-head scale already folded into ``w`` (reading R20).  So
    ``I[t,s] = sum_h w[t,h] * ReLU(e4m3(q[t,h]) . K[s])``, computed exactly in
    float64 from the decoded values.  ``q_codes`` ``[T, H, d]`` uint8 (E4M3),
    ``w`` ``[T, H]``, ``k_codes`` ``[N, d]`` uint8 (one E2M1 code per
    element), ``k_scales`` ``[N, d / 32]`` uint8 (E8M0).  Returns float64
    ``[T, N]`` (causal mask as in :func:`index_score`).
    """
    from .numfmt import e4m3_decode, mxfp4_decode_rows

    qd = e4m3_decode(np.asarray(q_codes, dtype=np.uint8))
    kd = mxfp4_decode_rows(k_codes, k_scales)
    if kd.ndim != 2:
        raise ValueError(f"bad key shape {kd.shape}")
    w = np.asarray(w, dtype=np.float64)
    T = qd.shape[0]
    out = np.empty((T, kd.shape[0]), dtype=np.float64)
    for t in range(T):
        dots = qd[t] @ kd.T                    # [H, N]
        out[t] = (w[t][:, None] * np.maximum(dots, 0.0)).sum(axis=0)
    if q_pos is not None:
        pos = np.asarray(q_pos, dtype=np.int64).reshape(T)
        block_end = ratio * np.arange(kd.shape[0], dtype=np.int64) + (ratio - 1)
        out[block_end[None, :] > pos[:, None]] = -np.inf
    return out


# ---------------------------------------------------------------------------
# (3) top-k
# ---------------------------------------------------------------------------

def topk(scores, k: int):
    """Fixed-shape top-k of each score row with a lower-index tie-break.

    Page 1, ``ARCHITECTURE_AND_MEMORY_AUDIT.md`` F3 (``tk = min(top_k, n_comp)``;
    ``total.topk(tk, -1)``) and page 3, ``GETTING+CUDAGRAPH_READY.md``,
    Section C item 3 (always ``k`` slots, invalid ones masked, no host read of
    the count).  Valid entries are those with a score above ``-inf``.
    Ordering is (score descending, index ascending); equal scores go to the
    lower index.  ``+0.0`` and ``-0.0`` are equal scores.

    Returns ``idx`` int32 ``[T, k]`` (unused slots ``-1``) and ``count`` int32
    ``[T]`` with ``count = min(k, number of valid entries)``.
    """
    s = np.asarray(scores, dtype=np.float64)
    if s.ndim == 1:
        s = s[None, :]
    T, N = s.shape
    idx = np.full((T, k), -1, dtype=np.int32)
    count = np.zeros(T, dtype=np.int32)
    positions = np.arange(N, dtype=np.int64)
    for t in range(T):
        row = s[t]
        valid = row > -np.inf            # also drops NaN (out of contract)
        vpos = positions[valid]
        vval = row[valid]
        order = np.lexsort((vpos, -vval))  # primary: -score asc; then index asc
        k_eff = min(k, vpos.size)
        idx[t, :k_eff] = vpos[order[:k_eff]]
        count[t] = k_eff
    return idx, count


def rescored_topk(scores_fp8, scores_exact, k: int, k_cand: int):
    """Two-stage selection of an E4M3 indexer whose recall must meet the exact
    one's (reading R29: page 1, ``ARCHITECTURE_AND_MEMORY_AUDIT.md``, the
    recall test of Tier 1, gate 4, against an exact-score reference, with the
    keys kept as FP8_E4M3 for the FP8 scoring path of page 1,
    ``single_shot_inference.py``, "B2").

    Stage 1: the ``k_cand`` best entries of each row by ``scores_fp8``
    (:func:`topk`'s rules).  Stage 2: of those, the ``k`` best by
    ``scores_exact`` (same rules: score descending, lower index first).
    ``scores_exact`` need only be meaningful at the stage-1 entries.  Returns
    ``idx [T, k]`` (unused slots -1) and ``count [T]`` = ``min(k, stage-1
    count)``, like :func:`topk`.
    """
    e = np.asarray(scores_exact, dtype=np.float64)
    if e.ndim == 1:
        e = e[None, :]
    cand, ccount = topk(scores_fp8, k_cand)
    T = cand.shape[0]
    idx = np.full((T, k), -1, dtype=np.int32)
    count = np.zeros(T, dtype=np.int32)
    for t in range(T):
        c = cand[t, :ccount[t]].astype(np.int64)
        order = c[np.lexsort((c, -e[t, c]))]
        k_eff = min(k, c.size)
        idx[t, :k_eff] = order[:k_eff]
        count[t] = k_eff
    return idx, count


# ---------------------------------------------------------------------------
# (4) gather into gather_buf
# ---------------------------------------------------------------------------

def gather(comp_kv, idx, count: int, swa, swa_head: int, swa_len: int):
    """Fill ``gather_buf`` with the selected compressed rows, then the SWA window.

    Page 1 commit message C2 (one preallocated ``(top_k + window, hd)`` buffer
    filled by slice assignment, compressed rows then SWA rows) and C3 (the ring
    may wrap); page 1, ``PERFORMANCE_AUDIT.md`` P2 (token ``i`` of an append
    goes to slot ``(swa_head + i) % ws``; ``swa_len = min(swa_len + T, ws)``).
    ``swa_head`` is the next write slot, so the live window, oldest first, is
    slots ``(swa_head - swa_len + j) mod W`` for ``j = 0..swa_len-1``.

    Returns ``(rows, n_valid)`` where ``rows`` holds exactly the ``n_valid =
    count + swa_len`` valid rows (dtype of the inputs, values copied).
    """
    comp_kv = np.asarray(comp_kv)
    swa = np.asarray(swa)
    W = swa.shape[0]
    sel = [comp_kv[int(idx[j])] for j in range(count)]
    win = [swa[(swa_head - swa_len + j) % W] for j in range(swa_len)]
    rows = sel + win
    if rows:
        out = np.stack(rows, axis=0)
    else:
        out = np.zeros((0,) + comp_kv.shape[1:], dtype=comp_kv.dtype)
    return out, count + swa_len


# ---------------------------------------------------------------------------
# (5) shared-KV sparse attention with a per-head sink
# ---------------------------------------------------------------------------

def sparse_attn(q, kv, sink=None, scale: Optional[float] = None, return_weights: bool = False):
    """One softmax over the gathered rows plus a per-head sink logit.

    Page 1, ``fmha_6warp_tma_multirow_multitile.cuh`` hunk "Sink bias
    correction (D5c: single softmax over [S_comp, S_swa + sink])": the sink is
    one extra logit per head, already in the scaled domain, that enters the
    softmax denominator but has no value row.  Page 1, ``fmha_multitile_op.py``
    (MQA: every query head reads the same K/V with head stride 0) and
    ``PERFORMANCE_AUDIT.md`` P4 (``v = k``): keys and values are the same rows.
    Scale ``1/sqrt(hd)`` (page 2, ``single_shot_inference.py``,
    ``eager_attention``).

    For head ``h`` with rows ``j < n``:
    ``s_j = scale * q[h] . kv[j]``, ``M = max(max_j s_j, sink[h])``,
    ``den = sum_j exp(s_j - M) + exp(sink[h] - M)``,
    ``out[h] = sum_j exp(s_j - M) kv[j] / den`` and ``lse[h] = M + ln(den)``.
    With no rows and no sink the output is zero and ``lse`` is ``-inf``.

    ``q``: ``[H, D]``, ``kv``: ``[n, D]``, ``sink``: ``[H]`` or None.
    Returns float64 ``out [H, D]``, ``lse [H]`` (and the ``[H, n]`` row
    weights and ``[H]`` sink weights when ``return_weights``).
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    H, D = q.shape
    n = kv.shape[0]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    s = scale * (q @ kv.T) if n else np.zeros((H, 0))
    if sink is not None:
        sk = np.asarray(sink, dtype=np.float64).reshape(H)
    else:
        sk = np.full(H, -np.inf)
    row_max = s.max(axis=1) if n else np.full(H, -np.inf)
    M = np.maximum(row_max, sk)
    out = np.zeros((H, D), dtype=np.float64)
    lse = np.full(H, -np.inf, dtype=np.float64)
    weights = np.zeros((H, n), dtype=np.float64)
    sink_w = np.zeros(H, dtype=np.float64)
    for h in range(H):
        if M[h] == -np.inf:
            continue  # nothing to attend to
        e = np.exp(s[h] - M[h])
        es = math.exp(sk[h] - M[h]) if sk[h] > -np.inf else 0.0
        den = e.sum() + es
        out[h] = (e[:, None] * kv).sum(axis=0) / den
        lse[h] = M[h] + math.log(den)
        weights[h] = e / den
        sink_w[h] = es / den
    if return_weights:
        return out, lse, weights, sink_w
    return out, lse


# ---------------------------------------------------------------------------
# (5b) RoPE and the mixed E4M3 / bf16 main KV rows
# ---------------------------------------------------------------------------

def rope_rotate(x, cos, sin, inverse: bool = False) -> np.ndarray:
    """Rotate the last ``2 * len(cos)`` entries of ``x`` (the RoPE dims) in
    (even, odd) pairs; every other entry is returned unchanged.

    Page 1, ``PERFORMANCE_AUDIT.md`` P5 (``_apply_rope`` /
    ``_apply_rope_inplace``): the RoPE part is the trailing ``rope_dim``
    entries, paired as ``0::2`` / ``1::2``; the inverse printed there is
    ``(e c + o s, -e s + o c)``, so the forward rotation is its inverse,
    ``(e c - o s, e s + o c)``.  ``cos``/``sin`` hold the table row of one
    position (``rope_dim / 2`` values).  float64.
    """
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos, dtype=np.float64)
    s = np.asarray(sin, dtype=np.float64)
    rd = 2 * c.shape[-1]
    out = x.copy()
    ev = x[..., x.shape[-1] - rd::2]
    od = x[..., x.shape[-1] - rd + 1::2]
    if inverse:
        out[..., x.shape[-1] - rd::2] = ev * c + od * s
        out[..., x.shape[-1] - rd + 1::2] = -ev * s + od * c
    else:
        out[..., x.shape[-1] - rd::2] = ev * c - od * s
        out[..., x.shape[-1] - rd + 1::2] = ev * s + od * c
    return out


def mixed_kv_row(y, rope_dim: int, cos=None, sin=None):
    """One main-KV row in the mixed storage of page 2, ``eager_attention``
    (the "B1 storage-native mixed path"): the NoPE part (all but the last
    ``rope_dim`` entries) quantised from float32 to E4M3 with one row scale
    (:func:`numfmt.quantize_e4m3_rows`), the RoPE part kept in bfloat16 —
    rotated first when a table row is given (a compressed entry: its RoPE
    part is rounded to bfloat16, rotated, and rounded again, as ``_apply_rope``
    does on bfloat16 input).  Returns ``(codes, scale, rope, row)`` with
    ``row`` the float64 values an attention reads back."""
    from .numfmt import bf16_round_f64, e4m3_decode, quantize_e4m3_rows

    y32 = np.asarray(y, dtype=np.float32)
    nope = y32.shape[-1] - rope_dim
    codes, scale = quantize_e4m3_rows(y32[None, :nope])
    rope = bf16_round_f64(y32[nope:].astype(np.float64))
    if cos is not None:
        rope = bf16_round_f64(rope_rotate(rope, cos, sin))
    row = np.concatenate([e4m3_decode(codes[0]) * np.float64(scale[0]), rope])
    return codes[0], scale[0], rope, row


# ---------------------------------------------------------------------------
# (6) one decode step for one layer
# ---------------------------------------------------------------------------

@dataclass
class SwaRing:
    """Sliding-window ring of the last ``W`` token KV rows (page 1, P2)."""

    rows: np.ndarray          # [W, D]
    head: int = 0             # next write slot
    length: int = 0           # live rows, <= W

    def append(self, row) -> None:
        W = self.rows.shape[0]
        self.rows[self.head] = row
        self.head = (self.head + 1) % W
        self.length = min(self.length + 1, W)


@dataclass
class LayerState:
    """One CSA layer's caches, float64 values plus host-known counters.

    Preallocated compressed caches with a running count ``n_comp`` follow
    page 1, ``PERFORMANCE_AUDIT.md`` P3 and commit message C1.
    """

    comp_kv: np.ndarray       # [max_comp, D]
    idx_keys: np.ndarray      # [max_comp, d_I]
    n_comp: int
    swa: SwaRing
    main_bias: np.ndarray     # [m, D] (or [m, 2D] overlapped)
    idx_bias: np.ndarray      # [m, d_I] (or [m, 2 d_I])
    sink: Optional[np.ndarray] = None
    main_norm: Optional[np.ndarray] = None
    idx_norm: Optional[np.ndarray] = None
    m: int = 4
    overlap: bool = False
    round_cache: Optional[callable] = field(default=None, repr=False)
    # E4M3 indexer keys (page 1, single_shot_inference.py, "B2": keys kept as
    # FP8_E4M3 in the cache): codes [max_comp, d_I] uint8 and float32 row
    # scales [max_comp]; when set they replace idx_keys
    idx_codes: Optional[np.ndarray] = None
    idx_scales: Optional[np.ndarray] = None
    # FP4 indexer keys (page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, C4; block
    # layout per reading R30): with ``idx_fp4`` set, ``idx_codes`` holds one
    # E2M1 code per element [max_comp, d_I] and ``idx_scales`` the E8M0
    # block scales [max_comp, d_I / 32] uint8
    idx_fp4: bool = False
    # Mixed main KV (page 2, eager_attention, "B1"): comp_kv and the SWA ring
    # hold the values of mixed rows (:func:`mixed_kv_row`); compressed entries
    # get RoPE from the comp tables at their block index, the output inverse
    # RoPE from the token tables at the token's position.  Tables:
    # [rows, rope_dim / 2].
    # Recall-restored E4M3 keys (reading R29): with ``fp8_rescore`` = k_cand
    # > 0 the layer keeps its keys twice, as codes (``idx_codes`` /
    # ``idx_scales``) and in ``idx_keys`` (rounded by ``round_cache``), and
    # the top-k is :func:`rescored_topk` of the E4M3 scores and the exact
    # scores over ``idx_keys``
    fp8_rescore: int = 0
    kv_mixed: bool = False
    rope_dim: int = 64
    rope_cos: Optional[np.ndarray] = None
    rope_sin: Optional[np.ndarray] = None
    comp_rope_cos: Optional[np.ndarray] = None
    comp_rope_sin: Optional[np.ndarray] = None


def decode_step(L: LayerState, *, q, q_idx, w_idx, kv_new, pos: int, top_k: int,
                z_main=None, c_main=None, z_idx=None, c_idx=None,
                scale: Optional[float] = None):
    """One token through one CSA layer, in the pages' order.

    Page 2, ``single_shot_inference.py``, ``eager_attention``: KV append into
    the SWA ring → compressor (main KV, then the indexer's key compressor) →
    indexer top-k → gather → attention.  The compressor only emits an entry
    when the new token completes a block (page 1, ``PERFORMANCE_AUDIT.md`` P7):
    ``pos % m == m - 1``.  ``z_*``/``c_*`` hold the rows of that block (for the
    overlapped form: the previous block's rows followed by this block's rows,
    or this block's rows alone for block 0).  ``L.round_cache`` (e.g. bf16
    rounding) is applied to entries written into the caches, which is what a
    later step reads back.  Mutates ``L`` and returns a dict of every
    intermediate.

    With ``L.fp8_rescore`` set as well (reading R29) the new key is also
    stored in ``idx_keys`` and the selection is :func:`rescored_topk`; ``q_idx``
    must then be real-valued (the exact scores use it unquantised).

    With E4M3 indexer keys (``L.idx_codes`` set) the compressed key is taken
    to float32 and quantised per row (:func:`numfmt.quantize_e4m3_rows`) into
    ``L.idx_codes`` / ``L.idx_scales``, and the scores are
    :func:`index_score_fp8`; with ``L.idx_fp4`` as well the key is quantised
    by :func:`numfmt.quantize_mxfp4_rows` instead and the scores are
    :func:`index_score_fp4` (the query stays E4M3).  A real-valued ``q_idx``
    is quantised per row as E4M3, one row per head, and each head's scale is folded into its weight
    with one binary32 product (reading R20: ReLU(s x) = s ReLU(x) for s > 0);
    a uint8 ``q_idx`` is taken as codes whose scales ``w_idx`` already
    carries.

    With mixed main KV (``L.kv_mixed``) the new token's row (already rotated
    by the caller, as the pages' ``kv_roped``) and each compressed entry
    (rotated here at its block index ``pos // m`` with the comp tables) are
    stored as :func:`mixed_kv_row` values, and the attention output gets the
    inverse rotation at ``pos`` (the pages' "Inverse RoPE" after the FMHA).
    """
    from .numfmt import quantize_e4m3_rows, quantize_mxfp4_rows

    m = L.m
    fp8 = L.idx_codes is not None
    if L.kv_mixed:  # the new token's row arrives with its RoPE applied
        L.swa.append(mixed_kv_row(kv_new, L.rope_dim)[3])
    else:
        L.swa.append(np.asarray(kv_new, dtype=np.float64))
    rnd = L.round_cache if L.round_cache is not None else (lambda a: a)
    new_entry = None
    if pos % m == m - 1:
        # The last block of the given rows is the one this token completes
        # (for the overlapped form with a previous block, rows 0..m-1 are
        # that previous block, so block 1 of the input is the new one).
        ym = compress(z_main, c_main, L.main_bias, m, overlap=L.overlap)[-1]
        yi = compress(z_idx, c_idx, L.idx_bias, m, overlap=L.overlap)[-1]
        if L.main_norm is not None:
            ym = kv_norm(ym, L.main_norm)
        if L.idx_norm is not None:
            yi = kv_norm(yi, L.idx_norm)
        if L.kv_mixed:
            blk = pos // m
            L.comp_kv[L.n_comp] = mixed_kv_row(ym, L.rope_dim, L.comp_rope_cos[blk], L.comp_rope_sin[blk])[3]
        else:
            L.comp_kv[L.n_comp] = rnd(ym)
        if fp8:
            quant = quantize_mxfp4_rows if L.idx_fp4 else quantize_e4m3_rows
            codes, kscale = quant(np.asarray(yi, dtype=np.float32)[None])
            L.idx_codes[L.n_comp] = codes[0]
            L.idx_scales[L.n_comp] = kscale[0]
        if not fp8 or L.fp8_rescore:
            L.idx_keys[L.n_comp] = rnd(yi)
        new_entry = (ym, yi)
        L.n_comp += 1
    N = L.n_comp
    if fp8:
        q_codes, w_fold = np.asarray(q_idx), np.asarray(w_idx)
        if q_codes.dtype != np.uint8:
            q_codes, q_scale = quantize_e4m3_rows(q_codes.astype(np.float32))
            w_fold = (w_fold.astype(np.float32) * q_scale).astype(np.float32)
        score_fn = index_score_fp4 if L.idx_fp4 else index_score_fp8
        scores = score_fn(q_codes[None], w_fold[None], L.idx_codes[:N], L.idx_scales[:N])[0]
    else:
        scores = index_score(np.asarray(q_idx)[None], np.asarray(w_idx)[None], L.idx_keys[:N])[0]
    if fp8 and L.fp8_rescore:
        exact = index_score(np.asarray(q_idx, dtype=np.float64)[None], np.asarray(w_idx)[None], L.idx_keys[:N])[0]
        idx, count = rescored_topk(scores[None], exact[None], top_k, L.fp8_rescore)
    else:
        idx, count = topk(scores[None], top_k)
    rows, n_valid = gather(L.comp_kv[:N], idx[0], int(count[0]), L.swa.rows, L.swa.head, L.swa.length)
    out, lse = sparse_attn(q, rows, L.sink, scale)
    if L.kv_mixed:  # inverse RoPE of the output at the token's position
        out = rope_rotate(out, L.rope_cos[pos], L.rope_sin[pos], inverse=True)
    return {
        "new_entry": new_entry,
        "scores": scores,
        "idx": idx[0],
        "count": int(count[0]),
        "rows": rows,
        "n_valid": n_valid,
        "out": out,
        "lse": lse,
    }


# ---------------------------------------------------------------------------
# (6b) one decode step of a heavily compressed (HCA) layer
# ---------------------------------------------------------------------------

def hca_decode_step(L: LayerState, *, q, kv_new, pos: int, z_main=None, c_main=None,
                    scale: Optional[float] = None):
    """One token through one HCA layer: the CSA step without the indexer.

    Page 1, ``PERFORMANCE_AUDIT.md`` (the ``forward_attention`` branches):
    layers with a compression ratio above 4 attend to ALL compressed entries
    followed by the SWA window (``torch.cat([kv_cache.comp_kv, swa_kv])``);
    page 2, ``single_shot_inference.py``, ``eager_attention`` (the same branch
    in the mixed-precision gather, ``gather_mixed_all``).  The compressor is the
    plain, non-overlapped ratio-``m`` reduce (page 1,
    ``hca_compress_reduce_kernel``), run when the token completes a block.
    ``L.idx_keys`` is not used.  With mixed main KV (``L.kv_mixed``) the rows
    are stored, rotated and rotated back as in :func:`decode_step` (the
    pages' ``gather_mixed_all`` is the mixed gather of this branch).
    Mutates ``L``; returns the new entry, the attended rows and
    ``out``/``lse``.
    """
    m = L.m
    if L.kv_mixed:
        L.swa.append(mixed_kv_row(kv_new, L.rope_dim)[3])
    else:
        L.swa.append(np.asarray(kv_new, dtype=np.float64))
    rnd = L.round_cache if L.round_cache is not None else (lambda a: a)
    new_entry = None
    if pos % m == m - 1:
        ym = compress(z_main, c_main, L.main_bias, m, overlap=False)[-1]
        if L.main_norm is not None:
            ym = kv_norm(ym, L.main_norm)
        if L.kv_mixed:
            blk = pos // m
            L.comp_kv[L.n_comp] = mixed_kv_row(ym, L.rope_dim, L.comp_rope_cos[blk], L.comp_rope_sin[blk])[3]
        else:
            L.comp_kv[L.n_comp] = rnd(ym)
        new_entry = ym
        L.n_comp += 1
    N = L.n_comp
    W = L.swa.rows.shape[0]
    win = [L.swa.rows[(L.swa.head - L.swa.length + j) % W] for j in range(L.swa.length)]
    D = L.comp_kv.shape[1]
    rows = np.concatenate([np.asarray(L.comp_kv[:N], dtype=np.float64),
                           np.stack(win) if win else np.zeros((0, D))], axis=0)
    out, lse = sparse_attn(q, rows, L.sink, scale)
    if L.kv_mixed:
        out = rope_rotate(out, L.rope_cos[pos], L.rope_sin[pos], inverse=True)
    return {"new_entry": new_entry, "rows": rows, "n_valid": rows.shape[0], "out": out, "lse": lse}


# ---------------------------------------------------------------------------
# (7) a prefill-shaped chunk of query tokens against the compressed history
# ---------------------------------------------------------------------------

def prefill_chunk(*, q, q_idx, w_idx, idx_keys, comp_kv, win_kv, pos0: int, top_k: int, window: int,
                  sink=None, scale: Optional[float] = None, ratio: int = 4):
    """Score, select and attend for ``T`` consecutive query tokens at once.

    The query at position ``p = pos0 + t`` does what one decode step at ``p``
    does after its own token and every block complete at ``p`` are in the
    caches (page 2, ``single_shot_inference.py``, ``eager_attention``): the
    index score over the compressed history with the causal block mask (page
    1, ``archived_plans/NEXT_STEPS.md``, Issue 2: block ``s`` visible iff
    ``ratio*s + ratio - 1 <= p``), the fixed-shape top-k, then one softmax
    over the selected compressed rows followed by the sliding window — the raw
    KV rows of positions ``max(0, p - window + 1) .. p``, oldest first — plus
    the sink.

    ``q``: ``[T, H, D]``, ``q_idx``: ``[T, H_I, d_I]``, ``w_idx``: ``[T, H_I]``,
    ``idx_keys``: ``[N, d_I]``, ``comp_kv``: ``[N, D]`` (the chunk's own
    blocks included: the mask hides those not yet complete), ``win_kv``:
    ``[T + window - 1, D]``, row ``r`` holding position ``pos0 - window + 1 + r``
    (rows of negative positions are never read).  Returns a dict with
    ``scores [T, N]``, ``idx [T, top_k]``, ``count [T]``, ``out [T, H, D]`` and
    ``lse [T, H]``.
    """
    q = np.asarray(q, dtype=np.float64)
    win_kv = np.asarray(win_kv, dtype=np.float64)
    comp_kv = np.asarray(comp_kv, dtype=np.float64)
    T = q.shape[0]
    pos = pos0 + np.arange(T, dtype=np.int64)
    scores = index_score(q_idx, w_idx, idx_keys, q_pos=pos, ratio=ratio)
    idx, count = topk(scores, top_k)
    out = np.zeros(q.shape, dtype=np.float64)
    lse = np.zeros(q.shape[:2], dtype=np.float64)
    for t in range(T):
        p = int(pos[t])
        first = max(0, p - window + 1)
        win = [win_kv[x - (pos0 - window + 1)] for x in range(first, p + 1)]
        sel = [comp_kv[int(idx[t, j])] for j in range(int(count[t]))]
        rows = np.stack(sel + win, axis=0)
        out[t], lse[t] = sparse_attn(q[t], rows, sink, scale)
    return {"scores": scores, "idx": idx, "count": count, "out": out, "lse": lse}
