"""Seeded synthetic inputs for the CSA decode path.

This module only draws random numbers and lays them out.  It holds none of
the method's arithmetic (no softmax, no scoring, no selection, no attention)
and is shared by the tests, the smoke check and the benchmark: the same seed
gives both the HIP path and the CPU oracle the same bits.

Storage types: ``"f32"`` arrays are float32; ``"bf16"`` arrays are returned as
uint16 bit patterns (rounded to nearest-even from float32 by torch), which the
oracle decodes exactly and the HIP path reads as bfloat16.

Workload shapes (one CSA layer each unless stated), from the decode workloads
this library is measured on:

* ``tiny``     — context 1024 (n_comp 256), batch 1, fp32; indexer 64x128,
  top_k 64, SWA 128; main attention 16 heads x 128.
* ``ctx8k``    — context 8192 (n_comp 2048), batch 1, bf16; top_k 512, SWA 128,
  main attention 64 heads x 512 (gather_buf 640 x 512).
* ``batch128k``— 8 sequences at context 131072 (n_comp 32768 each), bf16.
* ``ctx1m``    — context 1,000,000 (n_comp 250,000), batch 1, bf16, 30 layers.
* ``prefill``  — 2048 query tokens at positions 260096..262143 against 65536
  compressed blocks with the causal block mask.
* ``hca1m``    — an HCA layer (ratio 128, no indexer) at context 1,000,064
  (n_comp 7813 after the step), 30 layers; main attention as ``ctx1m``.

Context ``ctx`` counts the new token: it sits at position ``ctx - 1``.  With
ratio 4 and ``ctx % 4 == 0`` the new token completes block ``n_comp - 1``, so
every decode step compresses one block (the worst case) and the caches hold
``n_comp - 1`` entries before the step.  The SWA ring holds the previous
``min(pos, W)`` tokens with its next write slot at ``pos % W``.

Value distributions: compressor Z and C ~ N(0, 1) and B ~ N(0, 0.1^2);
indexer queries ~ N(0, 1)/sqrt(128) (the 1/sqrt(d_I) factor is folded into
q), head weights ~ N(0, 1), indexer keys ~ N(0, 1); main q, KV rows and
compressed entries ~ N(0, 1) then RMS-normalised per row for the bf16
workloads; sink logits ~ N(0, 1).  Seeds: ``1000 * config_number + layer``.
"""

from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Dict, Optional

import numpy as np

__all__ = ["Shape", "SHAPES", "CONFIG_NUMBER", "seed_for", "make_decode_inputs",
           "make_decode_inputs_torch", "make_prefill_inputs", "make_prefill_inputs_torch",
           "to_bf16_bits", "rng"]


@dataclass(frozen=True)
class Shape:
    name: str
    batch: int
    n_comp: int          # compressed entries after this step's compression
    ctx: int             # tokens including the new one
    h_i: int = 64        # indexer heads
    d_i: int = 128       # indexer key width
    h: int = 64          # main query heads
    d: int = 512         # main head dim (shared K = V)
    top_k: int = 512
    w: int = 128         # SWA window
    m: int = 4           # compression ratio
    dtype: str = "bf16"  # storage type of q, keys, caches
    layers: int = 1
    rms_norm: bool = True
    overlap: bool = False
    t: int = 1           # query tokens per sequence (prefill > 1)

    @property
    def pos(self) -> int:
        return self.ctx - 1

    @property
    def max_comp(self) -> int:
        return self.n_comp

    def gather_rows(self) -> int:
        return self.top_k + self.w


SHAPES: Dict[str, Shape] = {
    "tiny": Shape("tiny", batch=1, n_comp=256, ctx=1024, h=16, d=128, top_k=64,
                  dtype="f32", rms_norm=False),
    "ctx8k": Shape("ctx8k", batch=1, n_comp=2048, ctx=8192),
    "batch128k": Shape("batch128k", batch=8, n_comp=32768, ctx=131072),
    "ctx1m": Shape("ctx1m", batch=1, n_comp=250000, ctx=1000000, layers=30),
    "prefill": Shape("prefill", batch=1, n_comp=65536, ctx=262144, t=2048),
    # an HCA layer (ratio 128, no indexer) at 1M context; ctx = 7813 * 128 so
    # the step completes a block, as the CSA workloads do
    "hca1m": Shape("hca1m", batch=1, n_comp=7813, ctx=1_000_064, m=128, layers=30),
}

CONFIG_NUMBER = {"tiny": 1, "ctx8k": 2, "batch128k": 3, "ctx1m": 4, "prefill": 5, "hca1m": 6}


def seed_for(shape: Shape, layer: int = 0) -> int:
    return 1000 * CONFIG_NUMBER.get(shape.name, 9) + layer


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even (torch)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def _rms_rows(x: np.ndarray) -> np.ndarray:
    # input preparation only: unit-RMS rows, as the model normalises q and KV
    # before they reach the attention step
    ms = np.mean(x.astype(np.float64) ** 2, axis=-1, keepdims=True)
    return (x / np.sqrt(ms + 1e-6)).astype(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return to_bf16_bits(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def make_decode_inputs(shape: Shape, seed: int, max_comp: Optional[int] = None) -> dict:
    """Host (numpy) inputs for one decode step of one layer, batch-major.

    Returns a dict with the caches before the step (``comp_kv [B, max_comp, D]``,
    ``idx_keys [B, max_comp, d_I]``, ``swa [B, W, D]``), the layer weights
    (``main_bias [m, D]``, ``idx_bias [m, d_I]``, ``sink [H]``), the step's
    inputs (``q [B, H, D]``, ``q_idx [B, H_I, d_I]``, ``w_idx [B, H_I]``,
    ``kv_new [B, D]``, ``z_main``/``c_main [B, m, D]``, ``z_idx``/``c_idx
    [B, m, d_I]``) and the host-known counters ``n_comp`` (entries before the
    step), ``swa_head``, ``swa_len`` and ``pos``.  Cache slots at and beyond
    ``n_comp`` hold random bits as well: the step must overwrite slot
    ``n_comp`` and never read beyond it.
    """
    g = rng(seed)
    B, N, D, di, W, m = shape.batch, shape.n_comp, shape.d, shape.d_i, shape.w, shape.m
    mc = max_comp if max_comp is not None else N
    f32 = np.float32

    def normal(*sz, std=1.0):
        return (g.standard_normal(sz, dtype=f32) * f32(std)).astype(f32)

    def rows(*sz):
        x = normal(*sz)
        return _rms_rows(x) if shape.rms_norm else x

    width_main = 2 * D if shape.overlap else D
    width_idx = 2 * di if shape.overlap else di
    zrows = 2 * m if shape.overlap else m
    out = {
        "comp_kv": _store(rows(B, mc, D), shape.dtype),
        "idx_keys": _store(normal(B, mc, di), shape.dtype),
        "swa": _store(rows(B, W, D), shape.dtype),
        "main_bias": normal(m, width_main, std=0.1),
        "idx_bias": normal(m, width_idx, std=0.1),
        "sink": normal(shape.h),
        "q": _store(rows(B, shape.h, D), shape.dtype),
        "q_idx": _store(normal(B, shape.h_i, di, std=1.0 / np.sqrt(di)), shape.dtype),
        "w_idx": normal(B, shape.h_i),
        "kv_new": _store(rows(B, D), shape.dtype),
        "z_main": normal(B, zrows, width_main),
        "c_main": normal(B, zrows, width_main),
        "z_idx": normal(B, zrows, width_idx),
        "c_idx": normal(B, zrows, width_idx),
    }
    pos = shape.pos
    out.update(n_comp=N - 1 if pos % m == m - 1 else N, swa_head=pos % W,
               swa_len=min(pos, W), pos=pos)
    return out


def make_decode_inputs_torch(shape: Shape, seed: int, device, layers: Optional[int] = None):
    """Device-resident inputs for large caches, drawn with torch's seeded generator.

    Same layout and distributions as :func:`make_decode_inputs`, but generated
    on ``device`` (the multi-GB caches of the long-context workloads are not
    built on the host).  Returns a list (one dict per layer) of torch tensors
    plus the host-known counters.
    """
    import torch
    nl = layers if layers is not None else shape.layers
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    B, N, D, di, W, m = shape.batch, shape.n_comp, shape.d, shape.d_i, shape.w, shape.m
    width_main = 2 * D if shape.overlap else D
    width_idx = 2 * di if shape.overlap else di
    zrows = 2 * m if shape.overlap else m
    res = []
    for layer in range(nl):
        gen = torch.Generator(device=device)
        gen.manual_seed(seed_for(shape, layer) if seed is None else seed + layer)

        def normal(*sz, std=1.0):
            return torch.randn(*sz, generator=gen, device=device, dtype=torch.float32) * std

        def rows(*sz):
            x = normal(*sz)
            if shape.rms_norm:
                x = x * torch.rsqrt(x.square().mean(-1, keepdim=True) + 1e-6)
            return x

        d = {
            "comp_kv": rows(B, N, D).to(dt),
            "idx_keys": normal(B, N, di).to(dt),
            "swa": rows(B, W, D).to(dt),
            "main_bias": normal(m, width_main, std=0.1),
            "idx_bias": normal(m, width_idx, std=0.1),
            "sink": normal(shape.h),
            "q": rows(B, shape.h, D).to(dt),
            "q_idx": (normal(B, shape.h_i, di) / float(np.sqrt(di))).to(dt),
            "w_idx": normal(B, shape.h_i),
            "kv_new": rows(B, D).to(dt),
            "z_main": normal(B, zrows, width_main),
            "c_main": normal(B, zrows, width_main),
            "z_idx": normal(B, zrows, width_idx),
            "c_idx": normal(B, zrows, width_idx),
        }
        pos = shape.pos
        d.update(n_comp=N - 1 if pos % m == m - 1 else N, swa_head=pos % W,
                 swa_len=min(pos, W), pos=pos)
        res.append(d)
    return res


def make_prefill_inputs(shape: Shape, seed: int) -> dict:
    """Host (numpy) inputs of a prefill-shaped chunk: ``shape.t`` query tokens
    at positions ``pos0 .. pos0 + t - 1`` (``pos0 = ctx - t``) against
    ``n_comp`` compressed blocks (the chunk's own blocks included).

    Returns ``q_idx [t, H_I, d_I]``, ``w_idx [t, H_I]``, ``idx_keys [N, d_I]``,
    ``comp_kv [N, D]``, ``q [t, H, D]``, ``win_kv [t + W - 1, D]`` (row ``i``
    = the raw KV of position ``pos0 - W + 1 + i``), ``sink [H]`` and ``pos0``.
    """
    g = rng(seed)
    T, N, D, di, W = shape.t, shape.n_comp, shape.d, shape.d_i, shape.w
    f32 = np.float32

    def normal(*sz, std=1.0):
        return (g.standard_normal(sz, dtype=f32) * f32(std)).astype(f32)

    def rows(*sz):
        x = normal(*sz)
        return _rms_rows(x) if shape.rms_norm else x

    return {
        "q_idx": _store(normal(T, shape.h_i, di, std=1.0 / np.sqrt(di)), shape.dtype),
        "w_idx": normal(T, shape.h_i),
        "idx_keys": _store(normal(N, di), shape.dtype),
        "comp_kv": _store(rows(N, D), shape.dtype),
        "q": _store(rows(T, shape.h, D), shape.dtype),
        "win_kv": _store(rows(T + W - 1, D), shape.dtype),
        "sink": normal(shape.h),
        "pos0": shape.ctx - T,
    }


def make_prefill_inputs_torch(shape: Shape, seed: Optional[int], device) -> dict:
    """Device-resident prefill inputs (same layout and distributions as
    :func:`make_prefill_inputs`), drawn with torch's seeded generator."""
    import torch
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    T, N, D, di, W = shape.t, shape.n_comp, shape.d, shape.d_i, shape.w
    gen = torch.Generator(device=device)
    gen.manual_seed(seed_for(shape) if seed is None else seed)

    def normal(*sz, std=1.0):
        return torch.randn(*sz, generator=gen, device=device, dtype=torch.float32) * std

    def rows(*sz):
        x = normal(*sz)
        if shape.rms_norm:
            x = x * torch.rsqrt(x.square().mean(-1, keepdim=True) + 1e-6)
        return x

    return {
        "q_idx": (normal(T, shape.h_i, di) / float(np.sqrt(di))).to(dt),
        "w_idx": normal(T, shape.h_i),
        "idx_keys": normal(N, di).to(dt),
        "comp_kv": rows(N, D).to(dt),
        "q": rows(T, shape.h, D).to(dt),
        "win_kv": rows(T + W - 1, D).to(dt),
        "sink": normal(shape.h),
        "pos0": shape.ctx - T,
    }


def with_(shape: Shape, **kw) -> Shape:
    """A copy of ``shape`` with some fields changed (edge-case workloads)."""
    return replace(shape, **kw)


def cluster_direction(q_idx, w_idx):
    """Unit direction ``[B, d]`` of each sequence's indexer query heads with
    positive weight (their weighted sum); keys along it score high."""
    w = w_idx.float().clamp(min=0.0)
    u = (w[..., None] * q_idx.float()).sum(dim=1)
    return u / u.norm(dim=-1, keepdim=True).clamp(min=1e-30)


def cluster_recent_keys(idx_keys, q_idx, w_idx, end: int, count: int, seed: int, strength: float = 20.0):
    """Recent-context locality, in place: the ``count`` indexer keys before
    block ``end`` of every sequence are redrawn as unit normal noise plus
    ``strength`` times the unit direction of that sequence's query heads with
    positive weight (their weighted sum).  Those keys then outscore the rest
    of the cache, so the whole top-k falls in a few neighbouring blocks — the
    case in which per-slice candidate lists cannot prove the selection.

    ``idx_keys`` ``[B, N, d]``, ``q_idx`` ``[B, H, d]``, ``w_idx`` ``[B, H]``:
    torch tensors on one device."""
    import torch
    B, _, di = idx_keys.shape
    u = cluster_direction(q_idx, w_idx)
    gen = torch.Generator(device=idx_keys.device)
    gen.manual_seed(seed)
    noise = torch.randn(B, count, di, generator=gen, device=idx_keys.device, dtype=torch.float32)
    idx_keys[:, end - count:end] = (noise + strength * u[:, None, :]).to(idx_keys.dtype)
    return idx_keys
