"""Helpers for the GPU parity tests: host<->device conversion of synthetic
inputs and the comparison rules (tolerances stated where they are used)."""

from __future__ import annotations

import numpy as np
import torch

from oracle import numfmt

DEV = "cuda:0"


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 patterns -> device bfloat16 tensor (same bits)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def dev_f32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_store(a: np.ndarray) -> torch.Tensor:
    return dev_bf16(a) if a.dtype == np.uint16 else dev_f32(a)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """device bfloat16 -> uint16 patterns on the host."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a device bf16/f32 tensor."""
    if t.dtype == torch.bfloat16:
        return numfmt.bf16_bits_to_f64(host_bits(t))
    return t.detach().cpu().numpy().astype(np.float64)


def as_f64(a: np.ndarray) -> np.ndarray:
    """Exact float64 values of a host synthetic array (uint16 = bf16 bits)."""
    return numfmt.bf16_bits_to_f64(a) if a.dtype == np.uint16 else np.asarray(a, dtype=np.float64)


def rel_err(g, r) -> float:
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    if r.size == 0:
        return 0.0
    scale = max(np.abs(r).max(), 1e-30)
    return float(np.abs(g - r).max() / scale)


def assert_lse_close(g, r, abs_tol: float = 1e-2, rel_tol: float = 2e-2) -> None:
    """Log-sum-exp of the bf16 path: the relative rule of the other outputs
    (max |diff| / max |oracle|) and an absolute bound, both."""
    g = np.asarray(g, dtype=np.float64)
    r = np.asarray(r, dtype=np.float64)
    assert rel_err(g, r) <= rel_tol, rel_err(g, r)
    assert np.abs(g - r).max() <= abs_tol, np.abs(g - r).max()


def assert_bf16_close(g_bits: np.ndarray, exact: np.ndarray, ulps: int = 1) -> None:
    """bf16 output within `ulps` of round-to-nearest-even(exact)."""
    g = numfmt.bf16_bits_to_f64(g_bits)
    r = numfmt.bf16_round_f64(exact)
    _, e = np.frexp(np.where(r == 0, 1e-38, r))
    ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    bad = np.abs(g - r) > ulps * ulp
    assert not bad.any(), f"{bad.sum()} bf16 values off by more than {ulps} ulp (max diff {np.abs(g - r).max()})"


def assert_topk_gap_rule(gpu_idx: np.ndarray, gpu_count: int, oracle_scores: np.ndarray, k: int,
                         rel_gap: float = 1e-3) -> None:
    """Top-k agreement with the oracle's float64 scores: if the gap between the
    k-th and (k+1)-th oracle scores exceeds rel_gap * |s_k| the index sets must
    match exactly; otherwise every index in the symmetric difference must have
    an oracle score within rel_gap * |s_k| of s_k."""
    s = np.asarray(oracle_scores, dtype=np.float64)
    valid = np.flatnonzero(s > -np.inf)
    k_eff = min(k, valid.size)
    assert gpu_count == k_eff, f"count {gpu_count} != {k_eff}"
    sel = gpu_idx[:k_eff]
    assert (gpu_idx[k_eff:] == -1).all()
    assert len(set(sel.tolist())) == k_eff, "duplicate indices"
    if k_eff == 0:
        return
    order = valid[np.lexsort((valid, -s[valid]))]
    ref = set(order[:k_eff].tolist())
    sk = s[order[k_eff - 1]]
    tol = rel_gap * max(abs(sk), 1e-30)
    if k_eff < valid.size:
        gap = sk - s[order[k_eff]]
        if gap > tol:
            assert set(sel.tolist()) == ref, "top-k set differs although the k/k+1 gap is large"
            return
    diff = set(sel.tolist()) ^ ref
    for i in diff:
        assert abs(s[i] - sk) <= tol, f"index {i} score {s[i]} vs s_k {sk}"


def assert_fp4_key_close(codes_packed, scales, y):
    """A key the GPU quantised from its own float32 compressor output, next
    to the oracle's float64 key y: each block's exponent within one of the
    oracle's rule applied to y, each element within the largest E2M1 half
    gap (2^X) of y plus float32 slack."""
    c = numfmt.unpack_e2m1(np.asarray(codes_packed, dtype=np.uint8)[None])
    s = np.asarray(scales, dtype=np.uint8)[None]
    dec = numfmt.mxfp4_decode_rows(c, s)[0]
    _, rs = numfmt.quantize_mxfp4_rows(np.asarray(y, dtype=np.float32)[None])
    assert np.abs(s.astype(np.int64) - rs.astype(np.int64)).max() <= 1
    X = np.repeat(np.ldexp(1.0, s[0].astype(np.int64) - 127), 32)
    assert (np.abs(dec - y) <= X + 1e-5 * np.abs(y).max()).all()
