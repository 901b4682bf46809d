"""Thin ctypes binding of libcsa.so (include/csa.h), same names as the C ABI.

Argument marshalling only: tensors become device pointers, batch strides and
sizes are read from tensor shapes, the stream is torch's current stream.
Every step of the path runs in the HIP library; there is no fallback.  If the
library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcsa.so")

CSA_OK = 0
CSA_ERR_INVALID_ARG = -1
CSA_ERR_UNSUPPORTED = -2
CSA_ERR_LAUNCH = -3
CSA_ERR_WORKSPACE = -4
CSA_F32 = 0
CSA_BF16 = 1
CSA_FP8_E4M3 = 2
CSA_FP4_E2M1 = 3

_vp = ctypes.c_void_p
_i = ctypes.c_int
_ll = ctypes.c_longlong
_f = ctypes.c_float
_sz = ctypes.c_size_t


class CsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"CSA error {code}: {msg}")
        self.code = code


class LayerDesc(ctypes.Structure):
    _fields_ = [
        ("batch", _i), ("h", _i), ("d", _i), ("h_i", _i), ("d_i", _i), ("m", _i), ("w", _i),
        ("top_k", _i), ("overlap", _i), ("dtype", _i), ("out_dtype", _i),
        ("comp_kv", _vp), ("comp_kv_stride_b", _ll),
        ("idx_keys", _vp), ("idx_keys_stride_b", _ll),
        ("swa", _vp), ("swa_stride_b", _ll),
        ("max_comp", _i),
        ("main_bias", _vp), ("idx_bias", _vp), ("main_norm", _vp), ("idx_norm", _vp), ("sink", _vp),
        ("scale", _f),
        ("n_comp", _i), ("swa_head", _i), ("swa_len", _i),
        ("idx_dtype", _i), ("idx_scales", _vp), ("idx_scales_stride_b", _ll),
        ("kv_dtype", _i), ("rope_dim", _i),
        ("rope_cos", _vp), ("rope_sin", _vp), ("rope_rows", _i),
        ("comp_rope_cos", _vp), ("comp_rope_sin", _vp), ("comp_rope_rows", _i),
        ("idx_rescore", _i), ("idx_keys_exact", _vp), ("idx_keys_exact_stride_b", _ll),
    ]


class StepIO(ctypes.Structure):
    _fields_ = [
        ("pos", _i),
        ("q", _vp), ("q_stride_b", _ll),
        ("q_idx", _vp), ("q_idx_stride_b", _ll),
        ("w_idx", _vp), ("w_stride_b", _ll),
        ("kv_new", _vp), ("kv_new_stride_b", _ll),
        ("z_main", _vp), ("c_main", _vp), ("zc_main_stride_b", _ll),
        ("z_idx", _vp), ("c_idx", _vp), ("zc_idx_stride_b", _ll),
        ("scores", _vp), ("scores_stride_b", _ll),
        ("topk_idx", _vp), ("topk_count", _vp),
        ("gather_buf", _vp), ("gather_stride_b", _ll),
        ("n_valid", _vp),
        ("out", _vp), ("out_stride_b", _ll),
        ("lse", _vp),
    ]


_SIGS = {
    "csa_last_error": (ctypes.c_char_p, []),
    "csa_compress": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _ll, _ll, _vp]),
    "csa_index_score": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _i, _ll, _ll, _ll,
                             _ll, _ll, _vp]),
    "csa_quantize_fp8": (_i, [_vp, _i, _vp, _vp, _ll, _i, _vp]),
    "csa_quantize_fp4": (_i, [_vp, _i, _vp, _vp, _ll, _i, _vp]),
    "csa_index_score_fp4": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _ll, _ll, _ll, _ll, _ll, _ll,
                                 _vp]),
    "csa_quantize_query_fp8": (_i, [_vp, _i, _vp, _vp, _vp, _ll, _i, _i, _vp]),
    "csa_pack_kv_mixed": (_i, [_vp, _i, _vp, _ll, _i, _i, _vp]),
    "csa_index_score_fp8": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _i, _ll, _ll, _ll,
                                 _ll, _ll, _ll, _vp]),
    "csa_topk_workspace_size": (_sz, [_i, _i, _i, _i]),
    "csa_topk": (_i, [_vp, _i, _i, _i, _ll, _ll, _i, _vp, _vp, _vp, _sz, _vp]),
    "csa_gather": (_i, [_vp, _i, _vp, _vp, _i, _vp, _i, _i, _i, _vp, _vp, _i, _i, _i, _ll, _ll,
                        _ll, _vp]),
    "csa_sparse_attn_workspace_size": (_sz, [_i, _i, _i, _i]),
    "csa_sparse_attn": (_i, [_vp, _vp, _vp, _vp, _f, _vp, _vp, _i, _i, _i, _i, _i, _i, _ll, _ll,
                             _ll, _vp, _sz, _vp]),
    "csa_decode_step_workspace_size": (_sz, [ctypes.POINTER(LayerDesc)]),
    "csa_decode_step": (_i, [ctypes.POINTER(LayerDesc), ctypes.POINTER(StepIO), _vp, _sz, _vp]),
    "csa_decode_step_scan": (_i, [ctypes.POINTER(LayerDesc), ctypes.POINTER(StepIO), _vp, _sz, _vp]),
    "csa_decode_step_attend": (_i, [ctypes.POINTER(LayerDesc), ctypes.POINTER(StepIO), _vp, _sz, _vp]),
    "csa_decode_step_noalloc_max_bytes": (_sz, []),
    "csa_decode_step_noalloc": (_i, [ctypes.POINTER(LayerDesc), ctypes.POINTER(StepIO), _vp]),
    "csa_layer_advance": (_i, [ctypes.POINTER(LayerDesc), _i]),
    "csa_decode_step_dev_ring_size": (_sz, [ctypes.POINTER(LayerDesc)]),
    "csa_decode_step_dev": (_i, [ctypes.POINTER(LayerDesc), ctypes.POINTER(StepIO), _vp, _vp, _sz, _vp, _sz, _vp]),
    "csa_hca_decode_step_workspace_size": (_sz, [ctypes.POINTER(LayerDesc)]),
    "csa_hca_decode_step": (_i, [ctypes.POINTER(LayerDesc), ctypes.POINTER(StepIO), _vp, _sz, _vp]),
    "csa_hca_decode_step_dev_ring_size": (_sz, [ctypes.POINTER(LayerDesc)]),
    "csa_hca_decode_step_dev": (_i, [ctypes.POINTER(LayerDesc), ctypes.POINTER(StepIO), _vp, _vp, _sz, _vp, _sz,
                                     _vp]),
    "csa_index_topk_workspace_size": (_sz, [_i, _i, _i]),
    "csa_index_topk": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _ll, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_topk_fp8": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _ll, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_topk_fp8_rescored_workspace_size": (_sz, [_i, _i, _i, _i]),
    "csa_index_topk_fp4": (_i, [_vp, _vp, _vp, _vp, _i, _i, _i, _i, _ll, _i, _i, _vp, _vp, _vp, _sz, _vp]),
    "csa_index_topk_fp4_rescored": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _ll, _i, _i, _i, _vp, _vp, _vp, _sz,
                                         _vp]),
    "csa_index_topk_fp8_rescored": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _ll, _i, _i, _i, _vp, _vp, _vp, _sz,
                                         _vp]),
    "csa_prefill_attn": (_i, [_vp, _vp, _i, _vp, _vp, _i, _vp, _i, _ll, _vp, _f, _vp, _i, _vp, _i, _i, _i,
                              _vp]),
    "csa_prefill_attn_mixed": (_i, [_vp, _vp, _i, _vp, _vp, _i, _vp, _i, _ll, _vp, _vp, _i, _vp, _f, _vp, _i,
                                    _vp, _i, _i, _vp]),
}

_lib = None


_CALIB_SIGS = {
    "csa_read_probe": (_i, [_vp, _ll, _vp, _vp]),
    "csa_mfma_probe": (_i, [_vp, _i, _i, _i, _vp]),
    "csa_probe_workgroups": (_i, []),
    "csa_queue_probe": (_i, [_vp, _vp, _ll, _i, _vp, _ll, _vp, _vp]),
    "csa_handoff_probe": (_i, [_vp, _ll, _vp, _vp, _i, _i, _vp]),
}
CALIB_LIB_PATH = os.path.join(_PKG, "libcsa_calib.so")
_calib = None


def calib_lib() -> ctypes.CDLL:
    """The calibration probes' library (include/csa_calib.h), loaded on first use."""
    global _calib
    if _calib is None:
        if not os.path.exists(CALIB_LIB_PATH):
            raise RuntimeError(f"{CALIB_LIB_PATH} is missing: build it first (python -c "
                               "'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(CALIB_LIB_PATH)
        for name, (res, args) in _CALIB_SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _calib = L
    return _calib


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -c "
                               "'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != CSA_OK:
        raise CsaError(rc, lib().csa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def _inner_contig(t: torch.Tensor, name: str) -> None:
    # every dim but the batch dim must be dense row-major
    exp = 1
    for size, st in zip(reversed(t.shape[1:]), reversed(t.stride()[1:])):
        if size != 1 and st != exp:
            raise ValueError(f"{name}: inner dims must be contiguous (stride {t.stride()})")
        exp *= size


def csa_last_error() -> str:
    return lib().csa_last_error().decode()


def csa_compress(z, c, bias, out, m: int, overlap: int = 0, first_block: int = 0, norm_w=None,
                 n_blocks: Optional[int] = None, stream=None) -> None:
    """z, c: [B, rows, d or 2d] float32; bias [m, d or 2d]; out [B, n_blocks, d]."""
    for t, nm in ((z, "z"), (c, "c"), (out, "out")):
        _inner_contig(t, nm)
    B, nb, d = out.shape
    nb = nb if n_blocks is None else n_blocks
    _check(lib().csa_compress(_ptr(z), _ptr(c), _ptr(bias), _ptr(norm_w), _ptr(out), _dt(out), B, nb,
                              m, d, overlap, first_block, z.stride(0), out.stride(0), _stream(stream)))


def csa_index_score(q, w, k, scores, q_pos=None, ratio: int = 4, n: Optional[int] = None,
                    stream=None) -> None:
    """q [B, t, h_i, d_i]; w [B, t, h_i] float32; k [B, N, d_i]; scores [B, t, ld] float32."""
    for t_, nm in ((q, "q"), (w, "w"), (k, "k"), (scores, "scores")):
        _inner_contig(t_, nm)
    B, t, h_i, d_i = q.shape
    n = k.shape[1] if n is None else n
    _check(lib().csa_index_score(_ptr(q), _ptr(w), _ptr(k), _ptr(scores), _dt(q), B, t, h_i, d_i, n,
                                 _ptr(q_pos), ratio, q.stride(0), w.stride(0),
                                 k.stride(0) if k.shape[0] > 1 else 0, scores.stride(0),
                                 scores.shape[2], _stream(stream)))


def csa_quantize_fp8(x, codes, scales, stream=None) -> None:
    """x [..., d] float32 / bfloat16 (contiguous) -> codes [..., d] uint8, scales [...] float32."""
    for t_, nm in ((x, "x"), (codes, "codes"), (scales, "scales")):
        if not t_.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if codes.dtype != torch.uint8 or scales.dtype != torch.float32:
        raise TypeError("codes must be uint8 and scales float32")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if codes.shape != x.shape or scales.numel() != rows:
        raise ValueError("codes must match x and scales hold one value per row")
    _check(lib().csa_quantize_fp8(_ptr(x), _dt(x), _ptr(codes), _ptr(scales), rows, d, _stream(stream)))


def csa_quantize_fp4(x, codes, scales, stream=None) -> None:
    """x [..., d] float32 / bfloat16 (contiguous, d a multiple of 32) -> codes
    [..., d / 2] uint8 packed E2M1 (element 2j in the low nibble of byte j),
    scales [..., d / 32] uint8 E8M0."""
    for t_, nm in ((x, "x"), (codes, "codes"), (scales, "scales")):
        if not t_.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8:
        raise TypeError("codes and scales must be uint8")
    d = x.shape[-1]
    rows = x.numel() // d if d else 0
    if codes.shape != (*x.shape[:-1], d // 2) or scales.shape != (*x.shape[:-1], d // 32):
        raise ValueError("codes must be x's shape with d / 2, scales with d / 32")
    _check(lib().csa_quantize_fp4(_ptr(x), _dt(x), _ptr(codes), _ptr(scales), rows, d, _stream(stream)))


def csa_quantize_query_fp8(q, w, q_codes, w_folded, stream=None) -> None:
    """q [..., h, d] float32 / bfloat16 and w [..., h] float32 (contiguous) ->
    q_codes [..., h, d] uint8 E4M3 and w_folded [..., h] float32 (w times each
    head row's scale)."""
    for t_, nm in ((q, "q"), (w, "w"), (q_codes, "q_codes"), (w_folded, "w_folded")):
        if not t_.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if q_codes.dtype != torch.uint8 or w.dtype != torch.float32 or w_folded.dtype != torch.float32:
        raise TypeError("q_codes must be uint8, w and w_folded float32")
    h, d = q.shape[-2], q.shape[-1]
    rows = q.numel() // (h * d) if h * d else 0
    if q_codes.shape != q.shape or w.shape != q.shape[:-1] or w_folded.shape != w.shape:
        raise ValueError("q_codes must match q, w and w_folded be q's shape without d")
    _check(lib().csa_quantize_query_fp8(_ptr(q), _dt(q), _ptr(w), _ptr(q_codes), _ptr(w_folded), rows, h, d,
                                        _stream(stream)))


def _check_calib(rc: int, name: str) -> None:
    if rc != CSA_OK:
        raise CsaError(rc, f"{name}: bad arguments or launch failure")


def csa_mfma_probe(sink, waves_per_simd: int, iters: int, valu_per_mfma: int, stream=None) -> None:
    """Matrix-core issue ceiling (libcsa_calib.so; not a step of the method)."""
    _check_calib(calib_lib().csa_mfma_probe(_ptr(sink), int(waves_per_simd), int(iters), int(valu_per_mfma),
                                            _stream(stream)), "csa_mfma_probe")


def csa_read_probe(buf, sink, stream=None) -> None:
    """Read every byte of the contiguous device tensor buf once (libcsa_calib.so; calibration)."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    _check_calib(calib_lib().csa_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                            _stream(stream)), "csa_read_probe")


def csa_probe_workgroups() -> int:
    return int(calib_lib().csa_probe_workgroups())


def csa_queue_probe(row, buf, tiles: int, stamps, sink, stream=None) -> None:
    """Shared-row arrival behind every workgroup's own loads (libcsa_calib.so;
    calibration): row 16 KB, buf the workgroups' slices (or None for tiles 0),
    stamps int64 [csa_probe_workgroups(), 4]."""
    nbytes = buf.numel() * buf.element_size() if buf is not None else 0
    _check_calib(calib_lib().csa_queue_probe(_ptr(row), _ptr(buf), nbytes, int(tiles), _ptr(stamps), stamps.numel(),
                                             _ptr(sink), _stream(stream)), "csa_queue_probe")


def csa_handoff_probe(data, counter, out, wgs: int, handoff: bool, stream=None) -> None:
    """Workgroup results handed to the last workgroup inside one launch, or
    not (libcsa_calib.so; calibration): data float32 [>= 256 wgs], counter
    int32 [1] (zero before the first launch), out float32 [256]."""
    _check_calib(calib_lib().csa_handoff_probe(_ptr(data), data.numel(), _ptr(counter), _ptr(out), int(wgs),
                                               1 if handoff else 0, _stream(stream)), "csa_handoff_probe")


MIX_REC_BYTES = 592  # one mixed main-KV row: 448 E4M3 codes, 64 bf16 RoPE values, scale, pad


def csa_pack_kv_mixed(x, rec, stream=None) -> None:
    """x [..., 512] float32 / bfloat16 (contiguous) -> rec [..., 592] uint8 mixed records."""
    for t_, nm in ((x, "x"), (rec, "rec")):
        if not t_.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if rec.dtype != torch.uint8 or rec.shape[:-1] != x.shape[:-1] or rec.shape[-1] != MIX_REC_BYTES:
        raise ValueError("rec must be uint8 [..., 592] matching x's rows")
    rows = x.numel() // x.shape[-1]
    _check(lib().csa_pack_kv_mixed(_ptr(x), _dt(x), _ptr(rec), rows, x.shape[-1], 64, _stream(stream)))


def csa_index_score_fp8(q, w, k, k_scale, scores, q_pos=None, ratio: int = 4, n: Optional[int] = None,
                        stream=None) -> None:
    """q [B, t, 64, 128] uint8 E4M3; w [B, t, 64] float32 (query scales folded in);
    k [B, N, 128] uint8 E4M3; k_scale [B, N] float32; scores [B, t, ld] float32."""
    for t_, nm in ((q, "q"), (w, "w"), (k, "k"), (k_scale, "k_scale"), (scores, "scores")):
        _inner_contig(t_, nm)
    if q.dtype != torch.uint8 or k.dtype != torch.uint8:
        raise TypeError("q and k must hold uint8 E4M3 codes")
    B, t, h_i, d_i = q.shape
    n = k.shape[1] if n is None else n
    _check(lib().csa_index_score_fp8(_ptr(q), _ptr(w), _ptr(k), _ptr(k_scale), _ptr(scores), B, t, h_i, d_i,
                                     n, _ptr(q_pos), ratio, q.stride(0), w.stride(0),
                                     k.stride(0) if k.shape[0] > 1 else 0,
                                     k_scale.stride(0) if k_scale.shape[0] > 1 else 0, scores.stride(0),
                                     scores.shape[2], _stream(stream)))


def csa_topk_workspace_size(batch: int, t: int, n: int, k: int) -> int:
    return int(lib().csa_topk_workspace_size(batch, t, n, k))


def csa_topk(scores, k: int, idx, count, ws, n: Optional[int] = None, stream=None) -> None:
    """scores [B, t, ld] float32 (first n columns); idx [B, t, k] int32; count [B, t] int32."""
    _inner_contig(scores, "scores")
    B, t, ld = scores.shape
    n = ld if n is None else n
    _check(lib().csa_topk(_ptr(scores), B, t, n, ld, scores.stride(0), k, _ptr(idx), _ptr(count),
                          _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def csa_gather(comp_kv, idx, count, swa, swa_head: int, swa_len: int, gather_buf, n_valid,
               n_comp: Optional[int] = None, stream=None) -> None:
    """comp_kv [B, >=n_comp, d]; idx [B, k]; count [B]; swa [B, W, d]; gather_buf [B, k+W, d]."""
    for t_, nm in ((comp_kv, "comp_kv"), (swa, "swa"), (gather_buf, "gather_buf")):
        _inner_contig(t_, nm)
    B, _, d = gather_buf.shape
    k = idx.shape[1]
    W = swa.shape[1]
    n_comp = comp_kv.shape[1] if n_comp is None else n_comp
    _check(lib().csa_gather(_ptr(comp_kv), n_comp, _ptr(idx), _ptr(count), k, _ptr(swa), swa_head,
                            swa_len, W, _ptr(gather_buf), _ptr(n_valid), _dt(gather_buf), B, d,
                            comp_kv.stride(0), swa.stride(0), gather_buf.stride(0), _stream(stream)))


def csa_sparse_attn_workspace_size(batch: int, h: int, d: int, n_max: int) -> int:
    return int(lib().csa_sparse_attn_workspace_size(batch, h, d, n_max))


def csa_sparse_attn(q, kv, n_valid, sink, scale: float, out, lse=None, ws=None, stream=None) -> None:
    """q [B, h, d]; kv [B, n_max, d]; n_valid [B] int32; sink [h] or None; out [B, h, d]."""
    for t_, nm in ((q, "q"), (kv, "kv"), (out, "out")):
        _inner_contig(t_, nm)
    B, h, d = q.shape
    n_max = kv.shape[1]
    wsb = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().csa_sparse_attn(_ptr(q), _ptr(kv), _ptr(n_valid), _ptr(sink), scale, _ptr(out),
                                 _ptr(lse), _dt(q), _dt(out), B, h, d, n_max, q.stride(0),
                                 kv.stride(0), out.stride(0), _ptr(ws), wsb, _stream(stream)))


def csa_decode_step_workspace_size(layer: LayerDesc) -> int:
    return int(lib().csa_decode_step_workspace_size(ctypes.byref(layer)))


def csa_decode_step(layer: LayerDesc, io: StepIO, ws, stream=None) -> None:
    _check(lib().csa_decode_step(ctypes.byref(layer), ctypes.byref(io), _ptr(ws),
                                 ws.numel() * ws.element_size(), _stream(stream)))


def csa_decode_step_scan(layer: LayerDesc, io: StepIO, ws, stream=None) -> None:
    """The first part of csa_decode_step (jobs + scan with candidates)."""
    _check(lib().csa_decode_step_scan(ctypes.byref(layer), ctypes.byref(io), _ptr(ws),
                                      ws.numel() * ws.element_size(), _stream(stream)))


def csa_decode_step_attend(layer: LayerDesc, io: StepIO, ws, stream=None) -> None:
    """The rest of csa_decode_step (top-k, gather, attention), after csa_decode_step_scan."""
    _check(lib().csa_decode_step_attend(ctypes.byref(layer), ctypes.byref(io), _ptr(ws),
                                        ws.numel() * ws.element_size(), _stream(stream)))


def csa_decode_step_noalloc_max_bytes() -> int:
    return int(lib().csa_decode_step_noalloc_max_bytes())


def csa_decode_step_noalloc(layer: LayerDesc, io: StepIO, stream=None) -> None:
    """csa_decode_step with the library's own fixed scratch (no workspace)."""
    _check(lib().csa_decode_step_noalloc(ctypes.byref(layer), ctypes.byref(io), _stream(stream)))


def csa_decode_step_dev_ring_size(layer: LayerDesc) -> int:
    return lib().csa_decode_step_dev_ring_size(ctypes.byref(layer))


def csa_decode_step_dev(layer: LayerDesc, io: StepIO, state, ring, ws, stream=None) -> None:
    """state: int32 [5] device tensor (pos, n_comp, swa_head, swa_len, flags);
    ring: float32 device tensor of csa_decode_step_dev_ring_size(layer) bytes."""
    if state.dtype != torch.int32 or state.numel() < 5:
        raise ValueError("state must be int32 [5]")
    _check(lib().csa_decode_step_dev(ctypes.byref(layer), ctypes.byref(io), _ptr(state), _ptr(ring),
                                     ring.numel() * ring.element_size(), _ptr(ws), ws.numel() * ws.element_size(),
                                     _stream(stream)))


def csa_hca_decode_step_workspace_size(layer: LayerDesc) -> int:
    return lib().csa_hca_decode_step_workspace_size(ctypes.byref(layer))


def csa_hca_decode_step(layer: LayerDesc, io: StepIO, ws, stream=None) -> None:
    _check(lib().csa_hca_decode_step(ctypes.byref(layer), ctypes.byref(io), _ptr(ws),
                                     ws.numel() * ws.element_size(), _stream(stream)))


def csa_hca_decode_step_dev_ring_size(layer: LayerDesc) -> int:
    return lib().csa_hca_decode_step_dev_ring_size(ctypes.byref(layer))


def csa_hca_decode_step_dev(layer: LayerDesc, io: StepIO, state, ring, ws, stream=None) -> None:
    """state: int32 [5] device tensor (pos, n_comp, swa_head, swa_len, flags);
    ring: float32 device tensor of csa_hca_decode_step_dev_ring_size(layer) bytes."""
    if state.dtype != torch.int32 or state.numel() < 5:
        raise ValueError("state must be int32 [5]")
    _check(lib().csa_hca_decode_step_dev(ctypes.byref(layer), ctypes.byref(io), _ptr(state), _ptr(ring),
                                         ring.numel() * ring.element_size(), _ptr(ws), ws.numel() * ws.element_size(),
                                         _stream(stream)))


def csa_index_score_fp4(q, w, k, k_scales, scores, q_pos=None, ratio: int = 4, n: Optional[int] = None,
                        stream=None) -> None:
    """q [B, t, 64, 128] uint8 E4M3; w [B, t, 64] float32 (query scales folded in);
    k [B, N, 64] uint8 packed E2M1; k_scales [B, N, 4] uint8 E8M0 (one per 32
    elements); scores [B, t, ld] float32."""
    for t_, nm in ((q, "q"), (w, "w"), (k, "k"), (k_scales, "k_scales"), (scores, "scores")):
        _inner_contig(t_, nm)
    if q.dtype != torch.uint8 or k.dtype != torch.uint8 or k_scales.dtype != torch.uint8:
        raise TypeError("q, k and k_scales must be uint8")
    if k_scales.shape[-1] != 4 or k_scales.stride(0) % 4 != 0:
        raise ValueError("k_scales must be [B, N, 4] with a batch stride of whole words")
    B, t, h_i, d_i = q.shape
    n = k.shape[1] if n is None else n
    _check(lib().csa_index_score_fp4(_ptr(q), _ptr(w), _ptr(k), _ptr(k_scales), _ptr(scores), B, t, h_i, d_i,
                                     n, _ptr(q_pos), ratio, q.stride(0), w.stride(0),
                                     k.stride(0) if k.shape[0] > 1 else 0,
                                     k_scales.stride(0) // 4 if k_scales.shape[0] > 1 else 0, scores.stride(0),
                                     scores.shape[2], _stream(stream)))


def csa_layer_advance(layer: LayerDesc, pos: int) -> None:
    _check(lib().csa_layer_advance(ctypes.byref(layer), pos))


def make_layer_desc(*, comp_kv, idx_keys, swa, main_bias, idx_bias, sink, n_comp: int,
                    swa_head: int, swa_len: int, h: int, h_i: int, m: int = 4, top_k: int,
                    overlap: int = 0, out_dtype=None, scale: Optional[float] = None,
                    main_norm=None, idx_norm=None, idx_scales=None, rope=None, comp_rope=None,
                    idx_keys_exact=None, idx_rescore: int = 0) -> LayerDesc:
    """Fill a LayerDesc from cache tensors: comp_kv [B, max_comp, d], idx_keys
    [B, max_comp, d_i] (None for an HCA layer, with idx_bias None, h_i and
    top_k 0), swa [B, W, d].  idx_keys of torch.uint8 are E4M3 codes, with
    their row scales in idx_scales [B, max_comp] float32, or, with idx_scales
    uint8 [B, max_comp, 4], packed E2M1 codes [B, max_comp, d_i / 2] with
    their E8M0 block scales.  comp_kv and swa of
    torch.uint8 [B, rows, 592] are mixed main-KV records (d = 512), with
    rope = (cos, sin) and comp_rope = (cos, sin) float32 tables
    [rows, 32] of token positions and of block indices.  E4M3 keys with
    idx_rescore = k_cand > 0 also keep idx_keys_exact [B, max_comp, d_i]
    bf16 (the two-stage selection).  The returned struct keeps references to
    every tensor it points at."""
    B, max_comp, d = comp_kv.shape
    mixed = comp_kv.dtype == torch.uint8
    if mixed:
        if d != MIX_REC_BYTES or swa.dtype != torch.uint8 or rope is None or comp_rope is None:
            raise ValueError("mixed KV: comp_kv / swa uint8 [B, rows, 592] and both RoPE tables")
        d = 512
    L = LayerDesc()
    fp4 = idx_keys is not None and idx_keys.dtype == torch.uint8 and idx_scales is not None and \
        idx_scales.dtype == torch.uint8
    L.batch, L.h, L.d, L.h_i = B, h, d, h_i
    L.d_i = (idx_keys.shape[2] * (2 if fp4 else 1)) if idx_keys is not None else 0
    L.m, L.w, L.top_k, L.overlap = m, swa.shape[1], top_k, overlap
    L.dtype = CSA_BF16 if mixed else _dt(comp_kv)
    L.out_dtype = L.dtype if out_dtype is None else (CSA_BF16 if out_dtype == torch.bfloat16 else CSA_F32)
    if mixed:
        L.kv_dtype, L.rope_dim = CSA_FP8_E4M3, 64
        for t_ in (*rope, *comp_rope):
            if t_.dtype != torch.float32 or not t_.is_contiguous() or t_.shape[-1] != 32:
                raise ValueError("RoPE tables must be contiguous float32 [rows, 32]")
        L.rope_cos, L.rope_sin, L.rope_rows = rope[0].data_ptr(), rope[1].data_ptr(), rope[0].shape[0]
        L.comp_rope_cos, L.comp_rope_sin = comp_rope[0].data_ptr(), comp_rope[1].data_ptr()
        L.comp_rope_rows = comp_rope[0].shape[0]
    L.comp_kv, L.comp_kv_stride_b = comp_kv.data_ptr(), comp_kv.stride(0)
    L.idx_keys, L.idx_keys_stride_b = _ptr(idx_keys), (idx_keys.stride(0) if idx_keys is not None else 0)
    L.swa, L.swa_stride_b = swa.data_ptr(), swa.stride(0)
    L.max_comp = max_comp
    L.main_bias, L.idx_bias = main_bias.data_ptr(), _ptr(idx_bias)
    L.main_norm, L.idx_norm = _ptr(main_norm), _ptr(idx_norm)
    L.sink = _ptr(sink)
    L.scale = (1.0 / d ** 0.5) if scale is None else scale
    L.n_comp, L.swa_head, L.swa_len = n_comp, swa_head, swa_len
    if fp4:
        if idx_scales.shape != (B, max_comp, 4) or idx_scales.stride(1) != 4 or idx_scales.stride(2) != 1 or \
                idx_scales.stride(0) % 4 != 0:
            raise ValueError("E2M1 idx_keys need uint8 idx_scales [B, max_comp, 4] with whole-word rows")
        L.idx_dtype = CSA_FP4_E2M1
        L.idx_scales, L.idx_scales_stride_b = idx_scales.data_ptr(), idx_scales.stride(0) // 4
    elif idx_keys is not None and idx_keys.dtype == torch.uint8:
        if idx_scales is None or idx_scales.dtype != torch.float32:
            raise ValueError("E4M3 idx_keys need float32 idx_scales [B, max_comp]")
        L.idx_dtype = CSA_FP8_E4M3
        L.idx_scales, L.idx_scales_stride_b = idx_scales.data_ptr(), idx_scales.stride(0)
    else:
        L.idx_dtype = L.dtype
    if idx_rescore:
        L.idx_rescore = idx_rescore
        L.idx_keys_exact, L.idx_keys_exact_stride_b = _ptr(idx_keys_exact), (
            idx_keys_exact.stride(0) if idx_keys_exact is not None else 0)
    # the struct holds raw device pointers: keep the tensors alive with it
    L._keep = (comp_kv, idx_keys, swa, main_bias, idx_bias, sink, main_norm, idx_norm, idx_scales, rope, comp_rope,
               idx_keys_exact)
    return L


def make_step_io(*, pos: int, q, q_idx=None, w_idx=None, kv_new, z_main, c_main, z_idx=None, c_idx=None,
                 scores=None, topk_idx=None, topk_count=None, gather_buf=None, n_valid=None, out,
                 lse=None) -> StepIO:
    """q [B, h, d]; q_idx [B, h_i, d_i]; w_idx [B, h_i]; kv_new [B, d]; z/c [B, rows, width];
    scores [B, >=N]; topk_idx [B, k]; topk_count [B]; gather_buf [B, k+W, d]; out [B, h, d].
    The indexer fields may be None for an HCA step."""
    def st(t):
        return t.stride(0) if t is not None else 0

    io = StepIO()
    io.pos = pos
    io.q, io.q_stride_b = q.data_ptr(), q.stride(0)
    io.q_idx, io.q_idx_stride_b = _ptr(q_idx), st(q_idx)
    io.w_idx, io.w_stride_b = _ptr(w_idx), st(w_idx)
    io.kv_new, io.kv_new_stride_b = kv_new.data_ptr(), kv_new.stride(0)
    io.z_main, io.c_main, io.zc_main_stride_b = z_main.data_ptr(), c_main.data_ptr(), z_main.stride(0)
    io.z_idx, io.c_idx, io.zc_idx_stride_b = _ptr(z_idx), _ptr(c_idx), st(z_idx)
    io.scores, io.scores_stride_b = _ptr(scores), st(scores)
    io.topk_idx, io.topk_count = _ptr(topk_idx), _ptr(topk_count)
    io.gather_buf, io.gather_stride_b = _ptr(gather_buf), st(gather_buf)
    io.n_valid = _ptr(n_valid)
    io.out, io.out_stride_b = out.data_ptr(), out.stride(0)
    io.lse = _ptr(lse)
    # the struct holds raw device pointers: keep the tensors alive with it
    io._keep = (q, q_idx, w_idx, kv_new, z_main, c_main, z_idx, c_idx, scores, topk_idx, topk_count,
                gather_buf, n_valid, out, lse)
    return io


def csa_index_topk_workspace_size(t: int, n: int, top_k: int) -> int:
    return lib().csa_index_topk_workspace_size(t, n, top_k)


def csa_index_topk(q, w, k, idx, count, ws, pos0: int = -1, ratio: int = 4, n: Optional[int] = None,
                   stream=None) -> None:
    """q [t, 64, 128] bf16; w [t, 64] float32; k [N, 128] bf16 (first n rows);
    idx [t, top_k] int32; count [t] int32 or None; query row r sits at
    position pos0 + r (pos0 < 0: no causal mask)."""
    for t_, nm in ((q, "q"), (w, "w"), (k, "k"), (idx, "idx")):
        if not t_.is_contiguous():
            raise ValueError(f"{nm}: must be contiguous")
    t, h_i, d_i = q.shape
    n = k.shape[0] if n is None else n
    _check(lib().csa_index_topk(_ptr(q), _ptr(w), _ptr(k), t, h_i, d_i, n, pos0, ratio, idx.shape[1], _ptr(idx),
                                _ptr(count), _ptr(ws), ws.numel() * ws.element_size(), _stream(stream)))


def csa_index_topk_fp8(q, w, k, k_scale, idx, count, ws, pos0: int = -1, ratio: int = 4,
                       n: Optional[int] = None, stream=None) -> None:
    """q [t, 64, 128] uint8 E4M3; w [t, 64] float32 (query scales folded in);
    k [N, 128] uint8 E4M3 and k_scale [N] float32 (first n rows); idx, count,
    pos0 as for csa_index_topk."""
    for t_, nm in ((q, "q"), (w, "w"), (k, "k"), (k_scale, "k_scale"), (idx, "idx")):
        if not t_.is_contiguous():
            raise ValueError(f"{nm}: must be contiguous")
    if q.dtype != torch.uint8 or k.dtype != torch.uint8 or k_scale.dtype != torch.float32:
        raise TypeError("q and k must hold uint8 E4M3 codes, k_scale float32")
    t, h_i, d_i = q.shape
    n = k.shape[0] if n is None else n
    _check(lib().csa_index_topk_fp8(_ptr(q), _ptr(w), _ptr(k), _ptr(k_scale), t, h_i, d_i, n, pos0, ratio,
                                    idx.shape[1], _ptr(idx), _ptr(count), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))


def csa_index_topk_fp8_rescored_workspace_size(t: int, n: int, top_k: int, k_cand: int) -> int:
    return lib().csa_index_topk_fp8_rescored_workspace_size(t, n, top_k, k_cand)


def csa_index_topk_fp8_rescored(q, w, k8, k_scale, k16, idx, count, ws, k_cand: int, pos0: int = -1, ratio: int = 4,
                                n: Optional[int] = None, stream=None) -> None:
    """q [t, 64, 128] bf16; w [t, 64] float32 (plain weights); k8 [N, 128]
    uint8 E4M3, k_scale [N] float32 and k16 [N, 128] bf16 (the same keys);
    idx [t, top_k] int32; count [t] int32 or None; pos0 as csa_index_topk."""
    for t_, nm in ((q, "q"), (w, "w"), (k8, "k8"), (k_scale, "k_scale"), (k16, "k16"), (idx, "idx")):
        if not t_.is_contiguous():
            raise ValueError(f"{nm}: must be contiguous")
    if q.dtype != torch.bfloat16 or k16.dtype != torch.bfloat16 or k8.dtype != torch.uint8:
        raise TypeError("q and k16 must be bfloat16, k8 uint8 E4M3 codes")
    t, h_i, d_i = q.shape
    n = k8.shape[0] if n is None else n
    _check(lib().csa_index_topk_fp8_rescored(_ptr(q), _ptr(w), _ptr(k8), _ptr(k_scale), _ptr(k16), t, h_i, d_i, n,
                                             pos0, ratio, idx.shape[1], k_cand, _ptr(idx), _ptr(count), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(stream)))


def _fp4_keys(k, k_scales, nm):
    if not k.is_contiguous() or not k_scales.is_contiguous():
        raise ValueError(f"{nm} and k_scales must be contiguous")
    if k.dtype != torch.uint8 or k_scales.dtype != torch.uint8 or k.shape[-1] != 64 or \
            k_scales.shape != (*k.shape[:-1], 4):
        raise TypeError(f"{nm} must be uint8 [N, 64] packed E2M1, k_scales uint8 [N, 4] E8M0")


def csa_index_topk_fp4(q, w, k, k_scales, idx, count, ws, pos0: int = -1, ratio: int = 4,
                       n: Optional[int] = None, stream=None) -> None:
    """q [t, 64, 128] uint8 E4M3; w [t, 64] float32 (query scales folded in);
    k [N, 64] uint8 packed E2M1 and k_scales [N, 4] uint8 E8M0 (first n
    rows); idx, count, pos0 as for csa_index_topk."""
    for t_, nm in ((q, "q"), (w, "w"), (idx, "idx")):
        if not t_.is_contiguous():
            raise ValueError(f"{nm}: must be contiguous")
    _fp4_keys(k, k_scales, "k")
    if q.dtype != torch.uint8:
        raise TypeError("q must hold uint8 E4M3 codes")
    t, h_i, d_i = q.shape
    n = k.shape[0] if n is None else n
    _check(lib().csa_index_topk_fp4(_ptr(q), _ptr(w), _ptr(k), _ptr(k_scales), t, h_i, d_i, n, pos0, ratio,
                                    idx.shape[1], _ptr(idx), _ptr(count), _ptr(ws), ws.numel() * ws.element_size(),
                                    _stream(stream)))


def csa_index_topk_fp4_rescored(q, w, k4, k_scales, k16, idx, count, ws, k_cand: int, pos0: int = -1,
                                ratio: int = 4, n: Optional[int] = None, stream=None) -> None:
    """q [t, 64, 128] bf16; w [t, 64] float32 (plain weights); k4 [N, 64]
    uint8 packed E2M1, k_scales [N, 4] uint8 E8M0 and k16 [N, 128] bf16 (the
    same keys); idx [t, top_k] int32; count [t] int32 or None; ws of
    csa_index_topk_fp8_rescored_workspace_size bytes."""
    for t_, nm in ((q, "q"), (w, "w"), (k16, "k16"), (idx, "idx")):
        if not t_.is_contiguous():
            raise ValueError(f"{nm}: must be contiguous")
    _fp4_keys(k4, k_scales, "k4")
    if q.dtype != torch.bfloat16 or k16.dtype != torch.bfloat16:
        raise TypeError("q and k16 must be bfloat16")
    t, h_i, d_i = q.shape
    n = k4.shape[0] if n is None else n
    _check(lib().csa_index_topk_fp4_rescored(_ptr(q), _ptr(w), _ptr(k4), _ptr(k_scales), _ptr(k16), t, h_i, d_i, n,
                                             pos0, ratio, idx.shape[1], k_cand, _ptr(idx), _ptr(count), _ptr(ws),
                                             ws.numel() * ws.element_size(), _stream(stream)))


def csa_prefill_attn(q, comp_kv, idx, count, win_kv, window: int, pos0: int, sink, scale: float, out,
                     lse=None, n_comp: Optional[int] = None, stream=None) -> None:
    """q [t, h, d] bf16; comp_kv [N, d] bf16; idx [t, k] int32; count [t] int32
    or None; win_kv [t + window - 1, d] bf16 (row i = position
    pos0 - window + 1 + i); sink [h] float32 or None; out [t, h, d] float32
    or bf16; lse [t, h] float32 or None."""
    for t_, nm in ((q, "q"), (comp_kv, "comp_kv"), (idx, "idx"), (win_kv, "win_kv"), (out, "out")):
        if not t_.is_contiguous():
            raise ValueError(f"{nm}: must be contiguous")
    t, h, d = q.shape
    n_comp = comp_kv.shape[0] if n_comp is None else n_comp
    _check(lib().csa_prefill_attn(_ptr(q), _ptr(comp_kv), n_comp, _ptr(idx), _ptr(count), idx.shape[1],
                                  _ptr(win_kv), window, pos0, _ptr(sink), scale, _ptr(out), _dt(out), _ptr(lse),
                                  t, h, d, _stream(stream)))


def csa_prefill_attn_mixed(q, comp_rec, idx, count, win_rec, window: int, pos0: int, rope, sink, scale: float, out,
                           lse=None, n_comp: Optional[int] = None, stream=None) -> None:
    """csa_prefill_attn over mixed main-KV records: q [t, h, 512] bf16;
    comp_rec [N, 592] and win_rec [t + window - 1, 592] uint8 records;
    rope = (cos, sin) float32 [rows, 32] tables (out's RoPE dims rotated back
    at each query's position); the rest as csa_prefill_attn."""
    for t_, nm in ((q, "q"), (comp_rec, "comp_rec"), (idx, "idx"), (win_rec, "win_rec"), (out, "out")):
        if not t_.is_contiguous():
            raise ValueError(f"{nm}: must be contiguous")
    cos, sin = rope
    if cos.shape != sin.shape or cos.dim() != 2 or not (cos.is_contiguous() and sin.is_contiguous()):
        raise ValueError("rope: two contiguous [rows, 32] tables")
    t, h, _ = q.shape
    n_comp = comp_rec.shape[0] if n_comp is None else n_comp
    _check(lib().csa_prefill_attn_mixed(_ptr(q), _ptr(comp_rec), n_comp, _ptr(idx), _ptr(count), idx.shape[1],
                                        _ptr(win_rec), window, pos0, _ptr(cos), _ptr(sin), cos.shape[0], _ptr(sink),
                                        scale, _ptr(out), _dt(out), _ptr(lse), t, h, _stream(stream)))
