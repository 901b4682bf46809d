"""Benchmark: CSA decode steps/s at 1M context (n_comp 250,000) on one MI355X.

One step = one new token through 30 independent CSA layers (each with its own
seeded 64 MB indexer-key cache and 256 MB compressed-KV cache), i.e. 30 calls
of csa_decode_step on one stream: SWA append, compression of the block the
token completes, indexer scan over 250,000 keys, top-512, gather of 640 rows,
attention of 64 heads x 512 with a sink.  The 30-layer step is captured once
in a HIP graph and replayed; every replay redoes all the work (same token
position, so each replay rewrites the same cache slots with the same values).

Prints one JSON line.  `roofline` is for the dominant kernel (the indexer
scan), timed with HIP events on its launch stream; `cpu_baseline` is the
float64 CPU oracle timed on the host over a bounded sample of the same step.
"""

from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, TFLOP/s
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 matrix peak, TFLOP/s


def algorithmic_bytes(shape) -> dict:
    """Bytes each step of one layer must move at minimum (bf16 caches)."""
    N, di, hi, D, H, K, W, m = (shape.n_comp, shape.d_i, shape.h_i, shape.d, shape.h, shape.top_k,
                                shape.w, shape.m)
    scan = N * di * 2 + hi * di * 2 + hi * 4            # keys + q_idx + head weights
    topk = K * 4 + 4                                    # indices + count
    gather = 2 * (K + W) * D * 2                        # read + write rows
    attn = (K + W) * D * 2 + H * D * 2 + H * 4 + H * D * 2 + H * 4  # rows, q, sink, out, lse
    compress = (2 * m * D * 4 + m * D * 4 + D * 2) + (2 * m * di * 4 + m * di * 4 + di * 2)
    swa = 2 * D * 2
    per_layer = scan + topk + gather + attn + compress + swa
    # the standalone scan launch (csa_index_score) also writes its fp32 scores:
    # its own output, though materialising them is no part of the step's minimum
    scan_launch = scan + N * 4
    return {"scan": scan, "topk": topk, "gather": gather, "attn": attn, "compress": compress,
            "swa": swa, "per_layer": per_layer, "scan_launch": scan_launch}


def build_layers(csa, shape, dev):
    import torch
    import synth

    layers = []
    for x in synth.make_decode_inputs_torch(shape, seed=None, device=dev):
        B, K, W, D = shape.batch, shape.top_k, shape.w, shape.d
        L = csa.make_layer_desc(comp_kv=x["comp_kv"], idx_keys=x["idx_keys"], swa=x["swa"],
                                main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"],
                                n_comp=x["n_comp"], swa_head=x["swa_head"], swa_len=x["swa_len"],
                                h=shape.h, h_i=shape.h_i, m=shape.m, top_k=K)
        outs = dict(scores=torch.empty(B, shape.max_comp, device=dev),
                    topk_idx=torch.empty(B, K, dtype=torch.int32, device=dev),
                    topk_count=torch.empty(B, dtype=torch.int32, device=dev),
                    gather_buf=torch.zeros(B, K + W, D, dtype=torch.bfloat16, device=dev),
                    n_valid=torch.empty(B, dtype=torch.int32, device=dev),
                    out=torch.empty(B, shape.h, D, dtype=torch.bfloat16, device=dev),
                    lse=torch.empty(B, shape.h, device=dev))
        io = csa.make_step_io(pos=x["pos"], q=x["q"], q_idx=x["q_idx"], w_idx=x["w_idx"],
                              kv_new=x["kv_new"], z_main=x["z_main"], c_main=x["c_main"],
                              z_idx=x["z_idx"], c_idx=x["c_idx"], **outs)
        ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=dev)
        layers.append({"x": x, "L": L, "io": io, "outs": outs, "ws": ws})
    return layers


def run_step(csa, layers):
    for ly in layers:
        csa.csa_decode_step(ly["L"], ly["io"], ly["ws"])


def time_scan_kernel(csa, layers, shape, reps: int):
    """Average duration of one indexer-scan launch (csa_index_score, the
    kernel k_index_score_bf16): the 30 layers' launches (one per layer's
    cache, so every launch streams its 64 MB from HBM: 30 x 64 MB exceed the
    256 MB last-level cache) captured back to back in a HIP graph, replayed
    `reps` times between two HIP events recorded on the stream the graph runs
    on; the average includes the short gaps between consecutive launches."""
    import torch

    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for ly in layers:
                x, o = ly["x"], ly["outs"]
                csa.csa_index_score(x["q_idx"][:, None], x["w_idx"][:, None], x["idx_keys"],
                                    o["scores"][:, None], n=shape.n_comp, stream=stream)
        g.replay()
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    stream.synchronize()
    n = reps * len(layers)
    return e0.elapsed_time(e1) / n, n


def time_read_ceiling(csa, layers, reps: int):
    """The practical read ceiling of one launch: csa_read_probe (plain
    streaming loads, nothing else) over the same 30 key caches the scan
    reads, back to back in a graph like the scan's launches.  Returns
    (average launch us, bytes per launch)."""
    import torch

    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    bufs = [ly["x"]["idx_keys"] for ly in layers]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for b in bufs:
                csa.csa_read_probe(b, sink, stream=stream)
        g.replay()
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    stream.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * len(bufs)), bufs[0].numel() * bufs[0].element_size()


SCAN_SOURCES = ["index_score.hip", "common.h", "kernels.h", "topk_common.h", "step_prep.h", "compress_impl.h",
                "score_tile.h", "fp8_codec.h", "mixed_kv.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_index_score_bf16_ctx1m_hbm_traffic.md")


def scan_traffic():
    """HBM bytes per scan launch from the committed rocprofv3 counter summary,
    or None when it is missing or was taken on different scan sources."""
    import hashlib

    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = dict(re.findall(r"^\s*(scan_\w+):\s*(\S+)\s*$", text, flags=re.M))
    h = hashlib.sha256()
    for f in SCAN_SOURCES:
        with open(os.path.join(ROOT, "compressed_sparse_attention_reduce_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("scan_kernel_source_sha256") != h.hexdigest():
        return None
    try:
        return int(vals["scan_traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def time_fp8(csa, layers, shape, reps: int, steps: int):
    """The E4M3 indexer-key variant: every layer's bf16 key cache quantised
    once (per-row scales) and the query per head.  Times (a) the FP8 scan
    alone (csa_index_score_fp8, 30 launches captured back to back in a graph,
    like the bf16 scan) and (b) the whole 30-layer decode step with E4M3 keys
    (csa_decode_step, graph-replayed `steps` times).  Returns (average scan
    launch ms, algorithmic bytes per scan launch, ms per step)."""
    import torch

    n = shape.n_comp
    fl = []
    for ly in layers:
        x = ly["x"]
        kc = torch.zeros(1, shape.max_comp, 128, dtype=torch.uint8, device="cuda")
        ks = torch.zeros(1, shape.max_comp, dtype=torch.float32, device="cuda")
        csa.csa_quantize_fp8(x["idx_keys"][:, :n].contiguous(), kc[:, :n], ks[:, :n])
        # the standalone scan takes query codes with the scales folded into w
        # (the library's query quantiser); the decode step quantises the bf16
        # query itself, inside its timed region
        qc = torch.empty(1, 64, 128, dtype=torch.uint8, device="cuda")
        w8 = torch.empty(1, 64, dtype=torch.float32, device="cuda")
        csa.csa_quantize_query_fp8(x["q_idx"].contiguous(), x["w_idx"].contiguous(), qc, w8)
        L = csa.make_layer_desc(comp_kv=x["comp_kv"], idx_keys=kc, idx_scales=ks, swa=x["swa"],
                                main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"],
                                n_comp=x["n_comp"], swa_head=x["swa_head"], swa_len=x["swa_len"],
                                h=shape.h, h_i=shape.h_i, m=shape.m, top_k=shape.top_k)
        io = csa.make_step_io(pos=x["pos"], q=x["q"], q_idx=x["q_idx"], w_idx=x["w_idx"], kv_new=x["kv_new"],
                              z_main=x["z_main"], c_main=x["c_main"], z_idx=x["z_idx"], c_idx=x["c_idx"],
                              **ly["outs"])
        fl.append({"L": L, "io": io, "ws": ly["ws"], "qc": qc, "w8": w8, "kc": kc, "ks": ks, "outs": ly["outs"]})
    torch.cuda.synchronize()

    def timed(body, count):
        stream = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                body(stream)
            g.replay()
            stream.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(count):
                g.replay()
            e1.record(stream)
        stream.synchronize()
        return e0.elapsed_time(e1) / count

    def scans(stream):
        for f in fl:
            csa.csa_index_score_fp8(f["qc"][:, None], f["w8"][:, None], f["kc"], f["ks"],
                                    f["outs"]["scores"][:, None], n=n, stream=stream)

    def step(stream):
        for f in fl:
            csa.csa_decode_step(f["L"], f["io"], f["ws"], stream=stream)

    scan_ms = timed(scans, reps) / len(fl)
    step_ms = timed(step, steps)
    alg = n * 128 + n * 4 + 64 * 128 + 64 * 4 + n * 4  # keys + key scales + q + w read, scores written
    del fl
    return scan_ms, alg, step_ms


def time_mixed_kv(csa, layers, shape, steps: int):
    """The 30-layer decode step over mixed main KV (E4M3 NoPE codes + bf16
    RoPE part per 592-byte record, RoPE on the new compressed entry, inverse
    RoPE on the output): every layer's bf16 caches packed once with
    csa_pack_kv_mixed, the step graph-captured and replayed `steps` times.
    Returns ms per step."""
    import numpy as np
    import torch

    def tables(rows, offset, base):
        ang = (np.arange(rows)[:, None] + offset) * base ** (-2.0 * np.arange(32)[None, :] / 64)
        return (torch.from_numpy(np.cos(ang).astype(np.float32)).cuda(),
                torch.from_numpy(np.sin(ang).astype(np.float32)).cuda())

    rope = tables(shape.ctx + 8, 0.5, 10000.0)
    comp_rope = tables(shape.max_comp + 1, 0.25, 500.0)
    B, K, W = shape.batch, shape.top_k, shape.w
    ml = []
    for ly in layers:
        x = ly["x"]
        comp = torch.empty(B, shape.max_comp, csa.MIX_REC_BYTES, dtype=torch.uint8, device="cuda")
        swa = torch.empty(B, W, csa.MIX_REC_BYTES, dtype=torch.uint8, device="cuda")
        csa.csa_pack_kv_mixed(x["comp_kv"], comp)
        csa.csa_pack_kv_mixed(x["swa"], swa)
        L = csa.make_layer_desc(comp_kv=comp, idx_keys=x["idx_keys"], swa=swa, main_bias=x["main_bias"],
                                idx_bias=x["idx_bias"], sink=x["sink"], n_comp=x["n_comp"],
                                swa_head=x["swa_head"], swa_len=x["swa_len"], h=shape.h, h_i=shape.h_i,
                                m=shape.m, top_k=K, rope=rope, comp_rope=comp_rope)
        outs = dict(ly["outs"])
        outs["gather_buf"] = torch.zeros(B, K + W, csa.MIX_REC_BYTES, dtype=torch.uint8, device="cuda")
        io = csa.make_step_io(pos=x["pos"], q=x["q"], q_idx=x["q_idx"], w_idx=x["w_idx"], kv_new=x["kv_new"],
                              z_main=x["z_main"], c_main=x["c_main"], z_idx=x["z_idx"], c_idx=x["c_idx"], **outs)
        ml.append((L, io, ly["ws"]))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for L, io, ws in ml:
                csa.csa_decode_step(L, io, ws, stream=stream)
        g.replay()
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
    stream.synchronize()
    del ml, g
    return e0.elapsed_time(e1) / steps


def time_dev_step(csa, layers, shape, steps: int, warmup: int):
    """The 30-layer decode step with device-side counters
    (csa_decode_step_dev): one graph captured once and replayed, each replay
    a real next step (positions advance on the device, every fourth one
    completes a block into the cache).  The counters start `replays / 4 + 1`
    entries below the cache's capacity so that no completion finds it full.
    Returns ms per step."""
    import torch

    total = warmup + steps
    B = shape.batch
    dl = []
    for ly in layers:
        x = ly["x"]
        L = csa.make_layer_desc(comp_kv=x["comp_kv"], idx_keys=x["idx_keys"], swa=x["swa"],
                                main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"],
                                n_comp=x["n_comp"], swa_head=x["swa_head"], swa_len=x["swa_len"],
                                h=shape.h, h_i=shape.h_i, m=shape.m, top_k=shape.top_k)
        rows = {k: x[k][:, 0].contiguous() for k in ("z_main", "c_main", "z_idx", "c_idx")}
        io = csa.make_step_io(pos=0, q=x["q"], q_idx=x["q_idx"], w_idx=x["w_idx"], kv_new=x["kv_new"], **rows,
                              **ly["outs"])
        start = x["pos"] - shape.m + 1  # a block's first token
        state = torch.tensor([start, shape.n_comp - total // shape.m - 2, x["swa_head"], x["swa_len"], 0],
                             dtype=torch.int32, device="cuda")
        ring = torch.zeros(csa.csa_decode_step_dev_ring_size(L) // 4, device="cuda")
        dl.append((L, io, state, ring, ly["ws"]))
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for L, io, state, ring, ws in dl:
                csa.csa_decode_step_dev(L, io, state, ring, ws, stream=stream)
        for _ in range(warmup):
            g.replay()
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            g.replay()
        e1.record(stream)
    stream.synchronize()
    flags = sum(int(st[4]) for _, _, st, _, _ in dl)
    assert flags == 0, "a completed block found its cache full"
    del dl, g
    return e0.elapsed_time(e1) / steps


def time_prefill(csa, reps: int):
    """The prefill-shaped chunk (2048 queries at positions 260096..262143
    against 65536 compressed blocks, causal): csa_index_topk (multi-query
    MFMA score in chunks of 256 queries + per-query top-512) and
    csa_prefill_attn (64 heads x 512, 512 selected rows + the 128-token
    window per query), each timed with HIP events over `reps` calls; plus the
    score kernel alone on the chunk shape (8 launches of 256 queries captured
    in a graph) for its matrix-core rate."""
    import numpy as np
    import torch
    import synth

    shape = synth.SHAPES["prefill"]
    x = synth.make_prefill_inputs_torch(shape, None, "cuda")
    T, N, k, W = shape.t, shape.n_comp, shape.top_k, shape.w
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    cnt = torch.empty(T, dtype=torch.int32, device="cuda")
    ws = torch.empty(csa.csa_index_topk_workspace_size(T, N, k), dtype=torch.uint8, device="cuda")
    out = torch.empty(T, shape.h, shape.d, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(T, shape.h, device="cuda")
    scale = 1.0 / np.sqrt(shape.d)

    def topk():
        csa.csa_index_topk(x["q_idx"], x["w_idx"], x["idx_keys"], idx, cnt, ws, pos0=x["pos0"])

    def attn():
        csa.csa_prefill_attn(x["q"], x["comp_kv"], idx, cnt, x["win_kv"], W, x["pos0"], x["sink"], scale, out,
                             lse=lse)

    def timed(f, n):
        f()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            f()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    topk_ms = timed(topk, reps)
    attn_ms = timed(attn, reps)
    # the attention over mixed main-KV records (packed once, outside the timed region)
    comp_rec = torch.empty(N, csa.MIX_REC_BYTES, dtype=torch.uint8, device="cuda")
    win_rec = torch.empty(x["win_kv"].shape[0], csa.MIX_REC_BYTES, dtype=torch.uint8, device="cuda")
    csa.csa_pack_kv_mixed(x["comp_kv"], comp_rec)
    csa.csa_pack_kv_mixed(x["win_kv"], win_rec)
    ang = (np.arange(x["pos0"] + T)[:, None] + 0.5) * 10000.0 ** (-2.0 * np.arange(32)[None, :] / 64)
    rope = (torch.from_numpy(np.cos(ang).astype(np.float32)).cuda(),
            torch.from_numpy(np.sin(ang).astype(np.float32)).cuda())

    def attn_mixed():
        csa.csa_prefill_attn_mixed(x["q"], comp_rec, idx, cnt, win_rec, W, x["pos0"], rope, x["sink"], scale, out,
                                   lse=lse)

    attn_mixed_ms = timed(attn_mixed, reps)
    del comp_rec, win_rec, rope
    # the score kernel alone: the chunks' launches back to back in a graph
    rows = 256
    sc = torch.empty(1, rows, N, device="cuda")
    pos = torch.arange(x["pos0"], x["pos0"] + T, dtype=torch.int32, device="cuda")[None]
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for r0 in range(0, T, rows):
                csa.csa_index_score(x["q_idx"][None, r0:r0 + rows], x["w_idx"][None, r0:r0 + rows],
                                    x["idx_keys"][None], sc, q_pos=pos[:, r0:r0 + rows], stream=stream)
        g.replay()
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    stream.synchronize()
    launches = reps * (T // rows)
    score_us = e0.elapsed_time(e1) * 1e3 / launches
    flop = 2.0 * rows * 64 * 128 * N
    tflops = flop / (score_us * 1e-6) / 1e12
    attn_flop = 4.0 * T * shape.h * (k + W) * shape.d

    # the E4M3-key variant: keys and queries quantised once (per key row, per
    # query head row; the query scales folded into w), outside the timed region
    kc = torch.empty(N, 128, dtype=torch.uint8, device="cuda")
    ks = torch.empty(N, dtype=torch.float32, device="cuda")
    csa.csa_quantize_fp8(x["idx_keys"], kc, ks)
    qc = torch.empty(T, 64, 128, dtype=torch.uint8, device="cuda")
    w8 = torch.empty(T, 64, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    def topk8():  # the chunk's queries quantised (scales folded into w), then score + top-k
        csa.csa_quantize_query_fp8(x["q_idx"], x["w_idx"], qc, w8)
        csa.csa_index_topk_fp8(qc, w8, kc, ks, idx, cnt, ws, pos0=x["pos0"])

    topk8_ms = timed(topk8, reps)
    g8 = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g8, stream=stream):
            for r0 in range(0, T, rows):
                csa.csa_index_score_fp8(qc[None, r0:r0 + rows], w8[None, r0:r0 + rows], kc[None], ks[None], sc,
                                        q_pos=pos[:, r0:r0 + rows], stream=stream)
        g8.replay()
        stream.synchronize()
        e0.record(stream)
        for _ in range(reps):
            g8.replay()
        e1.record(stream)
    stream.synchronize()
    score8_us = e0.elapsed_time(e1) * 1e3 / launches
    tflops8 = flop / (score8_us * 1e-6) / 1e12
    return {
        "workload": "prefill chunk: 2048 queries at positions 260096..262143 against 65536 compressed "
                    "blocks (causal), indexer 64x128 bf16, top_k 512, main attention 64 heads x 512 bf16 "
                    "over 512 selected rows + the 128-token window per query",
        "index_topk_ms": round(topk_ms, 4),
        "attn_ms": round(attn_ms, 4),
        "chunk_ms": round(topk_ms + attn_ms, 4),
        "queries_per_s": round(T / ((topk_ms + attn_ms) * 1e-3), 1),
        "score_kernel": {
            "kernel": "k_index_score_mq",
            "bound": "mfma",
            "rows_per_launch": rows,
            "avg_launch_us": round(score_us, 2),
            "achieved": round(tflops, 1),
            "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
        },
        "attn_tflops": round(attn_flop / (attn_ms * 1e-3) / 1e12, 1),
        "mixed_kv_attn_ms": round(attn_mixed_ms, 4),
        "fp8_keys": {
            "index_topk_ms": round(topk8_ms, 4),
            "chunk_ms": round(topk8_ms + attn_ms, 4),
            "queries_per_s": round(T / ((topk8_ms + attn_ms) * 1e-3), 1),
            "score_kernel": {
                "kernel": "k_index_score_mq_fp8",
                "bound": "mfma",
                "rows_per_launch": rows,
                "avg_launch_us": round(score8_us, 2),
                "achieved": round(tflops8, 1),
                "peak": FP8_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s",
                "frac": round(tflops8 / FP8_MFMA_PEAK_TFLOPS, 4),
            },
        },
    }


def time_hca(csa, reps: int):
    """HCA layers at 1M context (ratio 128, 7813 compressed entries after the
    step, window 128, 64 heads x 512): 30 independent layer caches, one
    csa_hca_decode_step each, captured in one graph and replayed `reps`
    times; then the same over mixed main KV (the caches packed once with
    csa_pack_kv_mixed).  Returns the mean per-layer times and their
    algorithmic bytes."""
    import numpy as np
    import torch
    import synth

    shape = synth.SHAPES["hca1m"]
    xs = synth.make_decode_inputs_torch(shape, seed=None, device="cuda")

    def replay(steps):
        stream = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            with torch.cuda.graph(g, stream=stream):
                for L, io, ws in steps:
                    csa.csa_hca_decode_step(L, io, ws, stream=stream)
            g.replay()
            stream.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                g.replay()
            e1.record(stream)
        stream.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (reps * len(steps))

    def tables(rows, offset, base):
        ang = (np.arange(rows)[:, None] + offset) * base ** (-2.0 * np.arange(32)[None, :] / 64)
        return (torch.from_numpy(np.cos(ang).astype(np.float32)).cuda(),
                torch.from_numpy(np.sin(ang).astype(np.float32)).cuda())

    def layer_steps(mixed):
        steps = []
        rope = tables(shape.ctx + 8, 0.5, 10000.0) if mixed else None
        comp_rope = tables(shape.max_comp + 1, 0.25, 500.0) if mixed else None
        for x in xs:
            comp, swa = x["comp_kv"], x["swa"]
            if mixed:
                comp = torch.empty(1, shape.max_comp, csa.MIX_REC_BYTES, dtype=torch.uint8, device="cuda")
                swa = torch.empty(1, shape.w, csa.MIX_REC_BYTES, dtype=torch.uint8, device="cuda")
                csa.csa_pack_kv_mixed(x["comp_kv"], comp)
                csa.csa_pack_kv_mixed(x["swa"], swa)
            L = csa.make_layer_desc(comp_kv=comp, idx_keys=None, swa=swa, main_bias=x["main_bias"],
                                    idx_bias=None, sink=x["sink"], n_comp=x["n_comp"], swa_head=x["swa_head"],
                                    swa_len=x["swa_len"], h=shape.h, h_i=0, m=shape.m, top_k=0, rope=rope,
                                    comp_rope=comp_rope)
            out = torch.empty(1, shape.h, shape.d, dtype=torch.bfloat16, device="cuda")
            io = csa.make_step_io(pos=x["pos"], q=x["q"], kv_new=x["kv_new"], z_main=x["z_main"],
                                  c_main=x["c_main"], out=out)
            ws = torch.empty(csa.csa_hca_decode_step_workspace_size(L), dtype=torch.uint8, device="cuda")
            steps.append((L, io, ws))
        torch.cuda.synchronize()
        return steps

    us = replay(layer_steps(False))
    torch.cuda.empty_cache()
    us_mixed = replay(layer_steps(True))
    n, d, w, h, m = shape.n_comp, shape.d, shape.w, shape.h, shape.m
    # cache rows + window + q read, out written; the block's Z/C read and the entry written; the new row appended
    alg = (n + w) * d * 2 + h * d * 2 + h * d * 2 + 2 * m * d * 4 + d * 2 + 2 * d * 2
    # the same with 592-byte records for the rows, the entry and the appended row (kv_new read as bf16)
    rec = csa.MIX_REC_BYTES
    alg_mixed = (n + w) * rec + h * d * 2 + h * d * 2 + 2 * m * d * 4 + rec + d * 2 + rec
    del xs
    torch.cuda.empty_cache()
    return {
        "workload": "hca1m: one decode token through 30 HCA layers (ratio 128, no indexer), context 1,000,064 "
                    "(7813 compressed entries incl. the one this step completes, SWA 128 with wrap), batch 1, "
                    "main attention 64 heads x 512 bf16 with sink over every entry + the window",
        "us_per_layer": round(us, 3),
        "steps_per_s_30_layers": round(1e6 / (us * 30), 1),
        "alg_bytes_per_layer": alg,
        "achieved_gbps": round(alg / (us * 1e-6) / 1e9, 1),
        "frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        "mixed_kv": {
            "us_per_layer": round(us_mixed, 3),
            "steps_per_s_30_layers": round(1e6 / (us_mixed * 30), 1),
            "alg_bytes_per_layer": alg_mixed,
            "achieved_gbps": round(alg_mixed / (us_mixed * 1e-6) / 1e9, 1),
            "frac": round(alg_mixed / (us_mixed * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
        },
    }


def time_batch128k(csa, reps: int, n_caches: int = 8):
    """Batched decode at 128K context: 8 independent sequences (n_comp 32768
    each) through one csa_decode_step per layer, over `n_caches` independent
    layer caches (about 336 MB each, so successive layers read from HBM, not
    the 256 MB last-level cache), captured in one graph and replayed `reps`
    times.  Returns the mean time per layer step (all 8 sequences) and its
    algorithmic bytes."""
    import torch
    import synth

    shape = synth.with_(synth.SHAPES["batch128k"], layers=n_caches)
    layers = build_layers(csa, shape, torch.device("cuda:0"))
    stream = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for ly in layers:  # eager once, then capture
            csa.csa_decode_step(ly["L"], ly["io"], ly["ws"], stream=stream)
        with torch.cuda.graph(g, stream=stream):
            for ly in layers:
                csa.csa_decode_step(ly["L"], ly["io"], ly["ws"], stream=stream)
        g.replay()
        stream.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    stream.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * len(layers))
    alg = algorithmic_bytes(shape)["per_layer"] * shape.batch
    del layers
    torch.cuda.empty_cache()
    return {
        "workload": "batch128k: 8 independent sequences at context 131,072 (n_comp 32,768 each, SWA 128), one "
                    "decode token each through one CSA layer; indexer 64x128 bf16, top_k 512, main attention "
                    f"64 heads x 512 bf16 with sink; {n_caches} independent layer caches replayed in turn",
        "us_per_layer_step": round(us, 3),
        "layer_steps_per_s": round(1e6 / us, 1),
        "sequence_tokens_per_s_per_layer": round(shape.batch * 1e6 / us, 1),
        "alg_bytes_per_layer_step": alg,
        "achieved_gbps": round(alg / (us * 1e-6) / 1e9, 1),
        "frac": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
    }


def cpu_baseline(layers, shape, budget_s: float):
    """The float64 oracle on the host, layer by layer, until the budget is spent."""
    import numpy as np
    import oracle
    from oracle import numfmt

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        threads = 1
    cores = len(os.sched_getaffinity(0))

    def f64(t):
        import torch
        if t.dtype == torch.bfloat16:
            return numfmt.bf16_bits_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))
        return t.cpu().numpy().astype(np.float64)

    times = []
    for ly in layers:
        x = ly["x"]
        st = oracle.LayerState(comp_kv=f64(x["comp_kv"][0]), idx_keys=f64(x["idx_keys"][0]),
                               n_comp=x["n_comp"] - 0, swa=oracle.SwaRing(f64(x["swa"][0]), x["swa_head"],
                                                                        x["swa_len"]),
                               main_bias=f64(x["main_bias"]), idx_bias=f64(x["idx_bias"]),
                               sink=f64(x["sink"]), round_cache=numfmt.bf16_round_f64)
        # the GPU step already wrote this step's block into the caches; the
        # oracle recomputes it into the same slot
        st.n_comp = x["n_comp"]
        args = dict(q=f64(x["q"][0]), q_idx=f64(x["q_idx"][0]), w_idx=f64(x["w_idx"][0]),
                    kv_new=f64(x["kv_new"][0]), pos=x["pos"], top_k=shape.top_k,
                    z_main=f64(x["z_main"][0]), c_main=f64(x["c_main"][0]), z_idx=f64(x["z_idx"][0]),
                    c_idx=f64(x["c_idx"][0]), scale=1.0 / np.sqrt(shape.d))
        t0 = time.perf_counter()
        oracle.decode_step(st, **args)
        times.append(time.perf_counter() - t0)
        del st
        if sum(times) > budget_s:
            break
    per_layer = sum(times) / len(times)
    return {"value": 1.0 / (per_layer * shape.layers), "unit": "steps/s", "cores": min(threads, cores),
            "kind": "oracle",
            "sample": f"{len(times)} of {shape.layers} layers of one decode step at n_comp={shape.n_comp} "
                      f"(float64 numpy oracle, mean {per_layer:.3f} s/layer; steps/s = 1/(30 x mean))"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time (0 = skip)")
    ap.add_argument("--scan-reps", type=int, default=10)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the decode path runs "
              "on a single MI355X (multi-GPU sharding is not implemented)", file=sys.stderr)
        return 2

    import torch
    import compressed_sparse_attention_reduce_amd as csa
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    shape = synth.SHAPES["ctx1m"]
    csa.lib()
    layers = build_layers(csa, shape, dev)
    torch.cuda.synchronize()

    # eager warm-up, then a reference copy of layer 0's output
    for _ in range(max(1, args.warmup // 4)):
        run_step(csa, layers)
    torch.cuda.synchronize()
    ref_out = layers[0]["outs"]["out"].clone()
    ref_idx = layers[0]["outs"]["topk_idx"].clone()

    # eager timing (host launch overhead included)
    n_eager = max(3, min(20, args.steps // 10))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_eager):
        run_step(csa, layers)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / n_eager

    graph = None
    if args.mode == "graph":
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_step(csa, layers)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        # every replay must reproduce the eager result
        assert torch.equal(layers[0]["outs"]["out"], ref_out), "graph replay differs from eager"
        assert torch.equal(layers[0]["outs"]["topk_idx"], ref_idx), "graph replay differs from eager"

    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            run_step(csa, layers)
    e1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    ms_per_step = e0.elapsed_time(e1) / args.steps
    assert torch.equal(layers[0]["outs"]["out"], ref_out), "timed replays differ from eager"

    scan_ms, scan_launches = time_scan_kernel(csa, layers, shape, args.scan_reps)
    ceil_us, ceil_bytes = time_read_ceiling(csa, layers, args.scan_reps)
    ceil_gbs = ceil_bytes / (ceil_us * 1e-6) / 1e9
    ab = algorithmic_bytes(shape)
    scan_gbs = ab["scan_launch"] / (scan_ms * 1e-3) / 1e9
    step_bytes = ab["per_layer"] * shape.layers
    step_gbs = step_bytes / (ms_per_step * 1e-3) / 1e9

    fp8_ms, fp8_bytes, fp8_step_ms = time_fp8(csa, layers, shape, args.scan_reps, max(20, args.steps // 2))
    fp8_gbs = fp8_bytes / (fp8_ms * 1e-3) / 1e9
    mixed_ms = time_mixed_kv(csa, layers, shape, max(20, args.steps // 2))
    dev_ms = time_dev_step(csa, layers, shape, max(20, args.steps // 2), 4)

    cpu = None
    if args.cpu_budget > 0:
        cpu = cpu_baseline(layers, shape, args.cpu_budget)
    del layers  # the 1M-context caches make room for the prefill workload
    torch.cuda.empty_cache()
    prefill = time_prefill(csa, max(2, args.scan_reps // 2))
    hca = time_hca(csa, args.scan_reps)
    batch = time_batch128k(csa, max(10, args.steps // 4))

    res = {
        "metric": "CSA decode steps/s and indexer-scan HBM GB/s at 1M ctx (250K comp entries)",
        "value": round(1e3 / ms_per_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "ctx1m: one decode token through 30 CSA layers, context 1,000,000 "
                        "(n_comp 250,000, SWA 128 with wrap), batch 1, indexer 64x128 bf16, "
                        "top_k 512, main attention 64 heads x 512 bf16 with sink",
            "layers": shape.layers, "n_comp": shape.n_comp, "top_k": shape.top_k,
            "swa": shape.w, "batch": shape.batch, "mode": args.mode,
        },
        "scan_gbps": round(scan_gbs, 1),
        "step_gbps": round(step_gbs, 1),
        "step_hbm_frac": round(step_gbs / HBM_PEAK_GBS, 4),
        "eager_ms_per_step": round(eager_ms, 4),
        "wall_ms_timed": round(wall_ms, 2),
        "roofline": {
            "kernel": "k_index_score_bf16",
            "bound": "hbm",
            "achieved": round(scan_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(scan_gbs / HBM_PEAK_GBS, 4),
            "traffic": scan_traffic(),
            "alg_bytes_per_launch": ab["scan_launch"],
            "avg_launch_us": round(scan_ms * 1e3, 3),
            "launches_timed": scan_launches,
            # context: a plain streaming read of the same caches, one launch each
            "read_ceiling_gbps": round(ceil_gbs, 1),
            "read_ceiling_us": round(ceil_us, 3),
            "frac_of_read_ceiling": round(scan_gbs / ceil_gbs, 4),
        },
        "fp8_scan": {
            "kernel": "k_index_score_fp8",
            "avg_launch_us": round(fp8_ms * 1e3, 3),
            "alg_bytes_per_launch": fp8_bytes,
            "achieved_gbps": round(fp8_gbs, 1),
            "frac": round(fp8_gbs / HBM_PEAK_GBS, 4),
            "decode_steps_per_s": round(1e3 / fp8_step_ms, 2),
            "decode_ms_per_step": round(fp8_step_ms, 5),
        },
        "device_counters": {
            "workload": "ctx1m decode step as above through csa_decode_step_dev: one graph replayed, each replay "
                        "the next token (positions, block completions and the SWA ring advanced on the device)",
            "decode_steps_per_s": round(1e3 / dev_ms, 2),
            "decode_ms_per_step": round(dev_ms, 5),
        },
        "mixed_kv": {
            "workload": "ctx1m decode step as above with mixed main KV: every compressed entry and window row "
                        "a 592-byte record (448 E4M3 NoPE codes + scale, 64 bf16 RoPE values), RoPE on the new "
                        "entry, inverse RoPE on the output",
            "decode_steps_per_s": round(1e3 / mixed_ms, 2),
            "decode_ms_per_step": round(mixed_ms, 5),
        },
        "prefill": prefill,
        "hca": hca,
        "batch128k": batch,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
