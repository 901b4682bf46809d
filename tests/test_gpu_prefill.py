"""GPU parity of the prefill-shaped chunk (many query tokens at consecutive
positions against one compressed history) against the float64 CPU oracle.

* multi-query index score (csa_index_score with >= 16 query rows): 1e-4
  relative, and bit-identical to the one-query scan on the same inputs;
* csa_index_topk: bit-exact against the oracle's top-k of the GPU's own
  scores, and the gap rule against the oracle's float64 scores;
* csa_prefill_attn: bfloat16 outputs within 2e-2 relative of the oracle's
  attention over the same selected rows and window.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import numfmt
from tests.gpu_util import assert_lse_close, DEV, as_f64, assert_topk_gap_rule, dev_bf16, dev_f32, host_f64, rel_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import compressed_sparse_attention_reduce_amd as pkg
    pkg.lib()
    return pkg


def _g(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _bf16(g, shape, std=1.0):
    return synth.to_bf16_bits((g.standard_normal(shape, dtype=np.float32) * np.float32(std)))


def _visible(pos, n, ratio=4):
    return np.clip((np.asarray(pos, dtype=np.int64) - (ratio - 1)) // ratio + 1, 0, n)


# ---------------------------------------------------------------------------
# multi-query index score
# ---------------------------------------------------------------------------

MQ_CASES = [
    # name, B, t, n, causal
    ("mq_causal_ragged_batch2", 2, 37, 1000, True),
    ("mq_16_rows_31_keys", 1, 16, 31, False),
    ("mq_70_rows_4111_keys", 1, 70, 4111, True),
    ("mq_one_key", 3, 17, 1, False),
]


@pytest.mark.parametrize("case", MQ_CASES, ids=[c[0] for c in MQ_CASES])
def test_multi_query_score(csa, case):
    name, B, t, n, causal = case
    g = _g(t * 1000 + n)
    q = _bf16(g, (B, t, 64, 128), 1 / np.sqrt(128))
    w = g.standard_normal((B, t, 64), dtype=np.float32)
    K = _bf16(g, (B, n, 128))
    ld = n + 3
    scores = torch.full((B, t, ld), 123.0, device=DEV)
    pos_np = None
    pos = None
    if causal:
        pos_np = (4 * n - 2 * t - 9 + 2 * np.arange(B * t)).astype(np.int32).reshape(B, t)
        pos = torch.from_numpy(pos_np).to(DEV)
    csa.csa_index_score(dev_bf16(q), dev_f32(w), dev_bf16(K), scores, q_pos=pos, ratio=4)
    torch.cuda.synchronize()
    got = scores.cpu().numpy().astype(np.float64)
    assert (got[:, :, n:] == 123.0).all(), "wrote past n"
    for b in range(B):
        ref = oracle.index_score(as_f64(q[b]), w[b], as_f64(K[b]), q_pos=None if pos_np is None else pos_np[b])
        fin = np.isfinite(ref)
        assert (np.isfinite(got[b, :, :n]) == fin).all(), "mask differs"
        assert rel_err(got[b, :, :n][fin], ref[fin]) <= 1e-4


def test_multi_query_score_bit_identical_to_one_query_scan(csa):
    """24 query rows in one call (multi-query scan) and one row per call (the
    decode scan): the same bits for every (query, key)."""
    g = _g(77)
    t, n = 24, 2500
    q = dev_bf16(_bf16(g, (1, t, 64, 128), 1 / np.sqrt(128)))
    w = dev_f32(g.standard_normal((1, t, 64), dtype=np.float32))
    K = dev_bf16(_bf16(g, (1, n, 128)))
    many = torch.empty(1, t, n, device=DEV)
    csa.csa_index_score(q, w, K, many)
    one = torch.empty(1, t, n, device=DEV)
    for r in range(t):
        csa.csa_index_score(q[:, r:r + 1], w[:, r:r + 1], K, one[:, r:r + 1])
    torch.cuda.synchronize()
    assert torch.equal(many, one)


# ---------------------------------------------------------------------------
# fused score + top-k over the chunk
# ---------------------------------------------------------------------------

TOPK_CASES = [
    # name, t, n, k, pos0
    ("two_chunks_causal", 300, 2000, 64, 7800),
    ("fewer_visible_than_k", 20, 400, 512, 1000),
    ("no_mask", 17, 5000, 512, -1),
    ("k1_one_chunk", 40, 3000, 1, 11997),
    ("ragged_last_chunk", 261, 700, 128, 2600),
]


def _run_index_topk(csa, q, w, K, k, pos0, n=None):
    t = q.shape[0]
    n = K.shape[0] if n is None else n
    idx = torch.full((t, k), -5, dtype=torch.int32, device=DEV)
    cnt = torch.full((t,), -5, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(csa.csa_index_topk_workspace_size(t, n, k), 16), dtype=torch.uint8, device=DEV)
    ws.fill_(0xCD)  # needs no initialisation
    csa.csa_index_topk(q, w, K, idx, cnt, ws, pos0=pos0, n=n)
    return idx, cnt


@pytest.mark.parametrize("case", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_index_topk(csa, case):
    name, t, n, k, pos0 = case
    g = _g(t + 7 * n + k)
    qn = _bf16(g, (t, 64, 128), 1 / np.sqrt(128))
    wn = g.standard_normal((t, 64), dtype=np.float32)
    Kn = _bf16(g, (n, 128))
    q, w, K = dev_bf16(qn), dev_f32(wn), dev_bf16(Kn)
    idx, cnt = _run_index_topk(csa, q, w, K, k, pos0)
    # the GPU's own scores (same bits as the chunk scan), with the same mask
    scores = torch.empty(1, t, n, device=DEV)
    pos = None
    if pos0 >= 0:
        pos = torch.arange(pos0, pos0 + t, dtype=torch.int32, device=DEV)[None]
    csa.csa_index_score(q[None], w[None], K[None], scores, q_pos=pos)
    torch.cuda.synchronize()
    gs = scores[0].cpu().numpy().astype(np.float64)
    ri, rc = oracle.topk(gs, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    if pos0 >= 0:
        np.testing.assert_array_equal(rc, np.minimum(k, _visible(pos0 + np.arange(t), n)))
    # against the oracle's float64 scores on a few rows
    rows = sorted({0, t // 2, t - 1})
    ref = oracle.index_score(as_f64(qn[rows]), wn[rows], as_f64(Kn),
                             q_pos=None if pos0 < 0 else pos0 + np.array(rows))
    for i, r in enumerate(rows):
        assert_topk_gap_rule(idx[r].cpu().numpy(), int(cnt[r]), ref[i], k)


def test_index_topk_tied_scores_take_exact_path(csa):
    """Zero queries: every visible block scores 0, so the candidates of the
    row selector overflow and it falls back to the exact path; the answer is
    the lowest visible indices."""
    t, n, k = 20, 30000, 512
    q = torch.zeros(t, 64, 128, dtype=torch.bfloat16, device=DEV)
    w = dev_f32(_g(6).standard_normal((t, 64), dtype=np.float32))
    K = dev_bf16(_bf16(_g(7), (n, 128)))
    pos0 = 4 * 20000
    idx, cnt = _run_index_topk(csa, q, w, K, k, pos0)
    torch.cuda.synchronize()
    assert (cnt.cpu().numpy() == k).all()
    np.testing.assert_array_equal(idx.cpu().numpy(), np.tile(np.arange(k, dtype=np.int32), (t, 1)))


def test_index_topk_empty_history(csa):
    g = _g(5)
    q = dev_bf16(_bf16(g, (16, 64, 128)))
    w = dev_f32(g.standard_normal((16, 64), dtype=np.float32))
    K = torch.empty(0, 128, dtype=torch.bfloat16, device=DEV)
    idx, cnt = _run_index_topk(csa, q, w, K, 8, 0)
    torch.cuda.synchronize()
    assert (idx == -1).all() and (cnt == 0).all()


# ---------------------------------------------------------------------------
# E4M3 keys: multi-query FP8 score and score + top-k
# ---------------------------------------------------------------------------

def _fp8(g, shape_q, n):
    """E4M3 query (per head row) and keys (per key row), quantised by the
    oracle's quantiser; the query's scales folded into w."""
    q = (g.standard_normal(shape_q) / np.sqrt(128)).astype(np.float32)
    w = g.standard_normal(shape_q[:-1]).astype(np.float32)
    K = g.standard_normal((n, 128)).astype(np.float32)
    qc, qs = numfmt.quantize_e4m3_rows(q.reshape(-1, 128))
    kc, ks = numfmt.quantize_e4m3_rows(K) if n else (np.zeros((0, 128), np.uint8), np.zeros(0, np.float32))
    return qc.reshape(shape_q), (w * qs.reshape(w.shape)).astype(np.float32), kc, ks


MQ8_CASES = [
    # name, B, t, n, causal
    ("mq8_causal_ragged_batch2", 2, 37, 1000, True),
    ("mq8_16_rows_31_keys", 1, 16, 31, False),
    ("mq8_70_rows_4111_keys", 1, 70, 4111, True),
    ("mq8_one_key", 3, 17, 1, False),
    ("mq8_300_rows_2049_keys", 1, 300, 2049, True),
]


@pytest.mark.parametrize("case", MQ8_CASES, ids=[c[0] for c in MQ8_CASES])
def test_multi_query_score_fp8(csa, case):
    name, B, t, n, causal = case
    g = _g(t * 1000 + n + 5)
    qc, w, kc, ks = _fp8(g, (B, t, 64, 128), B * n)
    kc, ks = kc.reshape(B, n, 128), ks.reshape(B, n)
    ld = n + 3
    scores = torch.full((B, t, ld), 123.0, device=DEV)
    pos_np = None
    if causal:
        pos_np = (4 * n - 2 * t - 9 + 2 * np.arange(B * t)).astype(np.int32).reshape(B, t)
    csa.csa_index_score_fp8(torch.from_numpy(qc).to(DEV), dev_f32(w), torch.from_numpy(kc).to(DEV), dev_f32(ks),
                            scores, q_pos=None if pos_np is None else torch.from_numpy(pos_np).to(DEV))
    torch.cuda.synchronize()
    got = scores.cpu().numpy().astype(np.float64)
    assert (got[:, :, n:] == 123.0).all(), "wrote past n"
    for b in range(B):
        ref = oracle.index_score_fp8(qc[b], w[b], kc[b], ks[b], q_pos=None if pos_np is None else pos_np[b])
        fin = np.isfinite(ref)
        assert (np.isfinite(got[b, :, :n]) == fin).all(), "mask differs"
        assert rel_err(got[b, :, :n][fin], ref[fin]) <= 1e-4


def _run_index_topk_fp8(csa, qc, w8, kc, ks, k, pos0, n=None):
    t = qc.shape[0]
    n = kc.shape[0] if n is None else n
    idx = torch.full((t, k), -5, dtype=torch.int32, device=DEV)
    cnt = torch.full((t,), -5, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(csa.csa_index_topk_workspace_size(t, n, k), 16), dtype=torch.uint8, device=DEV)
    ws.fill_(0xCD)
    csa.csa_index_topk_fp8(qc, w8, kc, ks, idx, cnt, ws, pos0=pos0, n=n)
    return idx, cnt


@pytest.mark.parametrize("case", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_index_topk_fp8(csa, case):
    """Top-k over the FP8 chunk scan: bit-exact against the oracle's top-k of
    the same scan's scores (csa_index_score_fp8 runs the same multi-query
    kernel from 16 rows on), the gap rule against the oracle's FP8 scores."""
    name, t, n, k, pos0 = case
    g = _g(t + 7 * n + k + 1)
    qn, wn, kn, ksn = _fp8(g, (t, 64, 128), n)
    qc, w8, kc, ks = torch.from_numpy(qn).to(DEV), dev_f32(wn), torch.from_numpy(kn).to(DEV), dev_f32(ksn)
    idx, cnt = _run_index_topk_fp8(csa, qc, w8, kc, ks, k, pos0)
    scores = torch.empty(1, t, n, device=DEV)
    pos = None
    if pos0 >= 0:
        pos = torch.arange(pos0, pos0 + t, dtype=torch.int32, device=DEV)[None]
    assert t >= 16  # the standalone call takes the multi-query kernel too
    csa.csa_index_score_fp8(qc[None], w8[None], kc[None], ks[None], scores, q_pos=pos)
    torch.cuda.synchronize()
    gs = scores[0].cpu().numpy().astype(np.float64)
    ri, rc = oracle.topk(gs, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    if pos0 >= 0:
        np.testing.assert_array_equal(rc, np.minimum(k, _visible(pos0 + np.arange(t), n)))
    rows = sorted({0, t // 2, t - 1})
    ref = oracle.index_score_fp8(qn[rows], wn[rows], kn, ksn, q_pos=None if pos0 < 0 else pos0 + np.array(rows))
    for i, r in enumerate(rows):
        assert_topk_gap_rule(idx[r].cpu().numpy(), int(cnt[r]), ref[i], k)


def test_index_topk_fp8_empty_history(csa):
    g = _g(15)
    qn, wn, _, _ = _fp8(g, (16, 64, 128), 0)
    kc = torch.empty(0, 128, dtype=torch.uint8, device=DEV)
    ks = torch.empty(0, dtype=torch.float32, device=DEV)
    idx, cnt = _run_index_topk_fp8(csa, torch.from_numpy(qn).to(DEV), dev_f32(wn), kc, ks, 8, 0)
    torch.cuda.synchronize()
    assert (idx == -1).all() and (cnt == 0).all()


def test_prefill_fp8_keys_full_size_sampled(csa):
    """The 2048 x 65536 chunk with E4M3 keys and queries quantised on the GPU:
    counts, the top-512 of 16 sampled rows bit-exact against the oracle's
    top-k of the same kernel's scores, the gap rule and the scores against
    the oracle's FP8 score on two rows; the overlap with the bf16 top-512 is
    the format's own figure (E4M3 moves crowded scores across the threshold;
    the 0.99 gate is met by the two-stage selection,
    test_prefill_fp8_rescored_full_size_recall)."""
    shape = synth.SHAPES["prefill"]
    x = synth.make_prefill_inputs_torch(shape, None, DEV)
    T, N, k = shape.t, shape.n_comp, shape.top_k
    kc = torch.empty(N, 128, dtype=torch.uint8, device=DEV)
    ks = torch.empty(N, dtype=torch.float32, device=DEV)
    csa.csa_quantize_fp8(x["idx_keys"], kc, ks)
    qc = torch.empty(T, 64, 128, dtype=torch.uint8, device=DEV)
    w8 = torch.empty(T, 64, dtype=torch.float32, device=DEV)
    csa.csa_quantize_query_fp8(x["q_idx"], x["w_idx"], qc, w8)
    idx, cnt = _run_index_topk_fp8(csa, qc, w8, kc, ks, k, x["pos0"])
    idx16, _ = _run_index_topk(csa, x["q_idx"], x["w_idx"], x["idx_keys"], k, x["pos0"])
    torch.cuda.synchronize()
    pos = x["pos0"] + np.arange(T)
    assert (cnt.cpu().numpy() == np.minimum(k, _visible(pos, N))).all()
    rows = [0, 1, 2, 3, 255, 256, 257, 511, 1024, 1027, 1500, 1800, 2000, 2045, 2046, 2047]
    sel = torch.tensor(rows, device=DEV)
    scores = torch.empty(1, len(rows), N, device=DEV)
    csa.csa_index_score_fp8(qc[sel][None].contiguous(), w8[sel][None].contiguous(), kc[None], ks[None], scores,
                            q_pos=torch.from_numpy(pos[rows].astype(np.int32)).to(DEV)[None])
    torch.cuda.synchronize()
    gs = scores[0].cpu().numpy().astype(np.float64)
    ri, rc = oracle.topk(gs, k)
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    np.testing.assert_array_equal(gi[rows], ri)
    np.testing.assert_array_equal(gc[rows], rc)
    kcn, ksn = kc.cpu().numpy(), ks.cpu().numpy()
    for i in (0, len(rows) - 1):
        r = rows[i]
        ref = oracle.index_score_fp8(qc[r].cpu().numpy()[None], w8[r].cpu().numpy()[None], kcn, ksn,
                                     q_pos=np.array([pos[r]]))[0]
        fin = np.isfinite(ref)
        assert rel_err(gs[i][fin], ref[fin]) <= 1e-4
        assert_topk_gap_rule(gi[r], int(gc[r]), ref, k)
    i16 = idx16.cpu().numpy()
    overlap = np.mean([len(set(gi[r]) & set(i16[r])) / k for r in range(0, T, 64)])
    print(f"fp8 vs bf16 top-512 overlap over 32 sampled queries: {overlap:.4f}")
    assert overlap >= 0.85  # the format's figure; the gate needs the two-stage selection


# ---------------------------------------------------------------------------
# per-query attention over the selected rows and the window
# ---------------------------------------------------------------------------

ATTN_CASES = [
    # name, t, h, d, n_comp, k, window, pos0, sink, out_bf16, full_count
    ("h64_d512_clipped_windows", 40, 64, 512, 3000, 64, 128, 50, True, True, True),
    ("h16_d128_short_counts", 33, 16, 128, 500, 100, 16, 1000, True, True, False),
    ("h32_d256_f32_no_sink", 18, 32, 256, 700, 40, 8, 7, False, False, False),
    ("h64_d512_from_position0", 20, 64, 512, 0, 16, 128, 0, True, True, False),
]


def _attn_ref(q, comp, idx, cnt, win, window, pos0, sink, scale):
    t = q.shape[0]
    outs, lses = [], []
    for r in range(t):
        p = pos0 + r
        first = max(0, p - window + 1)
        wrows = [win[x - (pos0 - window + 1)] for x in range(first, p + 1)]
        sel = [comp[int(idx[r, j])] for j in range(int(cnt[r]))]
        o, l = oracle.sparse_attn(q[r], np.stack(sel + wrows), sink, scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_prefill_attn(csa, case):
    name, t, h, d, n_comp, k, window, pos0, use_sink, out_bf16, full = case
    g = _g(t * h + d + n_comp)
    qn = _bf16(g, (t, h, d))
    comp = _bf16(g, (max(n_comp, 1), d))
    win = _bf16(g, (t + window - 1, d))
    sink = g.standard_normal(h, dtype=np.float32) if use_sink else None
    idx = g.integers(0, max(n_comp, 1), size=(t, k)).astype(np.int32)
    cnt = np.full(t, k if n_comp else 0, dtype=np.int32) if full else \
        g.integers(0, k + 1, size=t).astype(np.int32) * (n_comp > 0)
    for r in range(t):
        idx[r, cnt[r]:] = -1
    out = torch.full((t, h, d), 7.0, dtype=torch.bfloat16 if out_bf16 else torch.float32, device=DEV)
    lse = torch.empty(t, h, device=DEV)
    scale = 1.0 / np.sqrt(d)
    comp_d = dev_bf16(comp)[:n_comp] if n_comp else dev_bf16(comp)
    csa.csa_prefill_attn(dev_bf16(qn), comp_d, torch.from_numpy(idx).to(DEV), torch.from_numpy(cnt).to(DEV),
                         dev_bf16(win), window, pos0, None if sink is None else dev_f32(sink), scale, out, lse=lse,
                         n_comp=n_comp)
    torch.cuda.synchronize()
    ro, rl = _attn_ref(as_f64(qn), as_f64(comp), idx, cnt, as_f64(win), window, pos0,
                       None if sink is None else sink.astype(np.float64), scale)
    assert rel_err(host_f64(out), ro) <= 2e-2
    assert_lse_close(lse.cpu().numpy(), rl)


# ---------------------------------------------------------------------------
# the whole chunk against the oracle's composition
# ---------------------------------------------------------------------------

def test_prefill_chunk_matches_oracle_composition(csa):
    shape = synth.with_(synth.SHAPES["prefill"], t=48, n_comp=900, ctx=3600, top_k=96)
    x = synth.make_prefill_inputs(shape, 5005)
    T, k, W = shape.t, shape.top_k, shape.w
    q_idx, w_idx, keys = dev_bf16(x["q_idx"]), dev_f32(x["w_idx"]), dev_bf16(x["idx_keys"])
    idx, cnt = _run_index_topk(csa, q_idx, w_idx, keys, k, x["pos0"])
    out = torch.empty(T, shape.h, shape.d, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(T, shape.h, device=DEV)
    csa.csa_prefill_attn(dev_bf16(x["q"]), dev_bf16(x["comp_kv"]), idx, cnt, dev_bf16(x["win_kv"]), W, x["pos0"],
                         dev_f32(x["sink"]), 1.0 / np.sqrt(shape.d), out, lse=lse)
    torch.cuda.synchronize()
    ref = oracle.prefill_chunk(q=as_f64(x["q"]), q_idx=as_f64(x["q_idx"]), w_idx=x["w_idx"],
                               idx_keys=as_f64(x["idx_keys"]), comp_kv=as_f64(x["comp_kv"]),
                               win_kv=as_f64(x["win_kv"]), pos0=x["pos0"], top_k=k, window=W, sink=x["sink"])
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    for r in range(T):
        assert_topk_gap_rule(gi[r], int(gc[r]), ref["scores"][r], k)
    # attention over the GPU's selection (near-tie swaps allowed above)
    ro, rl = _attn_ref(as_f64(x["q"]), as_f64(x["comp_kv"]), gi, gc, as_f64(x["win_kv"]), W, x["pos0"],
                       x["sink"].astype(np.float64), 1.0 / np.sqrt(shape.d))
    assert rel_err(host_f64(out), ro) <= 2e-2
    assert_lse_close(lse.cpu().numpy(), rl)
    same = [r for r in range(T) if (gi[r] == ref["idx"][r]).all()]
    assert len(same) >= T // 2
    assert rel_err(host_f64(out)[same], ref["out"][same]) <= 2e-2


# ---------------------------------------------------------------------------
# the full prefill workload (2048 queries, 65536 blocks), sampled
# ---------------------------------------------------------------------------

def test_prefill_full_size_sampled(csa):
    shape = synth.SHAPES["prefill"]
    x = synth.make_prefill_inputs_torch(shape, None, DEV)
    T, N, k, W = shape.t, shape.n_comp, shape.top_k, shape.w
    idx, cnt = _run_index_topk(csa, x["q_idx"], x["w_idx"], x["idx_keys"], k, x["pos0"])
    out = torch.empty(T, shape.h, shape.d, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(T, shape.h, device=DEV)
    csa.csa_prefill_attn(x["q"], x["comp_kv"], idx, cnt, x["win_kv"], W, x["pos0"], x["sink"],
                         1.0 / np.sqrt(shape.d), out, lse=lse)
    torch.cuda.synchronize()
    pos = x["pos0"] + np.arange(T)
    assert (cnt.cpu().numpy() == np.minimum(k, _visible(pos, N))).all()
    rows = [0, 1, 255, 256, 1027, 2046, 2047]
    sel = torch.tensor(rows, device=DEV)
    scores = torch.empty(1, len(rows), N, device=DEV)
    csa.csa_index_score(x["q_idx"][sel][None], x["w_idx"][sel][None], x["idx_keys"][None], scores,
                        q_pos=torch.from_numpy(pos[rows].astype(np.int32)).to(DEV)[None])
    torch.cuda.synchronize()
    gs = scores[0].cpu().numpy().astype(np.float64)
    ri, rc = oracle.topk(gs, k)
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    np.testing.assert_array_equal(gi[rows], ri)
    np.testing.assert_array_equal(gc[rows], rc)
    keys = host_f64(x["idx_keys"])
    for i in (0, len(rows) - 1):
        r = rows[i]
        ref = oracle.index_score(host_f64(x["q_idx"][r])[None], host_f64(x["w_idx"][r])[None], keys,
                                 q_pos=np.array([pos[r]]))[0]
        assert rel_err(gs[i][np.isfinite(ref)], ref[np.isfinite(ref)]) <= 1e-4
        assert_topk_gap_rule(gi[r], int(gc[r]), ref, k)
    comp = host_f64(x["comp_kv"])
    win = host_f64(x["win_kv"])
    qh = host_f64(x["q"][sel])
    sink = host_f64(x["sink"])
    outs = host_f64(out[sel])
    for i, r in enumerate(rows):
        p = int(pos[r])
        wrows = [win[xx - (x["pos0"] - W + 1)] for xx in range(p - W + 1, p + 1)]
        kv = np.concatenate([comp[gi[r, :gc[r]]], np.stack(wrows)])
        o, l = oracle.sparse_attn(qh[i], kv, sink, 1.0 / np.sqrt(shape.d))
        assert rel_err(outs[i], o) <= 2e-2
        assert_lse_close(lse[r].cpu().numpy(), l)


# ---------------------------------------------------------------------------
# E4M3 keys with the two-stage selection (E4M3 top-k_cand, then exact top-k)
# ---------------------------------------------------------------------------

RESCORED_CASES = [
    # name, t, n, k, k_cand, pos0
    ("two_chunks_causal", 300, 5000, 64, 128, 4 * 5000 - 400),
    ("fewer_visible_than_cand", 40, 1000, 32, 96, 4 * 30),
    ("no_mask_k_equal_cand", 20, 3000, 100, 100, -1),
    ("ragged_chunk_k512", 270, 9000, 512, 1024, -1),
]


def _rescored_inputs(g, t, n):
    f = numfmt.bf16_bits_to_f64
    q = synth.to_bf16_bits((g.standard_normal((t, 64, 128)) / np.sqrt(128)).astype(np.float32))
    w = g.standard_normal((t, 64)).astype(np.float32)
    K = synth.to_bf16_bits(g.standard_normal((n, 128)).astype(np.float32))
    kc, ks = numfmt.quantize_e4m3_rows(f(K).astype(np.float32))
    qc, qs = numfmt.quantize_e4m3_rows(f(q).reshape(-1, 128).astype(np.float32))
    return q, w, K, kc, ks, qc.reshape(t, 64, 128), (w * qs.reshape(t, 64)).astype(np.float32)


def _check_rescored_rows(csa, rows, qd, wd, k16, kc_dev, ks_dev, qc, w8, pos0, n, k, kcand, gi, gc, exact_rows):
    """Rows of the two-stage chunk selection: bit for bit the oracle's two
    stages over the GPU's E4M3 and bf16 scan scores of those rows; the gap
    rule against the float64 exact scores inside the first stage's set."""
    # at least 16 rows per call, so the E4M3 scores come from the multi-query
    # kernel the chunk's first stage uses (its float32 order is its own)
    ext = list(rows) + [r for r in range(qc.shape[0]) if r not in rows][:max(0, 16 - len(rows))]
    sel = torch.tensor(ext, device=DEV)
    pos = None if pos0 < 0 else torch.from_numpy((pos0 + np.asarray(ext)).astype(np.int32)).to(DEV)[None]
    s8 = torch.empty(1, len(ext), n, device=DEV)
    s16 = torch.empty(1, len(ext), n, device=DEV)
    csa.csa_index_score_fp8(torch.from_numpy(qc[ext]).to(DEV)[None], dev_f32(w8[ext])[None], kc_dev[None],
                            ks_dev[None], s8, q_pos=pos)
    csa.csa_index_score(qd[sel][None], wd[sel][None], k16[None], s16, q_pos=pos)
    torch.cuda.synchronize()
    s8 = s8[0, :len(rows)].cpu().numpy().astype(np.float64)
    s16 = s16[0, :len(rows)].cpu().numpy().astype(np.float64)
    want, wc = oracle.rescored_topk(s8, s16, k, kcand)
    np.testing.assert_array_equal(gi[rows], want)
    np.testing.assert_array_equal(gc[rows], wc)
    for i, r in enumerate(rows):
        stage1 = oracle.topk(s8[i][None], kcand)[0][0]
        stage1 = stage1[stage1 >= 0]
        inside = np.full(n, -np.inf)
        inside[stage1] = exact_rows[i][stage1]
        assert_topk_gap_rule(gi[r], int(gc[r]), inside, k)


@pytest.mark.parametrize("case", RESCORED_CASES, ids=[c[0] for c in RESCORED_CASES])
def test_index_topk_fp8_rescored(csa, case):
    name, t, n, k, kcand, pos0 = case
    g = _g(t * 3 + n + k + kcand)
    q, w, K, kcn, ksn, qc, w8 = _rescored_inputs(g, t, n)
    qd, wd, k16 = dev_bf16(q), dev_f32(w), dev_bf16(K)
    kc_dev, ks_dev = torch.from_numpy(kcn).to(DEV), dev_f32(ksn)
    idx = torch.full((t, k), -5, dtype=torch.int32, device=DEV)
    cnt = torch.full((t,), -5, dtype=torch.int32, device=DEV)
    ws = torch.empty(csa.csa_index_topk_fp8_rescored_workspace_size(t, n, k, kcand), dtype=torch.uint8, device=DEV)
    ws.fill_(0xCD)
    print(f"rescored chunk {name}", flush=True)
    csa.csa_index_topk_fp8_rescored(qd, wd, kc_dev, ks_dev, k16, idx, cnt, ws, kcand, pos0=pos0)
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    if pos0 >= 0:
        np.testing.assert_array_equal(gc, np.minimum(k, _visible(pos0 + np.arange(t), n)))
    else:
        assert (gc == min(k, n)).all()
    rows = sorted({0, 1, t // 2, t - 1})
    f = numfmt.bf16_bits_to_f64
    qpos = None if pos0 < 0 else pos0 + np.asarray(rows)
    exact = oracle.index_score(f(q[rows]), w[rows].astype(np.float64), f(K), q_pos=qpos)
    _check_rescored_rows(csa, rows, qd, wd, k16, kc_dev, ks_dev, qc, w8, pos0, n, k, kcand, gi, gc, exact)


def test_prefill_fp8_rescored_full_size_recall(csa):
    """The 2048 x 65536 chunk over E4M3 keys with the two-stage selection
    (top-512 of the E4M3 best 1024): sampled rows' selection exactly the
    oracle's two stages, and top-512 recall against the float64 exact
    indexer of at least 0.99 on each sampled row (the gate of page 1,
    ARCHITECTURE_AND_MEMORY_AUDIT.md, Tier 1 gate 4)."""
    shape = synth.SHAPES["prefill"]
    x = synth.make_prefill_inputs_torch(shape, None, DEV)
    T, N, k, kcand = shape.t, shape.n_comp, shape.top_k, 2 * shape.top_k
    kc_dev = torch.empty(N, 128, dtype=torch.uint8, device=DEV)
    ks_dev = torch.empty(N, dtype=torch.float32, device=DEV)
    csa.csa_quantize_fp8(x["idx_keys"], kc_dev, ks_dev)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    cnt = torch.empty(T, dtype=torch.int32, device=DEV)
    ws = torch.empty(csa.csa_index_topk_fp8_rescored_workspace_size(T, N, k, kcand), dtype=torch.uint8, device=DEV)
    csa.csa_index_topk_fp8_rescored(x["q_idx"], x["w_idx"], kc_dev, ks_dev, x["idx_keys"], idx, cnt, ws, kcand,
                                    pos0=x["pos0"])
    torch.cuda.synchronize()
    gi, gc = idx.cpu().numpy(), cnt.cpu().numpy()
    pos = x["pos0"] + np.arange(T)
    np.testing.assert_array_equal(gc, np.minimum(k, _visible(pos, N)))
    rows = [0, 1, 255, 256, 1027, 2046, 2047]
    f64q = host_f64(x["q_idx"][torch.tensor(rows, device=DEV)])
    wq = x["w_idx"][torch.tensor(rows, device=DEV)].cpu().numpy()
    exact = oracle.index_score(f64q, wq.astype(np.float64), host_f64(x["idx_keys"]), q_pos=pos[rows])
    qc, qs = numfmt.quantize_e4m3_rows(host_f64(x["q_idx"]).reshape(-1, 128).astype(np.float32))
    w8 = (x["w_idx"].cpu().numpy() * qs.reshape(T, 64)).astype(np.float32)
    _check_rescored_rows(csa, rows, x["q_idx"], x["w_idx"], x["idx_keys"], kc_dev, ks_dev, qc.reshape(T, 64, 128), w8,
                         x["pos0"], N, k, kcand, gi, gc, exact)
    recalls = []
    for i, r in enumerate(rows):
        ref = set(oracle.topk(exact[i][None], k)[0][0][:gc[r]].tolist())
        recalls.append(len(ref & set(gi[r, :gc[r]].tolist())) / max(len(ref), 1))
    print("two-stage top-512 recall on sampled chunk rows:", [round(v, 4) for v in recalls])
    assert min(recalls) >= 0.99
