"""GPU parity: every C-ABI entry point against the float64 CPU oracle on the
same seeded inputs.

Tolerances (from the accuracy targets of this path):
* float32 outputs: max|gpu - oracle| / max|oracle| <= 1e-4;
* bfloat16 outputs: relative error <= 2e-2, and bf16-stored compressor
  entries within 1 ulp of round-to-nearest-even(oracle);
* indices / copies (top-k on identical scores, gather): bit-exact;
* top-k against the oracle's own float64 scores: exact sets when the
  k/(k+1) gap exceeds 1e-3 relative, else only near-threshold swaps.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import numfmt
from tests.gpu_util import (assert_lse_close, DEV, as_f64, assert_bf16_close, assert_topk_gap_rule, dev_bf16, dev_f32,
                            dev_store, host_bits, host_f64, rel_err)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import compressed_sparse_attention_reduce_amd as pkg
    pkg.lib()
    return pkg


def _g(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------------------
# 1. compressor reduce
# ---------------------------------------------------------------------------

COMPRESS_CASES = [
    # name, batch, n_blocks, m, d, overlap, first_block, out_bf16, norm, extra_rows
    ("tiny_f32", 1, 1, 4, 128, 0, 0, False, False, 0),
    ("main_bf16_batch8", 8, 1, 4, 512, 0, 0, True, False, 0),
    ("prefill_ragged_tail", 2, 13, 4, 512, 0, 0, False, False, 3),
    ("overlap_from_block0", 2, 7, 4, 128, 1, 0, False, False, 2),
    ("overlap_streaming", 1, 3, 4, 512, 1, 5, True, False, 0),
    ("kv_norm_bf16", 2, 4, 4, 512, 0, 0, True, True, 0),
    ("ratio128", 1, 2, 128, 512, 0, 0, False, False, 0),
    ("ratio1", 1, 5, 1, 64, 0, 0, False, False, 0),
    ("odd_width", 3, 2, 4, 100, 0, 0, False, True, 0),
    ("no_blocks", 1, 0, 4, 128, 0, 0, False, False, 2),
]


@pytest.mark.parametrize("case", COMPRESS_CASES, ids=[c[0] for c in COMPRESS_CASES])
def test_compress(csa, case):
    name, B, nb, m, d, ov, fb, out_bf16, norm, extra = case
    g = _g(sum(map(ord, name)))
    width = 2 * d if ov else d
    lead = fb * m  # rows of earlier blocks (overlap streaming reads block fb-1)
    rows = lead + nb * m + extra
    Z = g.standard_normal((B, rows, width), dtype=np.float32)
    C = g.standard_normal((B, rows, width), dtype=np.float32)
    Bias = (g.standard_normal((m, width), dtype=np.float32) * 0.1).astype(np.float32)
    nw = g.standard_normal(d, dtype=np.float32) if norm else None
    dt = torch.bfloat16 if out_bf16 else torch.float32
    out = torch.full((B, max(nb, 1), d), 7.0, dtype=dt, device=DEV)
    z_d, c_d = dev_f32(Z), dev_f32(C)
    csa.csa_compress(z_d[:, lead:], c_d[:, lead:], dev_f32(Bias), out, m=m, overlap=ov, first_block=fb,
                     norm_w=None if nw is None else dev_f32(nw), n_blocks=nb)
    torch.cuda.synchronize()
    if nb == 0:
        assert (out.float() == 7.0).all()
        return
    for b in range(B):
        ref = oracle.compress(Z[b], C[b], Bias, m, overlap=bool(ov))[fb:fb + nb]
        if nw is not None:
            ref = oracle.kv_norm(ref, nw)
        if out_bf16:
            assert_bf16_close(host_bits(out[b]), ref)
            assert rel_err(host_f64(out[b]), ref) <= 2e-2
        else:
            assert rel_err(host_f64(out[b]), ref) <= 1e-4


# ---------------------------------------------------------------------------
# 2. lightning-indexer score
# ---------------------------------------------------------------------------

def _score_inputs(g, B, t, n, bf16, h_i=64, d_i=128):
    q = (g.standard_normal((B, t, h_i, d_i), dtype=np.float32) / np.float32(np.sqrt(d_i))).astype(np.float32)
    w = g.standard_normal((B, t, h_i), dtype=np.float32)
    K = g.standard_normal((B, n, d_i), dtype=np.float32)
    if bf16:
        q, K = synth.to_bf16_bits(q), synth.to_bf16_bits(K)
    return q, w, K


SCORE_CASES = [
    # name, B, t, n, bf16, causal
    ("bf16_ragged_tail", 2, 1, 1000, True, False),
    ("bf16_batch8", 8, 1, 4096, True, False),
    ("bf16_one_key", 1, 1, 1, True, False),
    ("bf16_31_keys", 1, 1, 31, True, False),
    ("bf16_33_keys", 3, 1, 33, True, False),
    ("bf16_causal_multiquery", 1, 5, 600, True, True),
    ("f32_tiny", 1, 1, 256, False, False),
    ("f32_causal", 2, 3, 77, False, True),
]


@pytest.mark.parametrize("case", SCORE_CASES, ids=[c[0] for c in SCORE_CASES])
def test_index_score(csa, case):
    name, B, t, n, bf16, causal = case
    g = _g(len(name) * 31 + n)
    q, w, K = _score_inputs(g, B, t, n, bf16)
    ld = n + 5
    scores = torch.full((B, t, ld), 123.0, device=DEV)
    pos = None
    pos_np = None
    if causal:
        pos_np = (4 * n - 4 * t - 10 + 3 * np.arange(B * t)).astype(np.int32).reshape(B, t)
        pos = torch.from_numpy(pos_np).to(DEV)
    csa.csa_index_score(dev_store(q), dev_f32(w), dev_store(K), scores, q_pos=pos, ratio=4)
    torch.cuda.synchronize()
    got = scores.cpu().numpy().astype(np.float64)
    assert (got[:, :, n:] == 123.0).all(), "wrote past n"
    for b in range(B):
        ref = oracle.index_score(as_f64(q[b]), w[b], as_f64(K[b]),
                                 q_pos=None if pos_np is None else pos_np[b], ratio=4)
        fin = np.isfinite(ref)
        assert (np.isfinite(got[b, :, :n]) == fin).all(), "mask differs"
        assert rel_err(got[b, :, :n][fin], ref[fin]) <= 1e-4


def test_index_score_full_size_sampled(csa):
    """n_comp = 250000 (1M context) in the bench's launch configuration; the
    oracle recomputes a sample of 4096 keys (plus the first and last tiles)."""
    shape = synth.SHAPES["ctx1m"]
    x = synth.make_decode_inputs_torch(shape, seed=None, device=DEV, layers=1)[0]
    n = shape.n_comp
    scores = torch.empty(1, 1, n, device=DEV)
    csa.csa_index_score(x["q_idx"][:, None], x["w_idx"][:, None], x["idx_keys"], scores)
    torch.cuda.synchronize()
    g = _g(44)
    sample = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n), g.integers(0, n, 4096)]))
    Ks = host_f64(x["idx_keys"][0, torch.from_numpy(sample).to(DEV)])
    ref = oracle.index_score(host_f64(x["q_idx"][0])[None], host_f64(x["w_idx"][0])[None], Ks)[0]
    got = scores[0, 0].cpu().numpy().astype(np.float64)[sample]
    assert rel_err(got, ref) <= 1e-4


# ---------------------------------------------------------------------------
# 2b. FP8 E4M3 indexer keys: quantisation (bit-exact) and the FP8 score
# ---------------------------------------------------------------------------

def _quant_rows(g, rows, d):
    x = (g.standard_normal((rows, d)) * np.exp(g.uniform(-6, 6, (rows, 1)))).astype(np.float32)
    x[0] = 0.0                                        # all-zero row: scale 1
    if rows > 2:
        x[1] = 0.0
        x[1, 0] = 448.0                               # scale exactly 1: the rest is encoded as given
        x[1, 1:12] = [1.0625, 1.1875, 1.9375, 2.0 ** -10, 3 * 2.0 ** -10, -0.0, 1e-30, 449.0,
                      -447.9, 2.0 ** -7 + 2.0 ** -12, -1.0625]
    if rows > 3:
        x[2] = -x[2]                                  # negative row maxima
    return x


QUANT_CASES = [("f32_128", 37, 128, False), ("bf16_512", 9, 512, True), ("f32_odd_width", 5, 100, False),
               ("f32_one_row_d1", 1, 1, False)]


@pytest.mark.parametrize("case", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_quantize_fp8_bit_exact(csa, case):
    name, rows, d, bf16 = case
    x = _quant_rows(_g(rows * 7 + d), rows, d)
    if bf16:
        xb = numfmt.f32_to_bf16_bits(x)
        xd = dev_bf16(xb)
        x = numfmt.bf16_bits_to_f64(xb).astype(np.float32)
    else:
        xd = torch.from_numpy(x).to(DEV)
    codes = torch.full((rows, d), 0x55, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(rows, dtype=torch.float32, device=DEV)
    csa.csa_quantize_fp8(xd, codes, scales)
    torch.cuda.synchronize()
    rc, rs = numfmt.quantize_e4m3_rows(x)
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    np.testing.assert_array_equal(codes.cpu().numpy(), rc)


def _fp8_inputs(g, B, t, n):
    """Query and keys drawn like the bf16 workloads, quantised by the oracle;
    the query's per-head scales are folded into w."""
    q = (g.standard_normal((B, t, 64, 128)) / np.sqrt(128)).astype(np.float32)
    w = g.standard_normal((B, t, 64)).astype(np.float32)
    K = g.standard_normal((B, n, 128)).astype(np.float32)
    qc, qs = numfmt.quantize_e4m3_rows(q.reshape(-1, 128))
    kc, ks = numfmt.quantize_e4m3_rows(K.reshape(-1, 128))
    w2 = (w * qs.reshape(B, t, 64)).astype(np.float32)
    return (qc.reshape(B, t, 64, 128), w2, kc.reshape(B, n, 128), ks.reshape(B, n), K)


FP8_SCORE_CASES = [
    # name, B, t, n, causal
    ("decode_ctx8k", 1, 1, 2048, False),
    ("ragged_tail", 1, 1, 1000, False),
    ("batch3", 3, 1, 4100, False),
    ("short", 1, 1, 17, False),
    ("causal_rows", 2, 3, 700, True),
    ("long_row", 1, 1, 65536, False),
]


@pytest.mark.parametrize("case", FP8_SCORE_CASES, ids=[c[0] for c in FP8_SCORE_CASES])
def test_index_score_fp8(csa, case):
    name, B, t, n, causal = case
    qc, w, kc, ks, _ = _fp8_inputs(_g(len(name) * 17 + n), B, t, n)
    ld = n + 3
    scores = torch.full((B, t, ld), 123.0, device=DEV)
    pos_np = (4 * n - 4 * t - 10 + 3 * np.arange(B * t)).astype(np.int32).reshape(B, t) if causal else None
    csa.csa_index_score_fp8(torch.from_numpy(qc).to(DEV), dev_f32(w), torch.from_numpy(kc).to(DEV),
                            dev_f32(ks), scores, q_pos=None if pos_np is None else torch.from_numpy(pos_np).to(DEV))
    torch.cuda.synchronize()
    got = scores.cpu().numpy().astype(np.float64)
    assert (got[:, :, n:] == 123.0).all(), "wrote past n"
    for b in range(B):
        ref = oracle.index_score_fp8(qc[b], w[b], kc[b], ks[b], q_pos=None if pos_np is None else pos_np[b])
        fin = np.isfinite(ref)
        assert (np.isfinite(got[b, :, :n]) == fin).all(), "mask differs"
        assert rel_err(got[b, :, :n][fin], ref[fin]) <= 1e-4


def test_index_score_fp8_full_size_sampled_and_recall(csa):
    """n = 250,000 FP8 keys quantised on the GPU from the 1M-context bf16
    cache: scores on a sample against the oracle; the FP8 top-512 against the
    bf16 scores' top-512.  That recall is a property of the format (E4M3's
    3-bit significand moves crowded scores across the threshold: 0.936 here,
    as the float64 study in test_fp8_recall.py finds), checked to stay at the
    format's figure; the 0.99 gate is met by the two-stage selection
    (test_decode_step_ctx1m_fp8_rescored_full_size_recall)."""
    shape = synth.SHAPES["ctx1m"]
    x = synth.make_decode_inputs_torch(shape, seed=None, device=DEV, layers=1)[0]
    n = shape.n_comp
    keys = x["idx_keys"][:, :n].contiguous()
    kc = torch.empty(1, n, 128, dtype=torch.uint8, device=DEV)
    ks = torch.empty(1, n, dtype=torch.float32, device=DEV)
    csa.csa_quantize_fp8(keys, kc, ks)
    q = x["q_idx"][:, None].contiguous()               # [1, 1, 64, 128] bf16
    qc = torch.empty(1, 1, 64, 128, dtype=torch.uint8, device=DEV)
    w8 = torch.empty(1, 1, 64, dtype=torch.float32, device=DEV)
    csa.csa_quantize_query_fp8(q, x["w_idx"][:, None].contiguous(), qc, w8)
    # the library's query codes and folded weights are the oracle's, bit for bit
    hqc, hw8 = _fp8_query(host_f64(q[0, 0]).astype(np.float32), x["w_idx"][0].cpu().numpy())
    np.testing.assert_array_equal(qc[0, 0].cpu().numpy(), hqc)
    np.testing.assert_array_equal(w8[0, 0].cpu().numpy().view(np.uint32), hw8.view(np.uint32))
    s8 = torch.empty(1, 1, n, device=DEV)
    csa.csa_index_score_fp8(qc, w8, kc, ks, s8)
    s16 = torch.empty(1, 1, n, device=DEV)
    csa.csa_index_score(q, x["w_idx"][:, None].contiguous(), keys, s16)
    torch.cuda.synchronize()
    g = _g(45)
    sample = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n), g.integers(0, n, 4096)]))
    idx = torch.from_numpy(sample).to(DEV)
    ref = oracle.index_score_fp8(hqc[None], hw8[None], kc[0, idx].cpu().numpy(), ks[0, idx].cpu().numpy())[0]
    assert rel_err(s8[0, 0].cpu().numpy().astype(np.float64)[sample], ref) <= 1e-4
    top8 = set(torch.topk(s8[0, 0], 512).indices.cpu().tolist())
    top16 = set(torch.topk(s16[0, 0], 512).indices.cpu().tolist())
    recall = len(top8 & top16) / 512
    print(f"fp8 top-512 recall vs bf16 keys at n=250000: {recall:.4f}")
    assert recall >= 0.93  # the format's own figure (0.9355); the gate needs the two-stage selection


# ---------------------------------------------------------------------------
# 3. top-k
# ---------------------------------------------------------------------------

def _run_topk(csa, scores_np, k, n=None):
    B, t, ld = scores_np.shape
    n = ld if n is None else n
    s = torch.from_numpy(np.ascontiguousarray(scores_np, dtype=np.float32)).to(DEV)
    idx = torch.full((B, t, k), -7, dtype=torch.int32, device=DEV)
    cnt = torch.full((B, t), -7, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(csa.csa_topk_workspace_size(B, t, n, k), 16), dtype=torch.uint8, device=DEV)
    ws.fill_(0xAB)  # the workspace needs no initialisation
    csa.csa_topk(s, k, idx, cnt, ws, n=n)
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


def _check_topk(scores_np, k, idx, cnt, n=None):
    B, t, ld = scores_np.shape
    n = ld if n is None else n
    for b in range(B):
        ri, rc = oracle.topk(scores_np[b, :, :n].astype(np.float64), k)
        np.testing.assert_array_equal(idx[b], ri)
        np.testing.assert_array_equal(cnt[b], rc)


TOPK_CASES = [
    # name, B, t, n, k, kind
    ("normal_1m_ctx", 1, 1, 250000, 512, "normal"),
    ("normal_8k_batch8", 8, 1, 2048, 512, "normal"),
    ("fewer_than_k", 2, 1, 300, 512, "normal"),
    ("k1", 1, 1, 5000, 1, "normal"),
    ("kmax_2048", 1, 1, 100000, 2048, "normal"),
    ("integer_ties", 1, 1, 20000, 512, "ties"),
    ("all_equal_overflow", 1, 1, 50000, 512, "equal"),
    ("signed_zero_and_masked", 2, 1, 5000, 512, "zeros"),
    ("causal_rows", 1, 3, 65536, 512, "causal"),
    ("exactly_k", 1, 1, 512, 512, "normal"),
    ("heavy_tail_cands", 1, 1, 200000, 512, "lowres"),
]


def _topk_scores(kind, B, t, n, g):
    if kind == "normal":
        return g.standard_normal((B, t, n), dtype=np.float32) * 5
    if kind == "ties":
        return g.integers(-3, 4, size=(B, t, n)).astype(np.float32)
    if kind == "equal":
        return np.full((B, t, n), 2.5, dtype=np.float32)
    if kind == "zeros":
        s = g.standard_normal((B, t, n), dtype=np.float32)
        s[:, :, ::3] = 0.0
        s[:, :, 1::7] = -0.0
        s[s < -0.5] = -np.inf
        s[:, :, :100] = np.where(g.random((B, t, 100)) < 0.5, 0.0, -0.0)
        return s
    if kind == "causal":
        s = g.standard_normal((B, t, n), dtype=np.float32)
        for tt in range(t):
            s[:, tt, n - 700 + 200 * tt:] = -np.inf
        return s
    if kind == "lowres":  # few distinct values near the top: large threshold bin
        return np.round(g.standard_normal((B, t, n)) * 2).astype(np.float32) + g.integers(0, 2, (B, t, n)).astype(np.float32) * np.float32(1e-3)
    raise ValueError(kind)


@pytest.mark.parametrize("case", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_topk(csa, case):
    name, B, t, n, k, kind = case
    s = _topk_scores(kind, B, t, n, _g(n + k))
    idx, cnt = _run_topk(csa, s, k)
    _check_topk(s, k, idx, cnt)


def test_topk_strided_rows_and_empty(csa):
    g = _g(5)
    s = g.standard_normal((3, 2, 1500), dtype=np.float32)
    idx, cnt = _run_topk(csa, s, 64, n=1200)  # ld 1500, only 1200 columns valid
    _check_topk(s, 64, idx, cnt, n=1200)
    idx, cnt = _run_topk(csa, np.zeros((1, 1, 4), np.float32), 8, n=0)
    assert (idx == -1).all() and (cnt == 0).all()


# ---------------------------------------------------------------------------
# 4. gather
# ---------------------------------------------------------------------------

GATHER_CASES = [
    # name, B, n_comp, k, count, W, head, len, d, bf16
    ("ctx1m_wrap", 1, 250000, 512, 512, 128, 64, 128, 512, True),
    ("batch_partial_count", 4, 3000, 512, 200, 128, 0, 128, 512, True),
    ("empty_cache", 2, 0, 512, 0, 128, 17, 40, 512, True),
    ("short_window", 1, 100, 64, 64, 128, 30, 30, 128, False),
    ("tiny_f32_wrap", 1, 256, 64, 64, 128, 0, 128, 128, False),
]


@pytest.mark.parametrize("case", GATHER_CASES, ids=[c[0] for c in GATHER_CASES])
def test_gather(csa, case):
    name, B, n_comp, k, count, W, head, ln, d, bf16 = case
    g = _g(n_comp + k + d)
    torch.manual_seed(n_comp + k + d)
    dt = torch.bfloat16 if bf16 else torch.float32
    comp = torch.randn(B, max(n_comp, 1), d, device=DEV).to(dt)
    swa = torch.randn(B, W, d, device=DEV).to(dt)
    idx_np = np.full((B, k), -1, np.int32)
    for b in range(B):
        if count:
            idx_np[b, :count] = g.choice(n_comp, size=count, replace=False)
    cnt_np = np.full(B, count, np.int32)
    buf = torch.zeros(B, k + W, d, dtype=dt, device=DEV)
    nv = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    csa.csa_gather(comp, torch.from_numpy(idx_np).to(DEV), torch.from_numpy(cnt_np).to(DEV), swa, head, ln,
                   buf, nv, n_comp=n_comp)
    torch.cuda.synchronize()
    rawc = comp.view(torch.int16 if bf16 else torch.int32).cpu().numpy()
    raws = swa.view(torch.int16 if bf16 else torch.int32).cpu().numpy()
    rawb = buf.view(torch.int16 if bf16 else torch.int32).cpu().numpy()
    for b in range(B):
        rows, n_valid = oracle.gather(rawc[b], idx_np[b], count, raws[b], head, ln)
        assert int(nv[b]) == n_valid
        np.testing.assert_array_equal(rawb[b, :n_valid], rows)
        assert (rawb[b, n_valid:] == 0).all(), "rows past n_valid were written"


# ---------------------------------------------------------------------------
# 5. sparse attention
# ---------------------------------------------------------------------------

ATTN_CASES = [
    # name, B, H, D, n_max, n_valid list, sink, bf16, out_bf16
    ("gather_buf_640", 1, 64, 512, 640, [640], True, True, True),
    ("ragged_37", 1, 64, 512, 640, [37], True, True, True),
    ("batch_mixed", 4, 64, 512, 640, [640, 1, 333, 129], True, True, False),
    # more splits than two rounds of workgroups on 256 compute units
    ("wide_batch_ragged", 8, 64, 512, 640, [640, 1, 333, 129, 0, 500, 640, 257], True, True, False),
    ("wide_d256", 16, 32, 256, 1000, [1000, 999, 128, 127, 1, 0, 640, 641] * 2, True, True, True),
    ("no_sink", 1, 32, 256, 96, [96], False, True, True),
    ("empty_with_sink", 1, 16, 128, 64, [0], True, True, False),
    ("empty_no_sink", 1, 16, 128, 64, [0], False, True, False),
    ("f32_tiny", 1, 16, 128, 192, [192], True, False, False),
    ("f32_ragged", 2, 16, 128, 192, [5, 0], True, False, False),
]


@pytest.mark.parametrize("case", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_sparse_attn(csa, case):
    name, B, H, D, n_max, nvs, use_sink, bf16, out_bf16 = case
    g = _g(H * D + n_max)
    q = g.standard_normal((B, H, D), dtype=np.float32)
    kv = g.standard_normal((B, n_max, D), dtype=np.float32)
    if bf16:
        q, kv = synth.to_bf16_bits(q), synth.to_bf16_bits(kv)
    sink = g.standard_normal(H, dtype=np.float32) if use_sink else None
    out = torch.full((B, H, D), 9.0, dtype=torch.bfloat16 if out_bf16 else torch.float32, device=DEV)
    lse = torch.empty(B, H, device=DEV)
    nv = torch.tensor(nvs, dtype=torch.int32, device=DEV)
    ws = torch.empty(csa.csa_sparse_attn_workspace_size(B, H, D, n_max), dtype=torch.uint8, device=DEV)
    scale = 1.0 / np.sqrt(D)
    csa.csa_sparse_attn(dev_store(q), dev_store(kv), nv, None if sink is None else dev_f32(sink), scale, out,
                        lse, ws)
    torch.cuda.synchronize()
    tol = 2e-2 if (bf16 or out_bf16) else 1e-4
    for b in range(B):
        ro, rl = oracle.sparse_attn(as_f64(q[b]), as_f64(kv[b])[: nvs[b]], sink, scale)
        go = host_f64(out[b])
        if nvs[b] == 0:
            assert (go == 0).all()
        else:
            assert rel_err(go, ro) <= tol, name
        gl = lse[b].cpu().numpy().astype(np.float64)
        if np.isinf(rl).all():
            assert np.isinf(gl).all() and (gl < 0).all()
        else:
            assert_lse_close(gl, rl, abs_tol=1e-2 if bf16 else 1e-5, rel_tol=2e-2 if bf16 else 1e-4)


# ---------------------------------------------------------------------------
# 6. fused decode step
# ---------------------------------------------------------------------------

def _run_step(csa, x, shape, with_lse=True):
    """Upload one decode step's inputs, run csa_decode_step, return device state."""
    B, D, K, W = shape.batch, shape.d, shape.top_k, shape.w
    dt = torch.bfloat16 if shape.dtype == "bf16" else torch.float32
    st = {k: dev_store(x[k]) for k in ("comp_kv", "idx_keys", "swa", "q", "q_idx", "kv_new")}
    for k in ("main_bias", "idx_bias", "sink", "w_idx", "z_main", "c_main", "z_idx", "c_idx"):
        st[k] = dev_f32(x[k])
    L = csa.make_layer_desc(comp_kv=st["comp_kv"], idx_keys=st["idx_keys"], swa=st["swa"],
                            main_bias=st["main_bias"], idx_bias=st["idx_bias"], sink=st["sink"],
                            n_comp=x["n_comp"], swa_head=x["swa_head"], swa_len=x["swa_len"], h=shape.h,
                            h_i=shape.h_i, m=shape.m, top_k=K, overlap=int(shape.overlap))
    outs = dict(scores=torch.full((B, x["comp_kv"].shape[1]), 55.0, device=DEV),
                topk_idx=torch.empty(B, K, dtype=torch.int32, device=DEV),
                topk_count=torch.empty(B, dtype=torch.int32, device=DEV),
                gather_buf=torch.zeros(B, K + W, D, dtype=dt, device=DEV),
                n_valid=torch.empty(B, dtype=torch.int32, device=DEV),
                out=torch.empty(B, shape.h, D, dtype=dt, device=DEV),
                lse=torch.empty(B, shape.h, device=DEV) if with_lse else None)
    io = csa.make_step_io(pos=x["pos"], q=st["q"], q_idx=st["q_idx"], w_idx=st["w_idx"], kv_new=st["kv_new"],
                          z_main=st["z_main"], c_main=st["c_main"], z_idx=st["z_idx"], c_idx=st["c_idx"],
                          **outs)
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    csa.csa_decode_step(L, io, ws)
    torch.cuda.synchronize()
    return st, outs, L


def _check_step(x, shape, st, outs, b):
    """Compare one sequence of a decode step with the oracle, stage by stage."""
    bf = shape.dtype == "bf16"
    m, K = shape.m, shape.top_k
    N0 = x["n_comp"]
    completes = x["pos"] % m == m - 1
    N = N0 + int(completes)
    # a. SWA append
    assert np.array_equal(host_f64(st["swa"][b, x["swa_head"]]), as_f64(x["kv_new"][b]))
    # b. compressed entries
    comp = host_f64(st["comp_kv"][b, :N])
    keys = host_f64(st["idx_keys"][b, :N])
    if completes:
        ym = oracle.compress(x["z_main"][b], x["c_main"][b], x["main_bias"], m, overlap=shape.overlap)[-1]
        yi = oracle.compress(x["z_idx"][b], x["c_idx"][b], x["idx_bias"], m, overlap=shape.overlap)[-1]
        if bf:
            assert_bf16_close(host_bits(st["comp_kv"][b, N0]), ym)
            assert_bf16_close(host_bits(st["idx_keys"][b, N0]), yi)
        else:
            assert rel_err(comp[N0], ym) <= 1e-4 and rel_err(keys[N0], yi) <= 1e-4
    np.testing.assert_array_equal(comp[:N0], as_f64(x["comp_kv"][b, :N0]))
    # c. scores (oracle on the cache as the GPU holds it)
    ref_s = oracle.index_score(as_f64(x["q_idx"][b])[None], x["w_idx"][b][None], keys)[0]
    got_s = outs["scores"][b, :N].cpu().numpy().astype(np.float64)
    assert rel_err(got_s, ref_s) <= 1e-4
    # d. top-k: bit-exact on the GPU's own scores, gap rule against the oracle's
    gi = outs["topk_idx"][b].cpu().numpy()
    gc = int(outs["topk_count"][b])
    oi, oc = oracle.topk(got_s[None], K)
    np.testing.assert_array_equal(gi, oi[0])
    assert gc == int(oc[0])
    assert_topk_gap_rule(gi, gc, ref_s, K)
    # e. gather (bit-exact, GPU selection)
    swa_rows = host_f64(st["swa"][b])
    head = (x["swa_head"] + 1) % shape.w
    ln = min(x["swa_len"] + 1, shape.w)
    rows, n_valid = oracle.gather(comp, gi, gc, swa_rows, head, ln)
    assert int(outs["n_valid"][b]) == n_valid
    np.testing.assert_array_equal(host_f64(outs["gather_buf"][b, :n_valid]), rows)
    # f. attention over the gathered rows
    ro, rl = oracle.sparse_attn(as_f64(x["q"][b]), rows, x["sink"], 1.0 / np.sqrt(shape.d))
    assert rel_err(host_f64(outs["out"][b]), ro) <= (2e-2 if bf else 1e-4)
    if outs["lse"] is not None:
        assert_lse_close(outs["lse"][b].cpu().numpy(), rl, abs_tol=1e-2 if bf else 1e-5, rel_tol=2e-2 if bf else 1e-4)


STEP_CASES = [
    # name, shape, seed, cache capacity (None = n_comp)
    ("tiny_f32", synth.SHAPES["tiny"], 1001, None),
    ("ctx8k_bf16", synth.SHAPES["ctx8k"], 2001, None),
    ("no_block_completion", synth.with_(synth.SHAPES["ctx8k"], ctx=8190, n_comp=2047), 2002, None),
    ("first_token", synth.with_(synth.SHAPES["ctx8k"], ctx=1, n_comp=0, top_k=64), 2003, 8),
    ("first_block", synth.with_(synth.SHAPES["ctx8k"], ctx=4, n_comp=1, top_k=64), 2004, None),
    ("overlap_bf16", synth.with_(synth.SHAPES["ctx8k"], ctx=4000, n_comp=1000, overlap=True), 2005, None),
    ("k_covers_all", synth.with_(synth.SHAPES["ctx8k"], ctx=800, n_comp=200), 2006, 256),
    ("tiny_f32_batch3", synth.with_(synth.SHAPES["tiny"], batch=3), 1002, None),
    # 5 x 80 fused workgroups would not all be resident at once: one top-k launch per
    # sequence and the separate attention, with the scan's candidate lists (n_comp 4000)
    # and without them (n_comp 1000 <= 4 top_k)
    ("bf16_batch5_lists", synth.with_(synth.SHAPES["ctx8k"], batch=5, ctx=16000, n_comp=3999), 2007, None),
    ("bf16_batch5_short", synth.with_(synth.SHAPES["ctx8k"], batch=5, ctx=4000, n_comp=999), 2008, None),
]


@pytest.mark.parametrize("case", STEP_CASES, ids=[c[0] for c in STEP_CASES])
def test_decode_step(csa, case):
    name, shape, seed, cap = case
    x = synth.make_decode_inputs(shape, seed, max_comp=cap)
    st, outs, _ = _run_step(csa, x, shape)
    for b in range(shape.batch):
        _check_step(x, shape, st, outs, b)


def test_decode_step_clustered_scores_refine_lists(csa):
    """600 consecutive indexer keys set to copies of the best key: every tile
    they fall in holds 16 of the top k, more than any candidate list keeps, so
    the union cannot prove the answer; the top-k re-reads the slots whose
    bound reaches the k-th largest listed key.  The result must still be the
    oracle's, ties between the copies broken by the lower index."""
    shape = synth.with_(synth.SHAPES["ctx8k"], ctx=131072, n_comp=32768)
    x = synth.make_decode_inputs(shape, 4001)
    n0 = x["n_comp"]
    s = oracle.index_score(as_f64(x["q_idx"][0])[None], x["w_idx"][0][None], as_f64(x["idx_keys"][0, :n0]))[0]
    x["idx_keys"][0, 10000:10600] = x["idx_keys"][0, int(np.argmax(s))]
    st, outs, _ = _run_step(csa, x, shape)
    _check_step(x, shape, st, outs, 0)
    # the scenario happened: the selection is (all but possibly one of) the copies
    gi = outs["topk_idx"][0].cpu().numpy()
    assert np.isin(gi, np.arange(10000, 10600)).sum() >= shape.top_k - 1


@pytest.mark.parametrize("n_comp", [2048, 32768])
def test_decode_step_all_scores_tied(csa, n_comp):
    """Every indexer key equal, so every score ties: the top k is the first k
    blocks.  At 32,768 blocks neither the lists, their refinement nor the
    streaming select can narrow the row to fewer than the pool holds, so the
    exact radix select decides; at 2048 (no lists) the streaming select
    holds the whole row."""
    shape = synth.with_(synth.SHAPES["ctx8k"], ctx=4 * n_comp, n_comp=n_comp)
    x = synth.make_decode_inputs(shape, 4004)
    x["idx_keys"][0, :] = x["idx_keys"][0, 0]
    x["c_idx"][0, :] = 0.0
    x["idx_bias"][:] = 0.0
    st, outs, _ = _run_step(csa, x, shape)
    _check_step(x, shape, st, outs, 0)


def test_decode_step_long_top_k_without_candidate_lists(csa):
    """top_k 2048 over 10,000 blocks: candidate lists would be too long, so
    the step runs the separate top-k and attention kernels."""
    shape = synth.with_(synth.SHAPES["ctx8k"], ctx=40000, n_comp=10000, top_k=2048)
    x = synth.make_decode_inputs(shape, 4002)
    st, outs, _ = _run_step(csa, x, shape)
    _check_step(x, shape, st, outs, 0)


def test_decode_step_batch128k_full_size(csa):
    shape = synth.SHAPES["batch128k"]
    x = synth.make_decode_inputs(shape, 3000)
    st, outs, _ = _run_step(csa, x, shape, with_lse=False)
    for b in range(shape.batch):
        _check_step(x, shape, st, outs, b)


CLUSTER_KEYS = 4096


@pytest.mark.parametrize("clustered", [0, 1, 2], ids=["random_keys", "clustered_recent_keys", "clustered_new_key"])
def test_decode_step_ctx1m_full_size(csa, clustered):
    """One layer of the 1M-context workload (n_comp 250,000, SWA wrap) through
    csa_decode_step, as the benchmark runs it; the oracle scores every key.
    Clustered: the 4096 most recent keys outscore the rest of the cache, so
    the candidate lists cannot prove the top-k and the step refines them by
    re-reading the slots that hold those keys.  With the new key: the block
    the step compresses lies along the same direction (every compressor row
    of the indexer holds it), so it tops the selection from its own list
    while the scan slot its position maps to is re-read."""
    shape = synth.SHAPES["ctx1m"]
    x = synth.make_decode_inputs_torch(shape, seed=None, device=DEV, layers=1)[0]
    if clustered:
        synth.cluster_recent_keys(x["idx_keys"], x["q_idx"], x["w_idx"], x["n_comp"], CLUSTER_KEYS, seed=4003)
    if clustered == 2:
        x["c_idx"][:] = 40.0 * synth.cluster_direction(x["q_idx"], x["w_idx"])[:, None, :]
    B, K, W, D = shape.batch, shape.top_k, shape.w, shape.d
    pristine_keys = x["idx_keys"][0, : x["n_comp"]].clone()
    L = csa.make_layer_desc(comp_kv=x["comp_kv"], idx_keys=x["idx_keys"], swa=x["swa"],
                            main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"],
                            n_comp=x["n_comp"], swa_head=x["swa_head"], swa_len=x["swa_len"], h=shape.h,
                            h_i=shape.h_i, top_k=K)
    outs = dict(scores=torch.empty(B, shape.max_comp, device=DEV),
                topk_idx=torch.empty(B, K, dtype=torch.int32, device=DEV),
                topk_count=torch.empty(B, dtype=torch.int32, device=DEV),
                gather_buf=torch.zeros(B, K + W, D, dtype=torch.bfloat16, device=DEV),
                n_valid=torch.empty(B, dtype=torch.int32, device=DEV),
                out=torch.empty(B, shape.h, D, dtype=torch.bfloat16, device=DEV),
                lse=torch.empty(B, shape.h, device=DEV))
    io = csa.make_step_io(pos=x["pos"], q=x["q"], q_idx=x["q_idx"], w_idx=x["w_idx"], kv_new=x["kv_new"],
                          z_main=x["z_main"], c_main=x["c_main"], z_idx=x["z_idx"], c_idx=x["c_idx"], **outs)
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    csa.csa_decode_step(L, io, ws)
    torch.cuda.synchronize()
    N = shape.n_comp
    assert torch.equal(x["idx_keys"][0, : N - 1], pristine_keys[: N - 1])
    yi = oracle.compress(x["z_idx"][0].cpu().numpy(), x["c_idx"][0].cpu().numpy(),
                         x["idx_bias"].cpu().numpy(), 4)[-1]
    assert_bf16_close(host_bits(x["idx_keys"][0, N - 1]), yi)
    keys = host_f64(x["idx_keys"][0, :N])
    ref_s = oracle.index_score(host_f64(x["q_idx"][0])[None], host_f64(x["w_idx"][0])[None], keys)[0]
    got_s = outs["scores"][0].cpu().numpy().astype(np.float64)
    assert rel_err(got_s, ref_s) <= 1e-4
    gi = outs["topk_idx"][0].cpu().numpy()
    oi, oc = oracle.topk(got_s[None], K)
    np.testing.assert_array_equal(gi, oi[0])
    assert_topk_gap_rule(gi, int(outs["topk_count"][0]), ref_s, K)
    if clustered:  # the scenario happened: the whole selection lies in the recent keys
        assert (gi >= x["n_comp"] - CLUSTER_KEYS).all()
    if clustered == 2:
        assert gi[0] == x["n_comp"]
    sel = host_f64(x["comp_kv"][0, torch.from_numpy(gi).to(DEV).long()])
    swa_rows = host_f64(x["swa"][0])
    head = (x["swa_head"] + 1) % W
    win = np.stack([swa_rows[(head - W + j) % W] for j in range(W)])
    rows = np.concatenate([sel, win])
    assert int(outs["n_valid"][0]) == K + W
    np.testing.assert_array_equal(host_f64(outs["gather_buf"][0]), rows)
    ro, rl = oracle.sparse_attn(host_f64(x["q"][0]), rows, host_f64(x["sink"]), 1.0 / np.sqrt(D))
    assert rel_err(host_f64(outs["out"][0]), ro) <= 2e-2
    assert_lse_close(outs["lse"][0].cpu().numpy(), rl)


def test_decode_steps_in_sequence(csa):
    """Nine consecutive steps (two block completions, ring wrap) with the host
    counters advanced by csa_layer_advance; each step checked against the
    oracle's evolving state."""
    shape = synth.with_(synth.SHAPES["ctx8k"], ctx=600, n_comp=150, top_k=64, w=8)
    x = synth.make_decode_inputs(shape, 4001, max_comp=200)
    g = _g(4002)
    dt = torch.bfloat16
    comp = dev_bf16(x["comp_kv"]); keys = dev_bf16(x["idx_keys"]); swa = dev_bf16(x["swa"])
    mb, ib, sink = dev_f32(x["main_bias"]), dev_f32(x["idx_bias"]), dev_f32(x["sink"])
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=keys, swa=swa, main_bias=mb, idx_bias=ib, sink=sink,
                            n_comp=x["n_comp"], swa_head=x["swa_head"], swa_len=x["swa_len"], h=64, h_i=64,
                            top_k=64)
    f = numfmt.bf16_bits_to_f64
    ost = oracle.LayerState(comp_kv=f(x["comp_kv"][0]), idx_keys=f(x["idx_keys"][0]), n_comp=x["n_comp"],
                            swa=oracle.SwaRing(f(x["swa"][0]), x["swa_head"], x["swa_len"]),
                            main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"],
                            round_cache=numfmt.bf16_round_f64)
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    for pos in range(x["pos"], x["pos"] + 9):
        q = synth.to_bf16_bits(g.standard_normal((1, 64, 512), dtype=np.float32))
        qi = synth.to_bf16_bits((g.standard_normal((1, 64, 128), dtype=np.float32) / np.float32(np.sqrt(128))))
        wi = g.standard_normal((1, 64), dtype=np.float32)
        kvn = synth.to_bf16_bits(g.standard_normal((1, 512), dtype=np.float32))
        zm, cm = g.standard_normal((2, 1, 4, 512), dtype=np.float32)
        zi, ci = g.standard_normal((2, 1, 4, 128), dtype=np.float32)
        outs = dict(scores=torch.empty(1, 200, device=DEV), topk_idx=torch.empty(1, 64, dtype=torch.int32, device=DEV),
                    topk_count=torch.empty(1, dtype=torch.int32, device=DEV),
                    gather_buf=torch.zeros(1, 72, 512, dtype=dt, device=DEV),
                    n_valid=torch.empty(1, dtype=torch.int32, device=DEV),
                    out=torch.empty(1, 64, 512, dtype=dt, device=DEV))
        io = csa.make_step_io(pos=pos, q=dev_bf16(q), q_idx=dev_bf16(qi), w_idx=dev_f32(wi), kv_new=dev_bf16(kvn),
                              z_main=dev_f32(zm), c_main=dev_f32(cm), z_idx=dev_f32(zi), c_idx=dev_f32(ci), **outs)
        csa.csa_decode_step(L, io, ws)
        csa.csa_layer_advance(L, pos)
        torch.cuda.synchronize()
        completes = pos % 4 == 3
        n0 = ost.n_comp
        oracle.decode_step(ost, q=f(q[0]), q_idx=f(qi[0]), w_idx=wi[0], kv_new=f(kvn[0]), pos=pos, top_k=64,
                           z_main=zm[0], c_main=cm[0], z_idx=zi[0], c_idx=ci[0], scale=1 / np.sqrt(512))
        assert (L.n_comp, L.swa_head, L.swa_len) == (ost.n_comp, ost.swa.head, ost.swa.length)
        N = ost.n_comp
        if completes:  # new entries within one bf16 ulp of the oracle's, then adopt the GPU's bits
            assert_bf16_close(host_bits(comp[0, n0]), oracle.compress(zm[0], cm[0], x["main_bias"], 4)[0])
            assert_bf16_close(host_bits(keys[0, n0]), oracle.compress(zi[0], ci[0], x["idx_bias"], 4)[0])
        ost.comp_kv[:N] = host_f64(comp[0, :N])
        ost.idx_keys[:N] = host_f64(keys[0, :N])
        ref_s = oracle.index_score(f(qi[0])[None], wi[0][None], ost.idx_keys[:N])[0]
        got_s = outs["scores"][0, :N].cpu().numpy().astype(np.float64)
        assert rel_err(got_s, ref_s) <= 1e-4
        gi, gc = outs["topk_idx"][0].cpu().numpy(), int(outs["topk_count"][0])
        np.testing.assert_array_equal(gi, oracle.topk(got_s[None], 64)[0][0])
        assert_topk_gap_rule(gi, gc, ref_s, 64)
        rows, n_valid = oracle.gather(ost.comp_kv[:N], gi, gc, ost.swa.rows, ost.swa.head, ost.swa.length)
        assert int(outs["n_valid"][0]) == n_valid
        np.testing.assert_array_equal(host_f64(outs["gather_buf"][0, :n_valid]), rows)
        ro, _ = oracle.sparse_attn(f(q[0]), rows, x["sink"], 1 / np.sqrt(512))
        assert rel_err(host_f64(outs["out"][0]), ro) <= 2e-2


def _assert_e4m3_key_close(codes, scale, y):
    """A GPU-quantised key row (codes, scale) against the oracle's float64
    compressed key y: the scale within 1e-5 of max|y| / 448 and every element
    within half an E4M3 unit in the last place plus the float32 slack of the
    compressor (the two sides may round a boundary case differently)."""
    y = np.asarray(y, dtype=np.float64)
    assert scale == pytest.approx(np.abs(y).max() / 448, rel=1e-5)
    dec = numfmt.e4m3_decode(codes) * scale
    bound = np.maximum(np.abs(y) * 2.0 ** -4, scale * 2.0 ** -10) + 1e-5 * np.abs(y).max()
    assert (np.abs(dec - y) <= bound).all()


def _fp8_query(qi, wi):
    """E4M3 query codes and head weights with the query's per-head scales folded in."""
    qc, qs = numfmt.quantize_e4m3_rows(qi.reshape(-1, qi.shape[-1]))
    return qc.reshape(qi.shape), (wi * qs.reshape(wi.shape)).astype(np.float32)


def test_decode_steps_in_sequence_fp8_keys(csa):
    """Nine consecutive steps over E4M3 indexer keys (two block completions,
    ring wrap): each new key quantised on the GPU within E4M3 rounding of the
    oracle's, then adopted; scores against the oracle's FP8 score on the
    cache as the GPU holds it, top-k, gather and attention as for bf16 keys."""
    shape = synth.with_(synth.SHAPES["ctx8k"], ctx=600, n_comp=150, top_k=64, w=8)
    x = synth.make_decode_inputs(shape, 4101, max_comp=200)
    g = _g(4102)
    dt = torch.bfloat16
    f = numfmt.bf16_bits_to_f64
    kc0, ks0 = numfmt.quantize_e4m3_rows(f(x["idx_keys"][0]).astype(np.float32))
    comp = dev_bf16(x["comp_kv"]); swa = dev_bf16(x["swa"])
    kc = torch.from_numpy(kc0[None].copy()).to(DEV)
    ks = dev_f32(ks0[None])
    mb, ib, sink = dev_f32(x["main_bias"]), dev_f32(x["idx_bias"]), dev_f32(x["sink"])
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=kc, idx_scales=ks, swa=swa, main_bias=mb, idx_bias=ib,
                            sink=sink, n_comp=x["n_comp"], swa_head=x["swa_head"], swa_len=x["swa_len"], h=64,
                            h_i=64, top_k=64)
    assert L.idx_dtype == csa.CSA_FP8_E4M3
    ost = oracle.LayerState(comp_kv=f(x["comp_kv"][0]), idx_keys=np.zeros((200, 128)), n_comp=x["n_comp"],
                            swa=oracle.SwaRing(f(x["swa"][0]), x["swa_head"], x["swa_len"]),
                            main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"],
                            round_cache=numfmt.bf16_round_f64, idx_codes=kc0.copy(), idx_scales=ks0.copy())
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    for pos in range(x["pos"], x["pos"] + 9):
        q = synth.to_bf16_bits(g.standard_normal((1, 64, 512), dtype=np.float32))
        # the step takes the bf16 query and plain weights and quantises the query itself
        qi = synth.to_bf16_bits(g.standard_normal((1, 64, 128), dtype=np.float32) / np.float32(np.sqrt(128)))
        wi = g.standard_normal((1, 64), dtype=np.float32)
        qc, w8 = _fp8_query(f(qi).astype(np.float32), wi)
        kvn = synth.to_bf16_bits(g.standard_normal((1, 512), dtype=np.float32))
        zm, cm = g.standard_normal((2, 1, 4, 512), dtype=np.float32)
        zi, ci = g.standard_normal((2, 1, 4, 128), dtype=np.float32)
        outs = dict(scores=torch.empty(1, 200, device=DEV), topk_idx=torch.empty(1, 64, dtype=torch.int32, device=DEV),
                    topk_count=torch.empty(1, dtype=torch.int32, device=DEV),
                    gather_buf=torch.zeros(1, 72, 512, dtype=dt, device=DEV),
                    n_valid=torch.empty(1, dtype=torch.int32, device=DEV),
                    out=torch.empty(1, 64, 512, dtype=dt, device=DEV))
        io = csa.make_step_io(pos=pos, q=dev_bf16(q), q_idx=dev_bf16(qi), w_idx=dev_f32(wi),
                              kv_new=dev_bf16(kvn), z_main=dev_f32(zm), c_main=dev_f32(cm), z_idx=dev_f32(zi),
                              c_idx=dev_f32(ci), **outs)
        print(f"fp8-key step pos={pos}", flush=True)
        csa.csa_decode_step(L, io, ws)
        csa.csa_layer_advance(L, pos)
        torch.cuda.synchronize()
        completes = pos % 4 == 3
        n0 = ost.n_comp
        oracle.decode_step(ost, q=f(q[0]), q_idx=f(qi[0]), w_idx=wi[0], kv_new=f(kvn[0]), pos=pos, top_k=64,
                           z_main=zm[0], c_main=cm[0], z_idx=zi[0], c_idx=ci[0], scale=1 / np.sqrt(512))
        assert (L.n_comp, L.swa_head, L.swa_len) == (ost.n_comp, ost.swa.head, ost.swa.length)
        N = ost.n_comp
        gkc, gks = kc[0].cpu().numpy(), ks[0].cpu().numpy()
        np.testing.assert_array_equal(gkc[:n0], ost.idx_codes[:n0])   # older keys untouched
        if completes:  # the new entry and key close to the oracle's, then adopt the GPU's
            assert_bf16_close(host_bits(comp[0, n0]), oracle.compress(zm[0], cm[0], x["main_bias"], 4)[0])
            _assert_e4m3_key_close(gkc[n0], float(gks[n0]), oracle.compress(zi[0], ci[0], x["idx_bias"], 4)[0])
        ost.comp_kv[:N] = host_f64(comp[0, :N])
        ost.idx_codes[:N], ost.idx_scales[:N] = gkc[:N], gks[:N]
        ref_s = oracle.index_score_fp8(qc, w8, ost.idx_codes[:N], ost.idx_scales[:N])[0]
        got_s = outs["scores"][0, :N].cpu().numpy().astype(np.float64)
        assert rel_err(got_s, ref_s) <= 1e-4
        gi, gc = outs["topk_idx"][0].cpu().numpy(), int(outs["topk_count"][0])
        np.testing.assert_array_equal(gi, oracle.topk(got_s[None], 64)[0][0])
        assert_topk_gap_rule(gi, gc, ref_s, 64)
        rows, n_valid = oracle.gather(ost.comp_kv[:N], gi, gc, ost.swa.rows, ost.swa.head, ost.swa.length)
        assert int(outs["n_valid"][0]) == n_valid
        np.testing.assert_array_equal(host_f64(outs["gather_buf"][0, :n_valid]), rows)
        ro, _ = oracle.sparse_attn(f(q[0]), rows, x["sink"], 1 / np.sqrt(512))
        assert rel_err(host_f64(outs["out"][0]), ro) <= 2e-2


def test_decode_step_ctx1m_fp8_keys_full_size(csa):
    """One layer of the 1M-context workload with E4M3 indexer keys (the cache
    quantised on the GPU from the bf16 keys): the new key within E4M3 rounding
    of the oracle's, every score against the oracle's FP8 score, the top-k
    exact on the GPU's scores and by the gap rule on the oracle's, gather and
    attention as for bf16 keys."""
    shape = synth.SHAPES["ctx1m"]
    x = synth.make_decode_inputs_torch(shape, seed=None, device=DEV, layers=1)[0]
    B, K, W, D = shape.batch, shape.top_k, shape.w, shape.d
    n0 = x["n_comp"]
    kc = torch.zeros(B, shape.max_comp, 128, dtype=torch.uint8, device=DEV)
    ks = torch.zeros(B, shape.max_comp, dtype=torch.float32, device=DEV)
    csa.csa_quantize_fp8(x["idx_keys"][:, :n0].contiguous(), kc[:, :n0], ks[:, :n0])
    # the step quantises the bf16 query itself; the oracle's codes and folded weights from the host
    qc, w8 = _fp8_query(host_f64(x["q_idx"]).astype(np.float32), x["w_idx"].cpu().numpy())
    torch.cuda.synchronize()
    pristine = kc[0, :n0].clone()
    L = csa.make_layer_desc(comp_kv=x["comp_kv"], idx_keys=kc, idx_scales=ks, swa=x["swa"],
                            main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"],
                            n_comp=n0, swa_head=x["swa_head"], swa_len=x["swa_len"], h=shape.h,
                            h_i=shape.h_i, top_k=K)
    outs = dict(scores=torch.empty(B, shape.max_comp, device=DEV),
                topk_idx=torch.empty(B, K, dtype=torch.int32, device=DEV),
                topk_count=torch.empty(B, dtype=torch.int32, device=DEV),
                gather_buf=torch.zeros(B, K + W, D, dtype=torch.bfloat16, device=DEV),
                n_valid=torch.empty(B, dtype=torch.int32, device=DEV),
                out=torch.empty(B, shape.h, D, dtype=torch.bfloat16, device=DEV),
                lse=torch.empty(B, shape.h, device=DEV))
    io = csa.make_step_io(pos=x["pos"], q=x["q"], q_idx=x["q_idx"], w_idx=x["w_idx"], kv_new=x["kv_new"],
                          z_main=x["z_main"], c_main=x["c_main"], z_idx=x["z_idx"], c_idx=x["c_idx"], **outs)
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    csa.csa_decode_step(L, io, ws)
    torch.cuda.synchronize()
    N = shape.n_comp
    assert N == n0 + 1
    assert torch.equal(kc[0, :n0], pristine)
    yi = oracle.compress(x["z_idx"][0].cpu().numpy(), x["c_idx"][0].cpu().numpy(),
                         x["idx_bias"].cpu().numpy(), 4)[-1]
    codes, scales = kc[0, :N].cpu().numpy(), ks[0, :N].cpu().numpy()
    _assert_e4m3_key_close(codes[n0], float(scales[n0]), yi)
    ref_s = oracle.index_score_fp8(qc, w8, codes, scales)[0]
    got_s = outs["scores"][0, :N].cpu().numpy().astype(np.float64)
    assert rel_err(got_s, ref_s) <= 1e-4
    # the step's own query quantisation is the host's bit for bit: the
    # standalone FP8 scan over the host's codes and folded weights gives the
    # step's scores exactly for every key the scan covered (the new key is
    # scored apart, by the workgroup that quantised it)
    s8 = torch.empty(1, 1, N, device=DEV)
    csa.csa_index_score_fp8(torch.from_numpy(qc[None]).to(DEV), dev_f32(w8[None]), kc[:, :N], ks[:, :N], s8)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s8[0, 0, :n0].cpu().numpy().view(np.uint32),
                                  outs["scores"][0, :n0].cpu().numpy().view(np.uint32))
    assert abs(float(s8[0, 0, n0]) - got_s[n0]) <= 1e-5 * np.abs(got_s).max()
    gi = outs["topk_idx"][0].cpu().numpy()
    oi, _ = oracle.topk(got_s[None], K)
    np.testing.assert_array_equal(gi, oi[0])
    assert_topk_gap_rule(gi, int(outs["topk_count"][0]), ref_s, K)
    sel = host_f64(x["comp_kv"][0, torch.from_numpy(gi).to(DEV).long()])
    swa_rows = host_f64(x["swa"][0])
    head = (x["swa_head"] + 1) % W
    win = np.stack([swa_rows[(head - W + j) % W] for j in range(W)])
    rows = np.concatenate([sel, win])
    assert int(outs["n_valid"][0]) == K + W
    np.testing.assert_array_equal(host_f64(outs["gather_buf"][0]), rows)
    ro, rl = oracle.sparse_attn(host_f64(x["q"][0]), rows, host_f64(x["sink"]), 1.0 / np.sqrt(D))
    assert rel_err(host_f64(outs["out"][0]), ro) <= 2e-2
    assert_lse_close(outs["lse"][0].cpu().numpy(), rl)


# ---------------------------------------------------------------------------
# 6b. HCA layer step (ratio-m compressor, attention over every entry + window)
# ---------------------------------------------------------------------------

HCA_SEQ_CASES = [
    # name, ratio m, heads, entries before, cache capacity, window
    ("ratio8_h64", 8, 64, 37, 48, 8),           # one job workgroup compresses a block
    ("ratio64_h16_fold", 64, 16, 5, 40, 8),     # the block folded into the one attention workgroup
    ("ratio32_h32_fold", 32, 32, 20, 300, 16),  # folded over workgroups of empty splits too
]


@pytest.mark.parametrize("case", HCA_SEQ_CASES, ids=[c[0] for c in HCA_SEQ_CASES])
def test_hca_steps_in_sequence(csa, case):
    """Twenty HCA steps (block completions, ring wrap) with the host counters
    advanced by csa_layer_advance; each step against the oracle's evolving
    state."""
    name, m, H, n0, max_comp, W = case
    D = 512
    g = _g(6001 + m)
    pos0 = n0 * m + (5 if m == 8 else m - 10)
    comp = dev_bf16(synth.to_bf16_bits(g.standard_normal((1, max_comp, D), dtype=np.float32)))
    swa = dev_bf16(synth.to_bf16_bits(g.standard_normal((1, W, D), dtype=np.float32)))
    mb = dev_f32(g.standard_normal((m, D), dtype=np.float32) * np.float32(0.1))
    sink = dev_f32(g.standard_normal(H, dtype=np.float32))
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=None, swa=swa, main_bias=mb, idx_bias=None, sink=sink,
                            n_comp=n0, swa_head=pos0 % W, swa_len=W, h=H, h_i=0, m=m, top_k=0)
    f = numfmt.bf16_bits_to_f64
    ost = oracle.LayerState(comp_kv=host_f64(comp[0]), idx_keys=np.zeros((max_comp, 1)), n_comp=n0,
                            swa=oracle.SwaRing(host_f64(swa[0]), pos0 % W, W), main_bias=host_f64(mb),
                            idx_bias=np.zeros((m, 1)), sink=host_f64(sink), m=m, round_cache=numfmt.bf16_round_f64)
    ws = torch.empty(csa.csa_hca_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    for pos in range(pos0, pos0 + 20):
        q = synth.to_bf16_bits(g.standard_normal((1, H, D), dtype=np.float32))
        kvn = synth.to_bf16_bits(g.standard_normal((1, D), dtype=np.float32))
        zm, cm = g.standard_normal((2, 1, m, D), dtype=np.float32)
        out = torch.empty(1, H, D, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty(1, H, device=DEV)
        n_valid = torch.empty(1, dtype=torch.int32, device=DEV)
        io = csa.make_step_io(pos=pos, q=dev_bf16(q), kv_new=dev_bf16(kvn), z_main=dev_f32(zm), c_main=dev_f32(cm),
                              out=out, lse=lse, n_valid=n_valid)
        csa.csa_hca_decode_step(L, io, ws)
        csa.csa_layer_advance(L, pos)
        torch.cuda.synchronize()
        nprev = ost.n_comp
        r = oracle.hca_decode_step(ost, q=f(q[0]), kv_new=f(kvn[0]), pos=pos, z_main=zm[0], c_main=cm[0],
                                   scale=1 / np.sqrt(D))
        assert (L.n_comp, L.swa_head, L.swa_len) == (ost.n_comp, ost.swa.head, ost.swa.length)
        if pos % m == m - 1:  # the new entry within one bf16 ulp, then adopt the GPU's bits
            assert_bf16_close(host_bits(comp[0, nprev]), oracle.compress(zm[0], cm[0], host_f64(mb), m)[0])
            ost.comp_kv[nprev] = host_f64(comp[0, nprev])
            r = oracle.sparse_attn(f(q[0]), np.concatenate([ost.comp_kv[:ost.n_comp], r["rows"][ost.n_comp:]]),
                                   host_f64(sink), 1 / np.sqrt(D))
            r = {"out": r[0], "lse": r[1], "n_valid": ost.n_comp + ost.swa.length}
        assert int(n_valid[0]) == r["n_valid"]
        assert rel_err(host_f64(out[0]), r["out"]) <= 2e-2
        assert_lse_close(lse[0].cpu().numpy(), r["lse"])


def test_hca_step_full_size(csa):
    """HCA at 1M context (ratio 128: 7812 entries + the one this step
    completes, window 128 with wrap), one layer, against the oracle over all
    7941 rows."""
    shape = synth.SHAPES["hca1m"]
    x = synth.make_decode_inputs_torch(shape, seed=None, device=DEV, layers=1)[0]
    H, D, W = shape.h, shape.d, shape.w
    L = csa.make_layer_desc(comp_kv=x["comp_kv"], idx_keys=None, swa=x["swa"], main_bias=x["main_bias"],
                            idx_bias=None, sink=x["sink"], n_comp=x["n_comp"], swa_head=x["swa_head"],
                            swa_len=x["swa_len"], h=H, h_i=0, m=shape.m, top_k=0)
    out = torch.empty(1, H, D, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(1, H, device=DEV)
    io = csa.make_step_io(pos=x["pos"], q=x["q"], kv_new=x["kv_new"], z_main=x["z_main"], c_main=x["c_main"],
                          out=out, lse=lse)
    ws = torch.empty(csa.csa_hca_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    csa.csa_hca_decode_step(L, io, ws)
    torch.cuda.synchronize()
    N = x["n_comp"] + 1
    assert N == shape.n_comp
    assert_bf16_close(host_bits(x["comp_kv"][0, N - 1]),
                      oracle.compress(host_f64(x["z_main"][0]), host_f64(x["c_main"][0]), host_f64(x["main_bias"]),
                                      shape.m)[0])
    head = (x["swa_head"] + 1) % W
    swa = host_f64(x["swa"][0])
    win = np.stack([swa[(head - W + j) % W] for j in range(W)])
    rows = np.concatenate([host_f64(x["comp_kv"][0, :N]), win])
    ro, rl = oracle.sparse_attn(host_f64(x["q"][0]), rows, host_f64(x["sink"]), 1 / np.sqrt(D))
    assert rel_err(host_f64(out[0]), ro) <= 2e-2
    assert_lse_close(lse[0].cpu().numpy(), rl)


def test_read_probe_runs(csa):
    """The calibration read (csa_read_probe) runs over a buffer with a ragged
    tail and leaves the sink alone for data whose xor is not its marker."""
    buf = torch.zeros(1_000_003 * 4, dtype=torch.uint8, device=DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=DEV)
    csa.csa_read_probe(buf, sink)
    torch.cuda.synchronize()
    assert int(sink[0]) == 0


def test_fp8_scans_decode_every_code_pair(csa):
    """Both FP8 scans (one query row per sequence; many rows per call) read
    their operands as OCP E4M3, subnormals included: query row i holds only
    finite code i in one byte of head 0 and its negation in head 1, key j only
    finite code j in the same byte, so with weights (1, 2) and unit key
    scales the score is the exact product p = e4m3(i) e4m3(j) when p > 0 and
    2|p| otherwise — compared bit for bit for all 254 x 254 pairs."""
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    n = len(codes)
    slot = 77  # any byte of the 128
    q = np.zeros((n, 64, 128), dtype=np.uint8)
    q[:, 0, slot] = codes
    q[:, 1, slot] = codes ^ 0x80
    k = np.zeros((n, 128), dtype=np.uint8)
    k[:, slot] = codes
    w = np.zeros((n, 64), dtype=np.float32)
    w[:, 0], w[:, 1] = 1.0, 2.0
    p = numfmt.e4m3_decode(codes)[:, None] * numfmt.e4m3_decode(codes)[None, :]
    want = np.where(p > 0, p, -2.0 * p)
    kd, ks = torch.from_numpy(k).to(DEV), torch.ones(n, device=DEV)
    # many query rows in one call (the multi-query scan)
    s1 = torch.empty(1, n, n, device=DEV)
    csa.csa_index_score_fp8(torch.from_numpy(q[None]).to(DEV), dev_f32(w[None]), kd[None], ks[None], s1)
    # one query row per sequence (the decode scan), keys shared
    s2 = torch.empty(n, 1, n, device=DEV)
    csa.csa_index_score_fp8(torch.from_numpy(q[:, None]).to(DEV), dev_f32(w[:, None]), kd[None].expand(n, n, 128),
                            ks[None].expand(n, n), s2)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s1[0].cpu().numpy().astype(np.float64), want)
    np.testing.assert_array_equal(s2[:, 0].cpu().numpy().astype(np.float64), want)


SPLIT_CASES = [
    # name, shape, fp8 keys
    ("ctx8k_bf16", synth.with_(synth.SHAPES["ctx8k"], n_comp=2048, ctx=8192), False),
    ("batch5_split_topk", synth.with_(synth.SHAPES["ctx8k"], batch=5, n_comp=3000, ctx=12000), False),
    ("tiny_f32", synth.SHAPES["tiny"], False),
    ("ctx8k_fp8_keys", synth.with_(synth.SHAPES["ctx8k"], n_comp=2048, ctx=8192), True),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_decode_step_two_calls_equal_one(csa, case):
    """csa_decode_step_scan then csa_decode_step_attend (the step's two parts,
    on one stream, one workspace) give bit for bit what csa_decode_step
    gives: scores, top-k, gather_buf, output, lse and the cache writes."""
    name, shape, fp8 = case
    x = synth.make_decode_inputs(shape, 9301 + len(name))
    B, K, W, D = shape.batch, shape.top_k, shape.w, shape.d
    res = []
    for split in (False, True):
        st = dev_store
        comp, swa = st(x["comp_kv"]), st(x["swa"])
        if fp8:
            kc, ks = numfmt.quantize_e4m3_rows(as_f64(x["idx_keys"]).reshape(-1, shape.d_i).astype(np.float32))
            keys = torch.from_numpy(kc.reshape(B, -1, shape.d_i)).to(DEV)
            scales = dev_f32(ks.reshape(B, -1))
        else:
            keys, scales = st(x["idx_keys"]), None
        L = csa.make_layer_desc(comp_kv=comp, idx_keys=keys, idx_scales=scales, swa=swa,
                                main_bias=dev_f32(x["main_bias"]), idx_bias=dev_f32(x["idx_bias"]),
                                sink=dev_f32(x["sink"]), n_comp=x["n_comp"], swa_head=x["swa_head"],
                                swa_len=x["swa_len"], h=shape.h, h_i=shape.h_i, top_k=K)
        dt = torch.float32 if shape.dtype == "f32" else torch.bfloat16
        outs = dict(scores=torch.full((B, shape.max_comp), 5.0, device=DEV),
                    topk_idx=torch.full((B, K), -3, dtype=torch.int32, device=DEV),
                    topk_count=torch.full((B,), -3, dtype=torch.int32, device=DEV),
                    gather_buf=torch.zeros(B, K + W, D, dtype=dt, device=DEV),
                    n_valid=torch.full((B,), -3, dtype=torch.int32, device=DEV),
                    out=torch.zeros(B, shape.h, D, dtype=dt, device=DEV), lse=torch.zeros(B, shape.h, device=DEV))
        io = csa.make_step_io(pos=x["pos"], q=st(x["q"]), q_idx=st(x["q_idx"]), w_idx=dev_f32(x["w_idx"]),
                              kv_new=st(x["kv_new"]), z_main=dev_f32(x["z_main"]), c_main=dev_f32(x["c_main"]),
                              z_idx=dev_f32(x["z_idx"]), c_idx=dev_f32(x["c_idx"]), **outs)
        ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
        print(f"two-call step {name}: split={split}", flush=True)
        if split:
            csa.csa_decode_step_scan(L, io, ws)
            csa.csa_decode_step_attend(L, io, ws)
        else:
            csa.csa_decode_step(L, io, ws)
        torch.cuda.synchronize()
        res.append((outs, comp, keys, scales, swa))
    (o1, *c1), (o2, *c2) = res
    N = shape.n_comp
    assert torch.equal(o1["scores"][:, :N], o2["scores"][:, :N])
    for k in ("topk_idx", "topk_count", "n_valid", "out", "lse"):
        assert torch.equal(o1[k], o2[k]), k
    nv = int(o1["n_valid"].min())
    assert nv == min(K, N) + W
    assert torch.equal(o1["gather_buf"][:, :nv], o2["gather_buf"][:, :nv])
    for a, b in zip(c1, c2):
        if a is not None:
            assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# E4M3 keys with the two-stage selection (E4M3 top-k_cand, then exact top-k)
# ---------------------------------------------------------------------------

def _rescored_layer(csa, x, B, max_comp, K, kc):
    f = numfmt.bf16_bits_to_f64
    kc0, ks0 = numfmt.quantize_e4m3_rows(f(x["idx_keys"]).reshape(-1, 128).astype(np.float32))
    codes = torch.from_numpy(kc0.reshape(B, max_comp, 128)).to(DEV)
    scales = dev_f32(ks0.reshape(B, max_comp))
    exact_keys = dev_bf16(x["idx_keys"])
    comp, swa = dev_bf16(x["comp_kv"]), dev_bf16(x["swa"])
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=codes, idx_scales=scales, swa=swa,
                            main_bias=dev_f32(x["main_bias"]), idx_bias=dev_f32(x["idx_bias"]),
                            sink=dev_f32(x["sink"]), n_comp=x["n_comp"], swa_head=x["swa_head"],
                            swa_len=x["swa_len"], h=64, h_i=64, top_k=K, idx_keys_exact=exact_keys,
                            idx_rescore=kc)
    return L, codes, scales, exact_keys, comp, swa


def _check_rescored_selection(csa, qi_dev, wi_dev, exact_keys, N, got_s8, gi, gc, exact_ref, K, kc, b=0):
    """The selection of the two-stage step: bit for bit the oracle's two
    stages applied to the GPU's own E4M3 scores and to the bfloat16 scan's
    scores (which the rescoring reproduces exactly); and by the gap rule
    against the float64 exact scores inside the first stage's set."""
    s16 = torch.empty(1, 1, N, device=DEV)
    csa.csa_index_score(qi_dev[b:b + 1, None].contiguous(), wi_dev[b:b + 1, None].contiguous(),
                        exact_keys[b:b + 1, :N].contiguous(), s16)
    torch.cuda.synchronize()
    s16 = s16[0, 0].cpu().numpy().astype(np.float64)
    want, wc = oracle.rescored_topk(got_s8[None], s16[None], K, kc)
    np.testing.assert_array_equal(gi, want[0])
    assert gc == wc[0]
    stage1 = oracle.topk(got_s8[None], kc)[0][0]
    inside = np.full(N, -np.inf)
    inside[stage1[stage1 >= 0]] = exact_ref[stage1[stage1 >= 0]]
    assert_topk_gap_rule(gi, gc, inside, K)


@pytest.mark.parametrize("B", [1, 5])
def test_decode_steps_in_sequence_fp8_rescored(csa, B):
    """Steps over E4M3 keys with the two-stage selection (top_k 64 out of the
    E4M3 best 128, two block completions; batch 5 takes the separate top-k):
    new key in both forms within rounding of the oracle's, then adopted;
    E4M3 scores against the oracle; the selection exactly as above; gather
    and attention against the oracle."""
    K, kc, W = 64, 128, 8
    shape = synth.with_(synth.SHAPES["ctx8k"], batch=B, ctx=12000, n_comp=3000, top_k=K, w=W)
    x = synth.make_decode_inputs(shape, 4201 + B, max_comp=3100)
    g = _g(4202 + B)
    f = numfmt.bf16_bits_to_f64
    L, codes, scales, exact_keys, comp, swa = _rescored_layer(csa, x, B, 3100, K, kc)
    osts = []
    for b in range(B):
        kc0, ks0 = codes[b].cpu().numpy(), scales[b].cpu().numpy()
        osts.append(oracle.LayerState(comp_kv=f(x["comp_kv"][b]), idx_keys=f(x["idx_keys"][b]), n_comp=x["n_comp"],
                                      swa=oracle.SwaRing(f(x["swa"][b]), x["swa_head"], x["swa_len"]),
                                      main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"],
                                      round_cache=numfmt.bf16_round_f64, idx_codes=kc0.copy(), idx_scales=ks0.copy(),
                                      fp8_rescore=kc))
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    for pos in range(x["pos"], x["pos"] + 6):
        q = synth.to_bf16_bits(g.standard_normal((B, 64, 512), dtype=np.float32))
        qi = synth.to_bf16_bits(g.standard_normal((B, 64, 128), dtype=np.float32) / np.float32(np.sqrt(128)))
        wi = g.standard_normal((B, 64), dtype=np.float32)
        kvn = synth.to_bf16_bits(g.standard_normal((B, 512), dtype=np.float32))
        zm, cm = g.standard_normal((2, B, 4, 512), dtype=np.float32)
        zi, ci = g.standard_normal((2, B, 4, 128), dtype=np.float32)
        outs = dict(scores=torch.empty(B, 3100, device=DEV), topk_idx=torch.empty(B, K, dtype=torch.int32, device=DEV),
                    topk_count=torch.empty(B, dtype=torch.int32, device=DEV),
                    gather_buf=torch.zeros(B, K + W, 512, dtype=torch.bfloat16, device=DEV),
                    n_valid=torch.empty(B, dtype=torch.int32, device=DEV),
                    out=torch.empty(B, 64, 512, dtype=torch.bfloat16, device=DEV), lse=torch.empty(B, 64, device=DEV))
        qi_dev, wi_dev = dev_bf16(qi), dev_f32(wi)
        io = csa.make_step_io(pos=pos, q=dev_bf16(q), q_idx=qi_dev, w_idx=wi_dev, kv_new=dev_bf16(kvn),
                              z_main=dev_f32(zm), c_main=dev_f32(cm), z_idx=dev_f32(zi), c_idx=dev_f32(ci), **outs)
        print(f"rescored fp8-key step pos={pos} B={B}", flush=True)
        csa.csa_decode_step(L, io, ws)
        csa.csa_layer_advance(L, pos)
        torch.cuda.synchronize()
        completes = pos % 4 == 3
        for b in range(B):
            ost = osts[b]
            n0 = ost.n_comp
            oracle.decode_step(ost, q=f(q[b]), q_idx=f(qi[b]), w_idx=wi[b], kv_new=f(kvn[b]), pos=pos, top_k=K,
                               z_main=zm[b], c_main=cm[b], z_idx=zi[b], c_idx=ci[b], scale=1 / np.sqrt(512))
            N = ost.n_comp
            assert L.n_comp == N
            if completes:
                yi = oracle.compress(zi[b], ci[b], x["idx_bias"], 4)[0]
                _assert_e4m3_key_close(codes[b, n0].cpu().numpy(), float(scales[b, n0]), yi)
                assert_bf16_close(host_bits(exact_keys[b, n0]), yi)
                assert_bf16_close(host_bits(comp[b, n0]), oracle.compress(zm[b], cm[b], x["main_bias"], 4)[0])
            ost.comp_kv[:N] = host_f64(comp[b, :N])
            ost.idx_keys[:N] = host_f64(exact_keys[b, :N])
            ost.idx_codes[:N], ost.idx_scales[:N] = codes[b, :N].cpu().numpy(), scales[b, :N].cpu().numpy()
            qc, w8 = _fp8_query(f(qi[b:b + 1]).astype(np.float32), wi[b:b + 1])
            ref_s8 = oracle.index_score_fp8(qc, w8, ost.idx_codes[:N], ost.idx_scales[:N])[0]
            got_s8 = outs["scores"][b, :N].cpu().numpy().astype(np.float64)
            assert rel_err(got_s8, ref_s8) <= 1e-4
            exact_ref = oracle.index_score(f(qi[b])[None], wi[b][None].astype(np.float64), ost.idx_keys[:N])[0]
            gi, gc = outs["topk_idx"][b].cpu().numpy(), int(outs["topk_count"][b])
            _check_rescored_selection(csa, qi_dev, wi_dev, exact_keys, N, got_s8, gi, gc, exact_ref, K, kc, b)
            rows, n_valid = oracle.gather(ost.comp_kv[:N], gi, gc, ost.swa.rows, ost.swa.head, ost.swa.length)
            assert int(outs["n_valid"][b]) == n_valid
            np.testing.assert_array_equal(host_f64(outs["gather_buf"][b, :n_valid]), rows)
            ro, rl = oracle.sparse_attn(f(q[b]), rows, x["sink"], 1 / np.sqrt(512))
            assert rel_err(host_f64(outs["out"][b]), ro) <= 2e-2
            assert rel_err(outs["lse"][b].cpu().numpy(), rl) <= 2e-2


def test_decode_step_ctx1m_fp8_rescored_full_size_recall(csa):
    """One 1M-context layer over E4M3 keys with the two-stage selection
    (top-512 of the E4M3 best 1024): the selection exactly as the oracle's
    two stages on the GPU's scores, and top-512 recall against the float64
    exact indexer of at least 0.99 (the gate of page 1,
    ARCHITECTURE_AND_MEMORY_AUDIT.md, Tier 1 gate 4)."""
    shape = synth.SHAPES["ctx1m"]
    x = synth.make_decode_inputs_torch(shape, seed=None, device=DEV, layers=1)[0]
    B, K, W, D, kc = 1, shape.top_k, shape.w, shape.d, 2 * shape.top_k
    n0 = x["n_comp"]
    codes = torch.zeros(B, shape.max_comp, 128, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, shape.max_comp, dtype=torch.float32, device=DEV)
    csa.csa_quantize_fp8(x["idx_keys"][:, :n0].contiguous(), codes[:, :n0], scales[:, :n0])
    exact_keys = x["idx_keys"]
    L = csa.make_layer_desc(comp_kv=x["comp_kv"], idx_keys=codes, idx_scales=scales, swa=x["swa"],
                            main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"], n_comp=n0,
                            swa_head=x["swa_head"], swa_len=x["swa_len"], h=shape.h, h_i=shape.h_i, top_k=K,
                            idx_keys_exact=exact_keys, idx_rescore=kc)
    outs = dict(scores=torch.empty(B, shape.max_comp, device=DEV),
                topk_idx=torch.empty(B, K, dtype=torch.int32, device=DEV),
                topk_count=torch.empty(B, dtype=torch.int32, device=DEV),
                gather_buf=torch.zeros(B, K + W, D, dtype=torch.bfloat16, device=DEV),
                n_valid=torch.empty(B, dtype=torch.int32, device=DEV),
                out=torch.empty(B, shape.h, D, dtype=torch.bfloat16, device=DEV),
                lse=torch.empty(B, shape.h, device=DEV))
    io = csa.make_step_io(pos=x["pos"], q=x["q"], q_idx=x["q_idx"], w_idx=x["w_idx"], kv_new=x["kv_new"],
                          z_main=x["z_main"], c_main=x["c_main"], z_idx=x["z_idx"], c_idx=x["c_idx"], **outs)
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    csa.csa_decode_step(L, io, ws)
    torch.cuda.synchronize()
    N = shape.n_comp
    got_s8 = outs["scores"][0, :N].cpu().numpy().astype(np.float64)
    exact_ref = oracle.index_score(host_f64(x["q_idx"][0])[None], x["w_idx"][0].cpu().numpy()[None].astype(np.float64),
                                   host_f64(exact_keys[0, :N]))[0]
    gi, gc = outs["topk_idx"][0].cpu().numpy(), int(outs["topk_count"][0])
    _check_rescored_selection(csa, x["q_idx"], x["w_idx"], exact_keys, N, got_s8, gi, gc, exact_ref, K, kc)
    ref = set(oracle.topk(exact_ref[None], K)[0][0].tolist())
    recall = len(ref & set(gi.tolist())) / K
    plain = len(ref & set(oracle.topk(got_s8[None], K)[0][0].tolist())) / K
    print(f"top-512 recall at n=250000: two-stage {recall:.4f}, E4M3 alone {plain:.4f}")
    assert recall >= 0.99
    sel = host_f64(x["comp_kv"][0, torch.from_numpy(gi).to(DEV).long()])
    nv = int(outs["n_valid"][0])
    np.testing.assert_array_equal(host_f64(outs["gather_buf"][0, :gc]), sel)
    assert nv == gc + W
