"""GPU parity of the prefill chunk's selection over FP4 keys (E2M1 with E8M0
block scales; page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, C4, block format per
reading R30) against the float64 oracle: the multi-query FP4 scan, the
chunked top-k over it, and the two-stage selection that restores recall.

Tolerances as the E4M3 chunk tests: scores within 1e-4 (max |diff| / max
|oracle|), selections bit for bit against the oracle applied to the GPU's
own scan scores and by the gap rule against the oracle's scores.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import numfmt
from tests.gpu_util import DEV, assert_topk_gap_rule, dev_bf16, dev_f32, host_f64, rel_err
from tests.test_gpu_prefill import TOPK_CASES, _visible

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import compressed_sparse_attention_reduce_amd as pkg
    pkg.lib()
    return pkg


def _g(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _fp4(g, shape_q, n):
    """E4M3 query (per head row, scales folded into w) and MXFP4 keys, by
    the oracle's quantisers; keys also returned unpacked for the oracle."""
    q = (g.standard_normal(shape_q) / np.sqrt(128)).astype(np.float32)
    w = g.standard_normal(shape_q[:-1]).astype(np.float32)
    K = g.standard_normal((n, 128)).astype(np.float32)
    qc, qs = numfmt.quantize_e4m3_rows(q.reshape(-1, 128))
    if n:
        kc, ks = numfmt.quantize_mxfp4_rows(K)
    else:
        kc, ks = np.zeros((0, 128), np.uint8), np.zeros((0, 4), np.uint8)
    return qc.reshape(shape_q), (w * qs.reshape(w.shape)).astype(np.float32), kc, ks


def _dev4(kc, ks):
    return torch.from_numpy(numfmt.pack_e2m1(kc)).to(DEV), torch.from_numpy(np.ascontiguousarray(ks)).to(DEV)


MQ4_CASES = [
    # name, B, t, n, causal
    ("mq4_causal_ragged_batch2", 2, 37, 1000, True),
    ("mq4_16_rows_31_keys", 1, 16, 31, False),
    ("mq4_70_rows_4111_keys", 1, 70, 4111, True),
    ("mq4_one_key", 3, 17, 1, False),
    ("mq4_300_rows_2049_keys", 1, 300, 2049, True),
]


@pytest.mark.parametrize("case", MQ4_CASES, ids=[c[0] for c in MQ4_CASES])
def test_multi_query_score_fp4(csa, case):
    """From 16 query rows per sequence csa_index_score_fp4 runs the
    multi-query kernel (the chunk's scan)."""
    name, B, t, n, causal = case
    g = _g(t * 1000 + n + 9)
    qc, w, kc, ks = _fp4(g, (B, t, 64, 128), B * n)
    kc, ks = kc.reshape(B, n, 128), ks.reshape(B, n, 4)
    ld = n + 3
    scores = torch.full((B, t, ld), 123.0, device=DEV)
    pos_np = None
    if causal:
        pos_np = (4 * n - 2 * t - 9 + 2 * np.arange(B * t)).astype(np.int32).reshape(B, t)
    kd, sd = _dev4(kc, ks)
    print(f"multi-query fp4 score {name}", flush=True)
    csa.csa_index_score_fp4(torch.from_numpy(qc).to(DEV), dev_f32(w), kd, sd, scores,
                            q_pos=None if pos_np is None else torch.from_numpy(pos_np).to(DEV))
    torch.cuda.synchronize()
    got = scores.cpu().numpy().astype(np.float64)
    assert (got[:, :, n:] == 123.0).all(), "wrote past n"
    for b in range(B):
        ref = oracle.index_score_fp4(qc[b], w[b], kc[b], ks[b], q_pos=None if pos_np is None else pos_np[b])
        fin = np.isfinite(ref)
        assert (np.isfinite(got[b, :, :n]) == fin).all(), "mask differs"
        assert rel_err(got[b, :, :n][fin], ref[fin]) <= 1e-4


def test_multi_query_fp4_decodes_every_code_and_scale(csa):
    """The multi-query kernel's operand order: 32 query rows, key j holding
    one nonzero element (code c at element e with block scale s, c over the
    16 codes, s over 60 .. 194, e over every element), head 0 of every row
    1.0 everywhere and head 1 -1.0 with weights (1, 2): every score one exact
    product, compared bit for bit."""
    g = _g(5400)
    cs, ss = np.meshgrid(np.arange(16), np.arange(60, 195), indexing="ij")
    cs, ss = cs.ravel(), ss.ravel()
    n = cs.size
    e = np.arange(n) % 128
    codes = np.zeros((n, 128), dtype=np.uint8)
    codes[np.arange(n), e] = cs
    scales = g.integers(60, 195, size=(n, 4)).astype(np.uint8)
    scales[np.arange(n), e // 32] = ss
    t = 32
    q = np.zeros((1, t, 64, 128), dtype=np.uint8)
    q[0, :, 0, :] = 0x38
    q[0, :, 1, :] = 0xB8
    w = np.zeros((1, t, 64), dtype=np.float32)
    w[0, :, 0], w[0, :, 1] = 1.0, 2.0
    v = numfmt.e2m1_decode(cs.astype(np.uint8)) * np.ldexp(1.0, ss - 127)
    want = np.where(v > 0, v, -2.0 * v)
    s = torch.empty(1, t, n, device=DEV)
    kd, sd = _dev4(codes, scales)
    csa.csa_index_score_fp4(torch.from_numpy(q).to(DEV), dev_f32(w), kd[None], sd[None], s)
    torch.cuda.synchronize()
    got = s[0].cpu().numpy().astype(np.float64)
    for r in (0, 1, t - 1):
        np.testing.assert_array_equal(got[r], want)


def _run_index_topk_fp4(csa, qc, w8, kd, sd, k, pos0, n=None):
    t = qc.shape[0]
    n = kd.shape[0] if n is None else n
    idx = torch.full((t, k), -5, dtype=torch.int32, device=DEV)
    cnt = torch.full((t,), -5, dtype=torch.int32, device=DEV)
    ws = torch.empty(max(csa.csa_index_topk_workspace_size(t, n, k), 16), dtype=torch.uint8, device=DEV)
    ws.fill_(0xCD)
    csa.csa_index_topk_fp4(qc, w8, kd, sd, idx, cnt, ws, pos0=pos0, n=n)
    return idx, cnt


@pytest.mark.parametrize("case", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_index_topk_fp4(csa, case):
    """Top-k over the FP4 chunk scan: bit-exact against the oracle's top-k of
    the same scan's scores, the gap rule against the oracle's FP4 scores."""
    name, t, n, k, pos0 = case
    g = _g(t + 7 * n + k + 3)
    qn, wn, kn, ksn = _fp4(g, (t, 64, 128), n)
    qc, w8 = torch.from_numpy(qn).to(DEV), dev_f32(wn)
    kd, sd = _dev4(kn, ksn)
    print(f"fp4 chunk top-k {name}", flush=True)
    idx, cnt = _run_index_topk_fp4(csa, qc, w8, kd, sd, k, pos0)
    scores = torch.empty(1, t, n, device=DEV)
    pos = None
    if pos0 >= 0:
        pos = torch.arange(pos0, pos0 + t, dtype=torch.int32, device=DEV)[None]
    assert t >= 16  # the standalone call takes the multi-query kernel too
    csa.csa_index_score_fp4(qc[None], w8[None], kd[None], sd[None], scores, q_pos=pos)
    torch.cuda.synchronize()
    gs = scores[0].cpu().numpy().astype(np.float64)
    ri, rc = oracle.topk(gs, k)
    np.testing.assert_array_equal(idx.cpu().numpy(), ri)
    np.testing.assert_array_equal(cnt.cpu().numpy(), rc)
    if pos0 >= 0:
        np.testing.assert_array_equal(rc, np.minimum(k, _visible(pos0 + np.arange(t), n)))
    rows = sorted({0, t // 2, t - 1})
    ref = oracle.index_score_fp4(qn[rows], wn[rows], kn, ksn, q_pos=None if pos0 < 0 else pos0 + np.array(rows))
    for i, r in enumerate(rows):
        assert_topk_gap_rule(idx[r].cpu().numpy(), int(cnt[r]), ref[i], k)


def test_index_topk_fp4_empty_history(csa):
    g = _g(17)
    qn, wn, _, _ = _fp4(g, (16, 64, 128), 0)
    kd = torch.empty(0, 64, dtype=torch.uint8, device=DEV)
    sd = torch.empty(0, 4, dtype=torch.uint8, device=DEV)
    idx, cnt = _run_index_topk_fp4(csa, torch.from_numpy(qn).to(DEV), dev_f32(wn), kd, sd, 8, 0)
    torch.cuda.synchronize()
    assert (idx == -1).all() and (cnt == 0).all()


RESCORED_CASES = [
    # name, t, n, k, k_cand, pos0
    ("two_chunks_causal", 300, 5000, 64, 256, 4 * 5000 - 400),
    ("fewer_visible_than_cand", 40, 1000, 32, 128, 4 * 30),
    ("no_mask_k_equal_cand", 20, 3000, 100, 100, -1),
    ("ragged_chunk_k512", 270, 9000, 512, 2048, -1),
]


def _rescored_inputs(g, t, n):
    f = numfmt.bf16_bits_to_f64
    q = synth.to_bf16_bits((g.standard_normal((t, 64, 128)) / np.sqrt(128)).astype(np.float32))
    w = g.standard_normal((t, 64)).astype(np.float32)
    K = synth.to_bf16_bits(g.standard_normal((n, 128)).astype(np.float32))
    kc, ks = numfmt.quantize_mxfp4_rows(f(K).astype(np.float32))
    qc, qs = numfmt.quantize_e4m3_rows(f(q).reshape(-1, 128).astype(np.float32))
    return q, w, K, kc, ks, qc.reshape(t, 64, 128), (w * qs.reshape(t, 64)).astype(np.float32)


def _check_rescored_rows(csa, rows, qd, wd, k16, kd, sd, qc, w8, pos0, n, k, kcand, gi, gc, exact_rows):
    """Rows of the two-stage chunk selection: bit for bit the oracle's two
    stages over the GPU's FP4 and bf16 scan scores of those rows (at least 16
    rows per call, so the FP4 scores come from the chunk's multi-query
    kernel); the gap rule against the float64 exact scores inside the first
    stage's set."""
    ext = list(rows) + [r for r in range(qc.shape[0]) if r not in rows][:max(0, 16 - len(rows))]
    sel = torch.tensor(ext, device=DEV)
    pos = None if pos0 < 0 else torch.from_numpy((pos0 + np.asarray(ext)).astype(np.int32)).to(DEV)[None]
    s4 = torch.empty(1, len(ext), n, device=DEV)
    s16 = torch.empty(1, len(ext), n, device=DEV)
    csa.csa_index_score_fp4(torch.from_numpy(qc[ext]).to(DEV)[None], dev_f32(w8[ext])[None], kd[None], sd[None], s4,
                            q_pos=pos)
    csa.csa_index_score(qd[sel][None], wd[sel][None], k16[None], s16, q_pos=pos)
    torch.cuda.synchronize()
    s4 = s4[0, :len(rows)].cpu().numpy().astype(np.float64)
    s16 = s16[0, :len(rows)].cpu().numpy().astype(np.float64)
    want, wc = oracle.rescored_topk(s4, s16, k, kcand)
    np.testing.assert_array_equal(gi[rows], want)
    np.testing.assert_array_equal(gc[rows], wc)
    for i, r in enumerate(rows):
        stage1 = oracle.topk(s4[i][None], kcand)[0][0]
        stage1 = stage1[stage1 >= 0]
        inside = np.full(n, -np.inf)
        inside[stage1] = exact_rows[i][stage1]
        assert_topk_gap_rule(gi[r], int(gc[r]), inside, k)


@pytest.mark.parametrize("case", RESCORED_CASES, ids=[c[0] for c in RESCORED_CASES])
def test_index_topk_fp4_rescored(csa, case):
    name, t, n, k, kcand, pos0 = case
    g = _g(t * 5 + n + k + kcand)
    q, w, K, kcn, ksn, qc, w8 = _rescored_inputs(g, t, n)
    qd, wd, k16 = dev_bf16(q), dev_f32(w), dev_bf16(K)
    kd, sd = _dev4(kcn, ksn)
    idx = torch.full((t, k), -5, dtype=torch.int32, device=DEV)
    cnt = torch.full((t,), -5, dtype=torch.int32, device=DEV)
    ws = torch.empty(csa.csa_index_topk_fp8_rescored_workspace_size(t, n, k, kcand), dtype=torch.uint8, device=DEV)
    ws.fill_(0xCD)
    print(f"fp4 rescored chunk {name}", flush=True)
    csa.csa_index_topk_fp4_rescored(qd, wd, kd, sd, k16, idx, cnt, ws, kcand, pos0=pos0)
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
    _check_rescored_rows(csa, rows, qd, wd, k16, kd, sd, qc, w8, pos0, n, k, kcand, gi, gc, exact)


def test_prefill_fp4_rescored_full_size_recall(csa):
    """The 2048 x 65536 chunk over FP4 keys with the two-stage selection
    (top-512 of the FP4 best 2048): sampled rows' selection exactly the
    oracle's two stages, and top-512 recall against the float64 exact
    indexer of at least 0.99 on each sampled row (page 1,
    ARCHITECTURE_AND_MEMORY_AUDIT.md, Tier 1 gate 4)."""
    shape = synth.SHAPES["prefill"]
    x = synth.make_prefill_inputs_torch(shape, None, DEV)
    T, N, k, kcand = shape.t, shape.n_comp, shape.top_k, 4 * shape.top_k
    kd = torch.empty(N, 64, dtype=torch.uint8, device=DEV)
    sd = torch.empty(N, 4, dtype=torch.uint8, device=DEV)
    csa.csa_quantize_fp4(x["idx_keys"], kd, sd)
    idx = torch.empty(T, k, dtype=torch.int32, device=DEV)
    cnt = torch.empty(T, dtype=torch.int32, device=DEV)
    ws = torch.empty(csa.csa_index_topk_fp8_rescored_workspace_size(T, N, k, kcand), dtype=torch.uint8, device=DEV)
    print("fp4 rescored prefill chunk, full size", flush=True)
    csa.csa_index_topk_fp4_rescored(x["q_idx"], x["w_idx"], kd, sd, x["idx_keys"], idx, cnt, ws, kcand,
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
    _check_rescored_rows(csa, rows, x["q_idx"], x["w_idx"], x["idx_keys"], kd, sd, qc.reshape(T, 64, 128), w8,
                         x["pos0"], N, k, kcand, gi, gc, exact)
    recalls = []
    for i, r in enumerate(rows):
        ref = set(oracle.topk(exact[i][None], k)[0][0][:gc[r]].tolist())
        recalls.append(len(ref & set(gi[r, :gc[r]].tolist())) / max(len(ref), 1))
    print("FP4 two-stage top-512 recall on sampled chunk rows:", [round(v, 4) for v in recalls])
    assert min(recalls) >= 0.99
