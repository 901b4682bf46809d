"""GPU parity of the FP4 indexer keys (page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md,
C4; block format per reading R30: E2M1 elements, one E8M0 scale per 32,
element 2j in the low nibble) against the float64 oracle.

Tolerances: codes and scales of the quantiser bit for bit; the scan's
scores within 1e-4 of the oracle's (max |diff| / max |oracle|) and bit for
bit where every score is one exact product; the selection, gather and
attention of the decode step by the rules of the other decode-step tests.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import numfmt
from tests.gpu_util import (DEV, assert_bf16_close, assert_fp4_key_close, assert_topk_gap_rule, dev_bf16, dev_f32,
                            host_bits, host_f64, rel_err)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import compressed_sparse_attention_reduce_amd as pkg
    pkg.lib()
    return pkg


def _g(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _words(scales_u8):
    """[..., N, d / 32] uint8 E8M0 (d = 128) -> the same bytes as the device's [..., N, 4] uint8."""
    return torch.from_numpy(np.ascontiguousarray(scales_u8, dtype=np.uint8)).to(DEV)


def _quant_rows_fp4(g, rows, d):
    """Rows over many magnitudes, with blocks placed on the scale rule's
    boundaries and on E2M1's rounding midpoints."""
    x = (g.standard_normal((rows, d)) * np.exp(g.uniform(-8, 8, (rows, 1)))).astype(np.float32)
    x[0] = 0.0                                        # zero blocks: scale 2^0, codes 0
    if rows > 1:
        x[1, :32] = 0.0
        x[1, 0] = 6.0                                 # amax exactly 6: X = 0, the rest encoded as given
        x[1, 1:10] = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -0.25, -5.0]
        if d > 32:
            x[1, 32:64] = 0.0
            x[1, 32] = np.nextafter(np.float32(6.0), np.float32(7.0))   # just above 6: X = 1
            x[1, 33:36] = [1.0, -0.5, 0.49]
    if rows > 2:
        x[2, :32] = 0.0
        x[2, 3] = np.float32(1.5e-38)                 # below 6 2^-128: X clamps to -127, 2.55 -> 3
        x[2, 4] = np.float32(-3e-39 * 4)              # -1.2e-38 -> -2.04 -> -2
    return x


QUANT_CASES = [("f32_128", 37, 128, False), ("bf16_512", 9, 512, True), ("f32_one_block", 3, 32, False),
               ("f32_many_rows", 2000, 128, False)]


@pytest.mark.parametrize("case", QUANT_CASES, ids=[c[0] for c in QUANT_CASES])
def test_quantize_fp4_bit_exact(csa, case):
    name, rows, d, bf16 = case
    x = _quant_rows_fp4(_g(rows * 5 + d), rows, d)
    if bf16:
        xb = numfmt.f32_to_bf16_bits(x)
        xd = dev_bf16(xb)
        x = numfmt.bf16_bits_to_f64(xb).astype(np.float32)
    else:
        xd = torch.from_numpy(x).to(DEV)
    codes = torch.full((rows, d // 2), 0x55, dtype=torch.uint8, device=DEV)
    scales = torch.full((rows, d // 32), 0x55, dtype=torch.uint8, device=DEV)
    print(f"quantize_fp4 {name}", flush=True)
    csa.csa_quantize_fp4(xd, codes, scales)
    torch.cuda.synchronize()
    rc, rs = numfmt.quantize_mxfp4_rows(x)
    np.testing.assert_array_equal(scales.cpu().numpy(), rs)
    np.testing.assert_array_equal(codes.cpu().numpy(), numfmt.pack_e2m1(rc))


def test_fp4_scan_decodes_every_code_and_scale(csa):
    """The scan reads its keys as E2M1 times E8M0 in the measured operand
    order: key j holds one nonzero element, code c at element e with that
    block's scale s (c over all 16 codes, s over 2 .. 251, e over all 128
    elements); query head 0 holds 1.0 everywhere and head 1 -1.0, weights
    (1, 2).  So the score is v = e2m1(c) 2^(s - 127) when v > 0 and 2|v|
    otherwise, each one exact product (s <= 251 keeps 2|v| finite, s >= 2
    keeps it normal): compared bit for bit."""
    g = _g(5100)
    cs, ss = np.meshgrid(np.arange(16), np.arange(2, 252), indexing="ij")
    cs, ss = cs.ravel(), ss.ravel()
    n = cs.size
    e = np.arange(n) % 128
    codes = np.zeros((n, 128), dtype=np.uint8)
    codes[np.arange(n), e] = cs
    scales = g.integers(2, 255, size=(n, 4)).astype(np.uint8)
    scales[np.arange(n), e // 32] = ss
    q = np.zeros((1, 1, 64, 128), dtype=np.uint8)
    q[0, 0, 0, :] = 0x38                               # E4M3 1.0
    q[0, 0, 1, :] = 0xB8                               # E4M3 -1.0
    w = np.zeros((1, 1, 64), dtype=np.float32)
    w[0, 0, 0], w[0, 0, 1] = 1.0, 2.0
    v = numfmt.e2m1_decode(cs.astype(np.uint8)) * np.ldexp(1.0, ss - 127)
    want = np.where(v > 0, v, -2.0 * v)
    s = torch.full((1, 1, n + 5), 7.0, device=DEV)
    kd = torch.from_numpy(numfmt.pack_e2m1(codes)[None]).to(DEV)
    csa.csa_index_score_fp4(torch.from_numpy(q).to(DEV), dev_f32(w), kd, _words(scales[None]), s, n=n)
    torch.cuda.synchronize()
    got = s[0, 0].cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(got[:n], want)
    assert (got[n:] == 7.0).all(), "wrote past n"
    # the oracle agrees on the same codes
    np.testing.assert_array_equal(oracle.index_score_fp4(q[0], w[0], codes, scales)[0], want)


def _fp4_inputs(g, B, t, n):
    """Query and keys drawn like the bf16 workloads, quantised by the oracle
    (query E4M3 per head row with its scale folded into w; keys MXFP4)."""
    q = (g.standard_normal((B, t, 64, 128)) / np.sqrt(128)).astype(np.float32)
    w = g.standard_normal((B, t, 64)).astype(np.float32)
    K = g.standard_normal((B, n, 128)).astype(np.float32)
    qc, qs = numfmt.quantize_e4m3_rows(q.reshape(-1, 128))
    kc, ks = numfmt.quantize_mxfp4_rows(K.reshape(-1, 128))
    w2 = (w * qs.reshape(B, t, 64)).astype(np.float32)
    return qc.reshape(B, t, 64, 128), w2, kc.reshape(B, n, 128), ks.reshape(B, n, 4)


FP4_SCORE_CASES = [
    # name, B, t, n, causal
    ("decode_ctx8k", 1, 1, 2048, False),
    ("ragged_tail", 1, 1, 1000, False),
    ("batch3", 3, 1, 4100, False),
    ("short", 1, 1, 17, False),
    ("causal_rows", 2, 3, 700, True),
    ("long_row", 1, 1, 65536, False),
]


@pytest.mark.parametrize("case", FP4_SCORE_CASES, ids=[c[0] for c in FP4_SCORE_CASES])
def test_index_score_fp4(csa, case):
    name, B, t, n, causal = case
    qc, w, kc, ks = _fp4_inputs(_g(len(name) * 19 + n), B, t, n)
    ld = n + 3
    scores = torch.full((B, t, ld), 123.0, device=DEV)
    pos_np = (4 * n - 4 * t - 10 + 3 * np.arange(B * t)).astype(np.int32).reshape(B, t) if causal else None
    print(f"index_score_fp4 {name}", flush=True)
    csa.csa_index_score_fp4(torch.from_numpy(qc).to(DEV), dev_f32(w),
                            torch.from_numpy(numfmt.pack_e2m1(kc)).to(DEV), _words(ks), scores,
                            q_pos=None if pos_np is None else torch.from_numpy(pos_np).to(DEV))
    torch.cuda.synchronize()
    got = scores.cpu().numpy().astype(np.float64)
    assert (got[:, :, n:] == 123.0).all(), "wrote past n"
    for b in range(B):
        ref = oracle.index_score_fp4(qc[b], w[b], kc[b], ks[b], q_pos=None if pos_np is None else pos_np[b])
        fin = np.isfinite(ref)
        assert (np.isfinite(got[b, :, :n]) == fin).all(), "mask differs"
        assert rel_err(got[b, :, :n][fin], ref[fin]) <= 1e-4


def test_index_score_fp4_full_size_sampled(csa):
    """n = 250,000 FP4 keys quantised on the GPU from the 1M-context bf16
    cache: sampled codes and scales bit for bit against the oracle's
    quantiser, sampled scores against the oracle's FP4 score."""
    shape = synth.SHAPES["ctx1m"]
    x = synth.make_decode_inputs_torch(shape, seed=None, device=DEV, layers=1)[0]
    n = shape.n_comp
    keys = x["idx_keys"][:, :n].contiguous()
    kc = torch.empty(1, n, 64, dtype=torch.uint8, device=DEV)
    ks = torch.empty(1, n, 4, dtype=torch.uint8, device=DEV)
    csa.csa_quantize_fp4(keys, kc, ks)
    q = x["q_idx"][:, None].contiguous()
    qc = torch.empty(1, 1, 64, 128, dtype=torch.uint8, device=DEV)
    w8 = torch.empty(1, 1, 64, dtype=torch.float32, device=DEV)
    csa.csa_quantize_query_fp8(q, x["w_idx"][:, None].contiguous(), qc, w8)
    s4 = torch.empty(1, 1, n, device=DEV)
    csa.csa_index_score_fp4(qc, w8, kc, ks, s4)
    torch.cuda.synchronize()
    g = _g(5101)
    sample = np.unique(np.concatenate([np.arange(64), np.arange(n - 64, n), g.integers(0, n, 4096)]))
    idx = torch.from_numpy(sample).to(DEV)
    rc, rs = numfmt.quantize_mxfp4_rows(host_f64(keys[0, idx]).astype(np.float32))
    np.testing.assert_array_equal(kc[0, idx].cpu().numpy(), numfmt.pack_e2m1(rc))
    np.testing.assert_array_equal(ks[0, idx].cpu().numpy(), rs)
    ref = oracle.index_score_fp4(qc[0].cpu().numpy(), w8[0].cpu().numpy(), rc, rs)[0]
    assert rel_err(s4[0, 0].cpu().numpy().astype(np.float64)[sample], ref) <= 1e-4


# ---------------------------------------------------------------------------
# the decode step over FP4 keys
# ---------------------------------------------------------------------------

def _fp8_query(qi, wi):
    qc, qs = numfmt.quantize_e4m3_rows(qi.reshape(-1, qi.shape[-1]))
    return qc.reshape(qi.shape), (wi * qs.reshape(wi.shape)).astype(np.float32)


def _fp4_rescored_layer(csa, x, B, max_comp, K, kc):
    f = numfmt.bf16_bits_to_f64
    c0, s0 = numfmt.quantize_mxfp4_rows(f(x["idx_keys"]).reshape(-1, 128).astype(np.float32))
    codes = torch.from_numpy(numfmt.pack_e2m1(c0).reshape(B, max_comp, 64)).to(DEV)
    scales = torch.from_numpy(s0.reshape(B, max_comp, 4)).to(DEV)
    exact_keys = dev_bf16(x["idx_keys"])
    comp, swa = dev_bf16(x["comp_kv"]), dev_bf16(x["swa"])
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=codes, idx_scales=scales, swa=swa,
                            main_bias=dev_f32(x["main_bias"]), idx_bias=dev_f32(x["idx_bias"]),
                            sink=dev_f32(x["sink"]), n_comp=x["n_comp"], swa_head=x["swa_head"],
                            swa_len=x["swa_len"], h=64, h_i=64, top_k=K, idx_keys_exact=exact_keys,
                            idx_rescore=kc)
    assert L.idx_dtype == csa.CSA_FP4_E2M1 and L.d_i == 128
    return L, codes, scales, exact_keys, comp, swa


def _check_rescored_selection(csa, qi_dev, wi_dev, exact_keys, N, got_s4, gi, gc, exact_ref, K, kc, b=0):
    """The two-stage selection bit for bit as the oracle's two stages on the
    GPU's own FP4 scores and the bfloat16 scan's scores (which the rescoring
    reproduces exactly), and by the gap rule against the float64 exact
    scores inside the first stage's set."""
    s16 = torch.empty(1, 1, N, device=DEV)
    csa.csa_index_score(qi_dev[b:b + 1, None].contiguous(), wi_dev[b:b + 1, None].contiguous(),
                        exact_keys[b:b + 1, :N].contiguous(), s16)
    torch.cuda.synchronize()
    s16 = s16[0, 0].cpu().numpy().astype(np.float64)
    want, wc = oracle.rescored_topk(got_s4[None], s16[None], K, kc)
    np.testing.assert_array_equal(gi, want[0])
    assert gc == wc[0]
    stage1 = oracle.topk(got_s4[None], kc)[0][0]
    inside = np.full(N, -np.inf)
    inside[stage1[stage1 >= 0]] = exact_ref[stage1[stage1 >= 0]]
    assert_topk_gap_rule(gi, gc, inside, K)


@pytest.mark.parametrize("B", [1, 5])
def test_decode_steps_in_sequence_fp4_rescored(csa, B):
    """Steps over FP4 keys with the two-stage selection (top_k 64 out of the
    FP4 best 128; two block completions; batch 5 takes the separate top-k):
    the new key in both forms within rounding of the oracle's, then adopted;
    FP4 scores against the oracle's; the selection exactly as above; gather
    and attention against the oracle."""
    K, kc, W = 64, 128, 8
    shape = synth.with_(synth.SHAPES["ctx8k"], batch=B, ctx=12000, n_comp=3000, top_k=K, w=W)
    x = synth.make_decode_inputs(shape, 5201 + B, max_comp=3100)
    g = _g(5202 + B)
    f = numfmt.bf16_bits_to_f64
    L, codes, scales, exact_keys, comp, swa = _fp4_rescored_layer(csa, x, B, 3100, K, kc)
    osts = []
    for b in range(B):
        c0 = numfmt.unpack_e2m1(codes[b].cpu().numpy())
        osts.append(oracle.LayerState(comp_kv=f(x["comp_kv"][b]), idx_keys=f(x["idx_keys"][b]), n_comp=x["n_comp"],
                                      swa=oracle.SwaRing(f(x["swa"][b]), x["swa_head"], x["swa_len"]),
                                      main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"],
                                      round_cache=numfmt.bf16_round_f64, idx_codes=c0,
                                      idx_scales=scales[b].cpu().numpy().copy(), idx_fp4=True, fp8_rescore=kc))
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
        print(f"rescored fp4-key step pos={pos} B={B}", flush=True)
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
            np.testing.assert_array_equal(numfmt.unpack_e2m1(codes[b, :n0].cpu().numpy()), ost.idx_codes[:n0])
            if completes:
                yi = oracle.compress(zi[b], ci[b], x["idx_bias"], 4)[0]
                assert_fp4_key_close(codes[b, n0].cpu().numpy(), scales[b, n0].cpu().numpy(), yi)
                assert_bf16_close(host_bits(exact_keys[b, n0]), yi)
                assert_bf16_close(host_bits(comp[b, n0]), oracle.compress(zm[b], cm[b], x["main_bias"], 4)[0])
            ost.comp_kv[:N] = host_f64(comp[b, :N])
            ost.idx_keys[:N] = host_f64(exact_keys[b, :N])
            ost.idx_codes[:N] = numfmt.unpack_e2m1(codes[b, :N].cpu().numpy())
            ost.idx_scales[:N] = scales[b, :N].cpu().numpy()
            qc, w8 = _fp8_query(f(qi[b:b + 1]).astype(np.float32), wi[b:b + 1])
            ref_s4 = oracle.index_score_fp4(qc, w8, ost.idx_codes[:N], ost.idx_scales[:N])[0]
            got_s4 = outs["scores"][b, :N].cpu().numpy().astype(np.float64)
            assert rel_err(got_s4, ref_s4) <= 1e-4
            exact_ref = oracle.index_score(f(qi[b])[None], wi[b][None].astype(np.float64), ost.idx_keys[:N])[0]
            gi, gc = outs["topk_idx"][b].cpu().numpy(), int(outs["topk_count"][b])
            _check_rescored_selection(csa, qi_dev, wi_dev, exact_keys, N, got_s4, gi, gc, exact_ref, K, kc, b)
            rows, n_valid = oracle.gather(ost.comp_kv[:N], gi, gc, ost.swa.rows, ost.swa.head, ost.swa.length)
            assert int(outs["n_valid"][b]) == n_valid
            np.testing.assert_array_equal(host_f64(outs["gather_buf"][b, :n_valid]), rows)
            ro, rl = oracle.sparse_attn(f(q[b]), rows, x["sink"], 1 / np.sqrt(512))
            assert rel_err(host_f64(outs["out"][b]), ro) <= 2e-2
            assert rel_err(outs["lse"][b].cpu().numpy(), rl) <= 2e-2


def test_decode_step_fp4_plain_selection(csa):
    """Without the second stage the step selects the top-k of the FP4 scores
    themselves: exact on the GPU's scores, by the gap rule on the oracle's."""
    K, W = 64, 8
    shape = synth.with_(synth.SHAPES["ctx8k"], ctx=8000, n_comp=1999, top_k=K, w=W)
    x = synth.make_decode_inputs(shape, 5301, max_comp=2100)
    g = _g(5302)
    f = numfmt.bf16_bits_to_f64
    L, codes, scales, exact_keys, comp, swa = _fp4_rescored_layer(csa, x, 1, 2100, K, 0)
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    pos = x["pos"]
    q = synth.to_bf16_bits(g.standard_normal((1, 64, 512), dtype=np.float32))
    qi = synth.to_bf16_bits(g.standard_normal((1, 64, 128), dtype=np.float32) / np.float32(np.sqrt(128)))
    wi = g.standard_normal((1, 64), dtype=np.float32)
    kvn = synth.to_bf16_bits(g.standard_normal((1, 512), dtype=np.float32))
    zm, cm = g.standard_normal((2, 1, 4, 512), dtype=np.float32)
    zi, ci = g.standard_normal((2, 1, 4, 128), dtype=np.float32)
    outs = dict(scores=torch.empty(1, 2100, device=DEV), topk_idx=torch.empty(1, K, dtype=torch.int32, device=DEV),
                topk_count=torch.empty(1, dtype=torch.int32, device=DEV),
                gather_buf=torch.zeros(1, K + W, 512, dtype=torch.bfloat16, device=DEV),
                n_valid=torch.empty(1, dtype=torch.int32, device=DEV),
                out=torch.empty(1, 64, 512, dtype=torch.bfloat16, device=DEV))
    io = csa.make_step_io(pos=pos, q=dev_bf16(q), q_idx=dev_bf16(qi), w_idx=dev_f32(wi), kv_new=dev_bf16(kvn),
                          z_main=dev_f32(zm), c_main=dev_f32(cm), z_idx=dev_f32(zi), c_idx=dev_f32(ci), **outs)
    print(f"plain fp4-key step pos={pos}", flush=True)
    csa.csa_decode_step(L, io, ws)
    torch.cuda.synchronize()
    N = L.n_comp if pos % 4 != 3 else L.n_comp + 1
    qc, w8 = _fp8_query(f(qi).astype(np.float32), wi)
    c_all = numfmt.unpack_e2m1(codes[0, :N].cpu().numpy())
    ref_s4 = oracle.index_score_fp4(qc, w8, c_all, scales[0, :N].cpu().numpy())[0]
    got_s4 = outs["scores"][0, :N].cpu().numpy().astype(np.float64)
    assert rel_err(got_s4, ref_s4) <= 1e-4
    gi, gc = outs["topk_idx"][0].cpu().numpy(), int(outs["topk_count"][0])
    np.testing.assert_array_equal(gi, oracle.topk(got_s4[None], K)[0][0])
    assert_topk_gap_rule(gi, gc, ref_s4, K)
    comp_h = host_f64(comp[0, :N])
    swa_h = host_f64(swa[0])
    head = (x["swa_head"] + 1) % W
    ln = min(x["swa_len"] + 1, W)
    rows, n_valid = oracle.gather(comp_h, gi, gc, swa_h, head, ln)
    assert int(outs["n_valid"][0]) == n_valid
    ro, _ = oracle.sparse_attn(f(q[0]), rows, x["sink"], 1 / np.sqrt(512))
    assert rel_err(host_f64(outs["out"][0]), ro) <= 2e-2


def test_decode_step_ctx1m_fp4_rescored_full_size_recall(csa):
    """One 1M-context layer over FP4 keys with the two-stage selection
    (top-512 of the FP4 best 2048): the selection exactly as the oracle's
    two stages on the GPU's scores, and top-512 recall against the float64
    exact indexer of at least 0.99 (page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md,
    Tier 1 gate 4)."""
    shape = synth.SHAPES["ctx1m"]
    x = synth.make_decode_inputs_torch(shape, seed=None, device=DEV, layers=1)[0]
    B, K, W, D, kc = 1, shape.top_k, shape.w, shape.d, 4 * shape.top_k
    n0 = x["n_comp"]
    codes = torch.zeros(B, shape.max_comp, 64, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, shape.max_comp, 4, dtype=torch.uint8, device=DEV)
    csa.csa_quantize_fp4(x["idx_keys"][:, :n0].contiguous(), codes[:, :n0], scales[:, :n0])
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
    print("ctx1m fp4 rescored step", flush=True)
    csa.csa_decode_step(L, io, ws)
    torch.cuda.synchronize()
    N = shape.n_comp
    got_s4 = outs["scores"][0, :N].cpu().numpy().astype(np.float64)
    exact_ref = oracle.index_score(host_f64(x["q_idx"][0])[None], x["w_idx"][0].cpu().numpy()[None].astype(np.float64),
                                   host_f64(exact_keys[0, :N]))[0]
    gi, gc = outs["topk_idx"][0].cpu().numpy(), int(outs["topk_count"][0])
    _check_rescored_selection(csa, x["q_idx"], x["w_idx"], exact_keys, N, got_s4, gi, gc, exact_ref, K, kc)
    ref = set(oracle.topk(exact_ref[None], K)[0][0].tolist())
    recall = len(ref & set(gi.tolist())) / K
    plain = len(ref & set(oracle.topk(got_s4[None], K)[0][0].tolist())) / K
    print(f"top-512 recall at n=250000: FP4 two-stage {recall:.4f}, FP4 alone {plain:.4f}")
    assert recall >= 0.99
    assert plain < 0.9
    sel = host_f64(x["comp_kv"][0, torch.from_numpy(gi).to(DEV).long()])
    np.testing.assert_array_equal(host_f64(outs["gather_buf"][0, :gc]), sel)
    assert int(outs["n_valid"][0]) == gc + W


def test_decode_steps_fp4_from_first_token(csa):
    """From token 0 over FP4 keys (an empty compressed cache, the first block
    completing at token 3, the window filling and wrapping), batch 2, plain
    selection: every step's new key, scores, selection, gather and attention
    against the oracle, the GPU's new entries adopted as in the other
    sequences."""
    B, H, D, Di, W, K, m, max_comp, steps = 2, 64, 512, 128, 8, 4, 4, 16, 11
    g = _g(5500)
    f = numfmt.bf16_bits_to_f64
    comp = torch.zeros(B, max_comp, D, dtype=torch.bfloat16, device=DEV)
    codes = torch.zeros(B, max_comp, Di // 2, dtype=torch.uint8, device=DEV)
    scales = torch.zeros(B, max_comp, Di // 32, dtype=torch.uint8, device=DEV)
    swa = torch.zeros(B, W, D, dtype=torch.bfloat16, device=DEV)
    mb = g.standard_normal((m, D), dtype=np.float32) * np.float32(0.1)
    ib = g.standard_normal((m, Di), dtype=np.float32) * np.float32(0.1)
    sink = g.standard_normal(H, dtype=np.float32)
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=codes, idx_scales=scales, swa=swa, main_bias=dev_f32(mb),
                            idx_bias=dev_f32(ib), sink=dev_f32(sink), n_comp=0, swa_head=0, swa_len=0, h=H, h_i=64,
                            top_k=K)
    assert L.idx_dtype == csa.CSA_FP4_E2M1
    osts = [oracle.LayerState(comp_kv=np.zeros((max_comp, D)), idx_keys=np.zeros((max_comp, Di)), n_comp=0,
                              swa=oracle.SwaRing(np.zeros((W, D))), main_bias=mb.astype(np.float64),
                              idx_bias=ib.astype(np.float64), sink=sink.astype(np.float64),
                              round_cache=numfmt.bf16_round_f64, idx_codes=np.zeros((max_comp, Di), np.uint8),
                              idx_scales=np.zeros((max_comp, Di // 32), np.uint8), idx_fp4=True) for _ in range(B)]
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    for pos in range(steps):
        q = synth.to_bf16_bits(g.standard_normal((B, H, D), dtype=np.float32))
        qi = synth.to_bf16_bits(g.standard_normal((B, 64, Di), dtype=np.float32) / np.float32(np.sqrt(Di)))
        wi = g.standard_normal((B, 64), dtype=np.float32)
        kvn = synth.to_bf16_bits(g.standard_normal((B, D), dtype=np.float32))
        zm, cm = g.standard_normal((2, B, m, D), dtype=np.float32)
        zi, ci = g.standard_normal((2, B, m, Di), dtype=np.float32)
        outs = dict(scores=torch.full((B, max_comp), 9.0, device=DEV),
                    topk_idx=torch.full((B, K), -7, dtype=torch.int32, device=DEV),
                    topk_count=torch.full((B,), -7, dtype=torch.int32, device=DEV),
                    gather_buf=torch.zeros(B, K + W, D, dtype=torch.bfloat16, device=DEV),
                    n_valid=torch.full((B,), -7, dtype=torch.int32, device=DEV),
                    out=torch.empty(B, H, D, dtype=torch.bfloat16, device=DEV), lse=torch.empty(B, H, device=DEV))
        io = csa.make_step_io(pos=pos, q=dev_bf16(q), q_idx=dev_bf16(qi), w_idx=dev_f32(wi), kv_new=dev_bf16(kvn),
                              z_main=dev_f32(zm), c_main=dev_f32(cm), z_idx=dev_f32(zi), c_idx=dev_f32(ci), **outs)
        print(f"fp4-key step from the first token, pos={pos}", flush=True)
        csa.csa_decode_step(L, io, ws)
        csa.csa_layer_advance(L, pos)
        torch.cuda.synchronize()
        for b in range(B):
            ost = osts[b]
            n0 = ost.n_comp
            oracle.decode_step(ost, q=f(q[b]), q_idx=f(qi[b]), w_idx=wi[b], kv_new=f(kvn[b]), pos=pos, top_k=K,
                               z_main=zm[b], c_main=cm[b], z_idx=zi[b], c_idx=ci[b], scale=1 / np.sqrt(D))
            N = ost.n_comp
            assert (L.n_comp, L.swa_head, L.swa_len) == (N, ost.swa.head, ost.swa.length)
            if N > n0:
                yi = oracle.compress(zi[b], ci[b], ib.astype(np.float64), m)[0]
                assert_fp4_key_close(codes[b, n0].cpu().numpy(), scales[b, n0].cpu().numpy(), yi)
                assert_bf16_close(host_bits(comp[b, n0]), oracle.compress(zm[b], cm[b], mb.astype(np.float64), m)[0])
            ost.comp_kv[:N] = host_f64(comp[b, :N])
            ost.idx_codes[:N] = numfmt.unpack_e2m1(codes[b, :N].cpu().numpy())
            ost.idx_scales[:N] = scales[b, :N].cpu().numpy()
            gi, gc = outs["topk_idx"][b].cpu().numpy(), int(outs["topk_count"][b])
            if N:
                qc, w8 = _fp8_query(f(qi[b:b + 1]).astype(np.float32), wi[b:b + 1])
                ref_s = oracle.index_score_fp4(qc, w8, ost.idx_codes[:N], ost.idx_scales[:N])[0]
                got_s = outs["scores"][b, :N].cpu().numpy().astype(np.float64)
                assert rel_err(got_s, ref_s) <= 1e-4
                np.testing.assert_array_equal(gi, oracle.topk(got_s[None], K)[0][0])
                assert_topk_gap_rule(gi, gc, ref_s, K)
            else:
                assert gc == 0 and (gi == -1).all()
            rows, n_valid = oracle.gather(ost.comp_kv[:N], gi, gc, ost.swa.rows, ost.swa.head, ost.swa.length)
            assert int(outs["n_valid"][b]) == n_valid
            np.testing.assert_array_equal(host_f64(outs["gather_buf"][b, :n_valid]), rows)
            ro, rl = oracle.sparse_attn(f(q[b]), rows, ost.sink, 1 / np.sqrt(D))
            assert rel_err(host_f64(outs["out"][b]), ro) <= 2e-2
            assert rel_err(outs["lse"][b].cpu().numpy(), rl) <= 2e-2
    assert L.n_comp == 2


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_decode_step_batch128k_lowp_keys_full_size(csa, fmt):
    """The batched 128K workload (8 sequences x 32,768 entries) with E4M3 or
    E2M1 indexer keys (quantised by the oracle), one decode step with plain
    selection: at this size each scan wave hands on 10 candidates (the
    threshold-search extraction).  Per sequence: the new key, every score
    against the oracle's, the top-k exact on the GPU's scores and by the gap
    rule on the oracle's, gather and attention against the oracle."""
    shape = synth.SHAPES["batch128k"]
    x = synth.make_decode_inputs(shape, 5600 if fmt == "e2m1" else 5601)
    B, K, W, D, Di, N0 = shape.batch, shape.top_k, shape.w, shape.d, shape.d_i, x["n_comp"]
    f = numfmt.bf16_bits_to_f64
    kf = f(x["idx_keys"]).reshape(-1, Di).astype(np.float32)
    if fmt == "e2m1":
        c, sc = numfmt.quantize_mxfp4_rows(kf)
        codes = torch.from_numpy(numfmt.pack_e2m1(c).reshape(B, -1, Di // 2)).to(DEV)
        scales = torch.from_numpy(sc.reshape(B, -1, Di // 32)).to(DEV)
    else:
        c, sc = numfmt.quantize_e4m3_rows(kf)
        codes = torch.from_numpy(c.reshape(B, -1, Di)).to(DEV)
        scales = dev_f32(sc.reshape(B, -1))
    comp, swa = dev_bf16(x["comp_kv"]), dev_bf16(x["swa"])
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=codes, idx_scales=scales, swa=swa,
                            main_bias=dev_f32(x["main_bias"]), idx_bias=dev_f32(x["idx_bias"]),
                            sink=dev_f32(x["sink"]), n_comp=N0, swa_head=x["swa_head"], swa_len=x["swa_len"],
                            h=shape.h, h_i=shape.h_i, top_k=K)
    assert L.idx_dtype == (csa.CSA_FP4_E2M1 if fmt == "e2m1" else csa.CSA_FP8_E4M3)
    outs = dict(scores=torch.empty(B, shape.max_comp, device=DEV),
                topk_idx=torch.empty(B, K, dtype=torch.int32, device=DEV),
                topk_count=torch.empty(B, dtype=torch.int32, device=DEV),
                gather_buf=torch.zeros(B, K + W, D, dtype=torch.bfloat16, device=DEV),
                n_valid=torch.empty(B, dtype=torch.int32, device=DEV),
                out=torch.empty(B, shape.h, D, dtype=torch.bfloat16, device=DEV),
                lse=torch.empty(B, shape.h, device=DEV))
    io = csa.make_step_io(pos=x["pos"], q=dev_bf16(x["q"]), q_idx=dev_bf16(x["q_idx"]), w_idx=dev_f32(x["w_idx"]),
                          kv_new=dev_bf16(x["kv_new"]), z_main=dev_f32(x["z_main"]), c_main=dev_f32(x["c_main"]),
                          z_idx=dev_f32(x["z_idx"]), c_idx=dev_f32(x["c_idx"]), **outs)
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    print(f"batch128k step over {fmt} keys", flush=True)
    csa.csa_decode_step(L, io, ws)
    torch.cuda.synchronize()
    completes = x["pos"] % 4 == 3
    N = N0 + (1 if completes else 0)
    for b in range(B):
        if completes:  # the new key within rounding of the oracle's, then the GPU's adopted
            yi = oracle.compress(x["z_idx"][b], x["c_idx"][b], x["idx_bias"], 4)[-1]
            if fmt == "e2m1":
                assert_fp4_key_close(codes[b, N0].cpu().numpy(), scales[b, N0].cpu().numpy(), yi)
            else:
                got = numfmt.e4m3_decode(codes[b, N0].cpu().numpy()) * float(scales[b, N0])
                y = np.asarray(yi, np.float32).astype(np.float64)
                assert (np.abs(got - y) <= np.maximum(np.abs(y) * 2.0 ** -4, np.abs(y).max() / 448 * 2.0 ** -10)
                        + 1e-5 * np.abs(y).max()).all()
        qc, w8 = _fp8_query(f(x["q_idx"][b:b + 1]).astype(np.float32), x["w_idx"][b:b + 1])
        if fmt == "e2m1":
            ref_s = oracle.index_score_fp4(qc, w8, numfmt.unpack_e2m1(codes[b, :N].cpu().numpy()),
                                           scales[b, :N].cpu().numpy())[0]
        else:
            ref_s = oracle.index_score_fp8(qc, w8, codes[b, :N].cpu().numpy(), scales[b, :N].cpu().numpy())[0]
        got_s = outs["scores"][b, :N].cpu().numpy().astype(np.float64)
        assert rel_err(got_s, ref_s) <= 1e-4
        gi, gc = outs["topk_idx"][b].cpu().numpy(), int(outs["topk_count"][b])
        np.testing.assert_array_equal(gi, oracle.topk(got_s[None], K)[0][0])
        assert_topk_gap_rule(gi, gc, ref_s, K)
        comp_b = host_f64(comp[b, :N])
        swa_b = host_f64(swa[b])
        rows, n_valid = oracle.gather(comp_b, gi, gc, swa_b, (x["swa_head"] + 1) % W, min(x["swa_len"] + 1, W))
        assert int(outs["n_valid"][b]) == n_valid
        np.testing.assert_array_equal(host_f64(outs["gather_buf"][b, :n_valid]), rows)
        ro, rl = oracle.sparse_attn(f(x["q"][b]), rows, x["sink"], 1 / np.sqrt(D))
        assert rel_err(host_f64(outs["out"][b]), ro) <= 2e-2
        assert rel_err(outs["lse"][b].cpu().numpy(), rl) <= 2e-2
