"""CPU: pins of the FP4 indexer keys in the oracle — the E2M1 codec, the
E8M0 block scales, the packing, the FP4 index score, the FP4 decode step —
and the recall study that sets their two-stage candidate count.

The FP4 indexer cache is page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, C4; its
block format (E2M1 elements, one E8M0 scale per 32, element 2j in the low
nibble) is reading R30.  The E2M1 values below are the format's definition
(1 sign, 2 exponent bits with bias 1, 1 mantissa bit, exponent field 0 =
subnormal 0.5 m, no inf or NaN), written out as a table."""

import math

import numpy as np
import pytest

import oracle
import synth
from oracle import numfmt

# code -> value, the whole E2M1 format
E2M1 = {0x0: 0.0, 0x1: 0.5, 0x2: 1.0, 0x3: 1.5, 0x4: 2.0, 0x5: 3.0, 0x6: 4.0, 0x7: 6.0,
        0x8: -0.0, 0x9: -0.5, 0xA: -1.0, 0xB: -1.5, 0xC: -2.0, 0xD: -3.0, 0xE: -4.0, 0xF: -6.0}


def _g(seed):
    return np.random.Generator(np.random.PCG64(seed))


def test_e2m1_decode_every_code():
    vals = numfmt.e2m1_decode(np.arange(16, dtype=np.uint8))
    assert vals.tolist() == [E2M1[c] for c in range(16)]
    assert math.copysign(1.0, vals[8]) == -1.0
    assert numfmt.E2M1_MAX == 6.0 and numfmt.MX_BLOCK == 32


def test_e2m1_encode_round_trip_and_zero():
    codes = np.array([c for c in range(16) if c != 0x8], dtype=np.uint8)
    np.testing.assert_array_equal(numfmt.e2m1_encode(numfmt.e2m1_decode(codes)), codes)
    # a zero result is code 0, whatever the sign of the input
    assert numfmt.e2m1_encode(np.array([-0.0, 0.0, -0.2, 0.2])).tolist() == [0, 0, 0, 0]


def test_e2m1_encode_ties_to_even_and_saturation():
    enc = lambda x: int(numfmt.e2m1_encode(np.array([x]))[0])  # noqa: E731
    # midpoints between neighbours go to the even code
    assert [enc(x) for x in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)] == [0x0, 0x2, 0x2, 0x4, 0x4, 0x6, 0x6]
    assert [enc(-x) for x in (0.75, 1.25, 1.75, 2.5, 3.5, 5.0)] == [0xA, 0xA, 0xC, 0xC, 0xE, 0xE]
    # just off the midpoints
    assert enc(0.26) == 0x1 and enc(0.74) == 0x1 and enc(5.01) == 0x7 and enc(4.99) == 0x6
    # beyond 6 saturates
    assert enc(6.5) == 0x7 and enc(1e30) == 0x7 and enc(-1e30) == 0xF


def test_e2m1_encode_is_nearest_by_brute_force():
    g = _g(41)
    x = np.concatenate([g.uniform(-7, 7, 4000), g.standard_normal(1000) * 0.3])
    got = numfmt.e2m1_decode(numfmt.e2m1_encode(x))
    grid = np.array(sorted(set(E2M1.values())))
    best = np.abs(np.clip(x, -6, 6)[:, None] - grid[None, :]).min(axis=1)
    np.testing.assert_array_equal(np.abs(np.clip(x, -6, 6) - got), best)


def test_e8m0_decode():
    assert numfmt.e8m0_decode(np.array([127, 128, 126, 0, 254], dtype=np.uint8)).tolist() == \
        [1.0, 2.0, 0.5, 2.0 ** -127, 2.0 ** 127]


def _block(amax, n=32, seed=0):
    """A float32 block whose largest magnitude is amax (at element 5)."""
    b = (_g(seed).uniform(-1, 1, n) * amax * 0.9).astype(np.float32)
    b[5] = np.float32(amax)
    return b


def test_mxfp4_scale_closed_forms():
    """The block exponent X is the least integer with max|block| <= 6 2^X."""
    q = lambda b: int(numfmt.quantize_mxfp4_rows(b[None])[1][0, 0]) - 127  # noqa: E731
    for k in (-20, -3, 0, 1, 7, 40):
        six = 6.0 * 2.0 ** k
        assert q(_block(six)) == k                                   # exactly 6 2^k: no saturation at X = k
        assert q(_block(np.nextafter(np.float32(six), np.float32(np.inf)))) == k + 1
        assert q(_block(3.0 * 2.0 ** k)) == k - 1                    # 3 2^k = 6 2^(k-1)
        assert q(_block(np.nextafter(np.float32(3.0 * 2.0 ** k), np.float32(np.inf)))) == k
        assert q(_block(4.0 * 2.0 ** k)) == k                        # 4 2^k needs X = k
    assert int(numfmt.quantize_mxfp4_rows(np.zeros((1, 32), np.float32))[1][0, 0]) == 127   # zero block: X = 0
    tiny = np.zeros((1, 32), np.float32)
    tiny[0, 3] = np.float32(1e-45)                                  # a subnormal: X clamps to -127
    c, s = numfmt.quantize_mxfp4_rows(tiny)
    assert int(s[0, 0]) == 0 and c[0, 3] == 0                        # 1e-45 < 0.25 2^-127 rounds to 0


def test_mxfp4_exact_when_representable():
    """Blocks of E2M1 values times 2^X that hold +-6 2^X quantise exactly."""
    g = _g(42)
    rows, d = 6, 128
    codes = g.integers(0, 16, size=(rows, d)).astype(np.uint8)
    X = g.integers(-30, 30, size=(rows, d // 32))
    for r in range(rows):
        for b in range(d // 32):
            codes[r, 32 * b + (r + b) % 32] = 0x7 if (r + b) % 2 else 0xF
    x = (np.vectorize(E2M1.get)(codes) * np.repeat(2.0 ** X, 32, axis=1)).astype(np.float32)
    c, s = numfmt.quantize_mxfp4_rows(x)
    want = np.where(codes == 0x8, 0, codes)                          # -0 is stored as +0
    np.testing.assert_array_equal(c, want)
    np.testing.assert_array_equal(s.astype(np.int64), X + 127)
    np.testing.assert_array_equal(numfmt.mxfp4_decode_rows(c, s), x.astype(np.float64))


def test_mxfp4_error_bound_and_blocks_independent():
    """Each element decodes to within half the E2M1 gap at its magnitude
    (0.25 2^X below 2, 0.5 2^X up to 4, 2^X above), and a block's scale
    depends on its own 32 elements only."""
    g = _g(43)
    x = (g.standard_normal((50, 128)) * np.exp(g.uniform(-5, 5, (50, 1)))).astype(np.float32)
    c, s = numfmt.quantize_mxfp4_rows(x)
    dec = numfmt.mxfp4_decode_rows(c, s)
    p = np.repeat(2.0 ** (s.astype(np.int64) - 127), 32, axis=1)
    a = np.abs(x) / p
    half_gap = np.where(a <= 2, 0.25, np.where(a <= 4, 0.5, 1.0)) * p
    assert (np.abs(dec - x) <= half_gap).all()
    x2 = x.copy()
    x2[:, 32:64] *= 1000.0
    c2, s2 = numfmt.quantize_mxfp4_rows(x2)
    np.testing.assert_array_equal(c2[:, :32], c[:, :32])
    np.testing.assert_array_equal(s2[:, [0, 2, 3]], s[:, [0, 2, 3]])


def test_pack_e2m1_nibble_order():
    """Element 2j in the low nibble of byte j (reading R30)."""
    c = np.array([[0x1, 0x2, 0xF, 0x7]], dtype=np.uint8)
    p = numfmt.pack_e2m1(c)
    assert p.tolist() == [[0x21, 0x7F]]
    np.testing.assert_array_equal(numfmt.unpack_e2m1(p), c)
    r = _g(44).integers(0, 16, size=(7, 64)).astype(np.uint8)
    np.testing.assert_array_equal(numfmt.unpack_e2m1(numfmt.pack_e2m1(r)), r)


def test_index_score_fp4_brute_force():
    """Pure-Python sums over decoded values from the table above."""
    g = _g(45)
    H, D, N = 3, 64, 5
    qc = g.integers(0, 0x7F, size=(1, H, D)).astype(np.uint8) | (g.integers(0, 2, (1, H, D)) << 7).astype(np.uint8)
    qc[qc == 0xFF] = 0
    kc = g.integers(0, 16, size=(N, D)).astype(np.uint8)
    ks = g.integers(120, 134, size=(N, D // 32)).astype(np.uint8)
    w = g.standard_normal((1, H))
    got = oracle.index_score_fp4(qc, w, kc, ks)
    qv = numfmt.e4m3_decode(qc)
    for s in range(N):
        tot = 0.0
        for h in range(H):
            dot = math.fsum(float(qv[0, h, j]) * E2M1[int(kc[s, j])] * 2.0 ** (int(ks[s, j // 32]) - 127)
                            for j in range(D))
            tot += w[0, h] * max(dot, 0.0)
        assert got[0, s] == pytest.approx(tot, rel=1e-12, abs=1e-300)
    masked = oracle.index_score_fp4(qc, w, kc, ks, q_pos=[7], ratio=4)
    assert np.isneginf(masked[0, 2:]).all() and np.array_equal(masked[0, :2], got[0, :2])


def _mut_encode_ties_up(x):
    """E2M1 rounding with ties away from zero."""
    x = np.asarray(x, dtype=np.float64)
    return _ORIG["e2m1_encode"](x + np.sign(x) * 1e-9)


def _mut_e8m0_bias(s):
    return np.ldexp(1.0, np.asarray(s, dtype=np.int64) - 126)


def _mut_quantize_max4(x):
    """Block exponent chosen as if 4 were E2M1's largest magnitude."""
    f = np.asarray(x, dtype=np.float32).astype(np.float64)
    rows, d = f.shape
    blk = f.reshape(rows, d // 32, 32)
    amax = np.abs(blk).max(axis=2)
    X = np.where(amax > 0, np.ceil(np.log2(np.where(amax > 0, amax, 1) / 4.0)), 0).astype(np.int64)
    codes = numfmt.e2m1_encode(blk / np.ldexp(1.0, X)[:, :, None]).reshape(rows, d)
    return codes, (X + 127).astype(np.uint8)


def _mut_pack_swapped(c):
    c = np.asarray(c, dtype=np.uint8)
    return ((c[..., 0::2] << 4) | c[..., 1::2]).astype(np.uint8)


def _mut_decode_next_block(codes, scales):
    s = np.roll(np.asarray(scales), 1, axis=-1)
    return numfmt.e2m1_decode(codes) * np.repeat(numfmt.e8m0_decode(s), 32, axis=-1)


_ORIG = {"e2m1_encode": numfmt.e2m1_encode}


@pytest.mark.parametrize("name,mutant,pins", [
    ("e2m1_encode", _mut_encode_ties_up, ["test_e2m1_encode_ties_to_even_and_saturation"]),
    ("e8m0_decode", _mut_e8m0_bias, ["test_e8m0_decode", "test_mxfp4_exact_when_representable"]),
    ("quantize_mxfp4_rows", _mut_quantize_max4, ["test_mxfp4_scale_closed_forms",
                                                 "test_mxfp4_exact_when_representable"]),
    ("pack_e2m1", _mut_pack_swapped, ["test_pack_e2m1_nibble_order"]),
    ("mxfp4_decode_rows", _mut_decode_next_block, ["test_index_score_fp4_brute_force",
                                                   "test_mxfp4_exact_when_representable"]),
])
def test_mutation_fp4_pins_catch_planted_mistakes(monkeypatch, name, mutant, pins):
    """A planted slip in the oracle's FP4 codec fails the pins above: ties
    away from zero, an E8M0 bias of 126, a block exponent sized for 4 rather
    than 6, swapped nibbles, the neighbouring block's scale."""
    monkeypatch.setattr(numfmt, name, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            globals()[pin]()


def _fp4_state(g, D=16, di=64, H=4, W=6, m=1, max_comp=64):
    return oracle.LayerState(
        comp_kv=np.zeros((max_comp, D)), idx_keys=np.zeros((max_comp, di)), n_comp=0,
        swa=oracle.SwaRing(np.zeros((W, D))), main_bias=g.standard_normal((m, D)) * 0.1,
        idx_bias=g.standard_normal((m, di)) * 0.1, sink=g.standard_normal(H), m=m,
        idx_codes=np.zeros((max_comp, di), np.uint8), idx_scales=np.zeros((max_comp, di // 32), np.uint8),
        idx_fp4=True)


def test_decode_step_fp4_keys_equal_exact_keys_when_representable():
    """With ratio 1 the compressed key is the content row; rows of E2M1
    values times a per-block power of two holding +-6 2^X quantise exactly,
    so the FP4 step must match a float64 step over the same keys (with the
    E4M3 query's decoded values): codes, scales, scores, selection, output."""
    g = _g(46)
    D, di, H = 16, 64, 4
    Lf = _fp4_state(g, D=D, di=di, H=H)
    Lp = oracle.LayerState(comp_kv=np.zeros((64, D)), idx_keys=np.zeros((64, di)), n_comp=0,
                           swa=oracle.SwaRing(np.zeros((6, D))), main_bias=Lf.main_bias, idx_bias=Lf.idx_bias,
                           sink=Lf.sink, m=1)
    for pos in range(20):
        kc = g.integers(0, 16, size=(1, di)).astype(np.uint8)
        X = g.integers(-6, 6, size=di // 32)
        for b in range(di // 32):
            kc[0, 32 * b + (pos + b) % 32] = 0x7
        y = np.vectorize(E2M1.get)(kc) * np.repeat(2.0 ** X, 32)[None]
        qc = g.integers(0, 0x7F, size=(4, di)).astype(np.uint8)
        inp = dict(q=g.standard_normal((H, D)), w_idx=g.standard_normal(4), kv_new=g.standard_normal(D),
                   z_main=g.standard_normal((1, D)), c_main=g.standard_normal((1, D)),
                   z_idx=g.standard_normal((1, di)), c_idx=y)
        rp = oracle.decode_step(Lp, pos=pos, top_k=5, q_idx=numfmt.e4m3_decode(qc), **inp)
        rf = oracle.decode_step(Lf, pos=pos, top_k=5, q_idx=qc, **inp)
        np.testing.assert_array_equal(Lf.idx_codes[pos], np.where(kc[0] == 0x8, 0, kc[0]))
        np.testing.assert_array_equal(Lf.idx_scales[pos].astype(np.int64), X + 127)
        np.testing.assert_allclose(rf["scores"], rp["scores"], rtol=1e-13, atol=1e-300)
        np.testing.assert_array_equal(rf["idx"], rp["idx"])
        np.testing.assert_allclose(rf["out"], rp["out"], rtol=1e-12, atol=1e-13)


def test_decode_step_fp4_two_stage_is_composition():
    """With fp8_rescore the FP4 step keeps the bf16 key beside the codes and
    selects rescored_topk(FP4 scores, exact scores)."""
    g = _g(47)
    di = 64
    L = _fp4_state(g, di=di, m=4)
    L.fp8_rescore, L.round_cache = 6, numfmt.bf16_round_f64
    for pos in range(40):
        inp = dict(q=g.standard_normal((4, 16)), q_idx=g.standard_normal((4, di)), w_idx=g.standard_normal(4),
                   kv_new=g.standard_normal(16), z_main=g.standard_normal((4, 16)),
                   c_main=g.standard_normal((4, 16)), z_idx=g.standard_normal((4, di)),
                   c_idx=g.standard_normal((4, di)))
        r = oracle.decode_step(L, pos=pos, top_k=3, **inp)
        N = L.n_comp
        if r["new_entry"] is not None:
            y = np.asarray(r["new_entry"][1], np.float32)
            c, s = numfmt.quantize_mxfp4_rows(y[None])
            np.testing.assert_array_equal(L.idx_codes[N - 1], c[0])
            np.testing.assert_array_equal(L.idx_scales[N - 1], s[0])
            np.testing.assert_array_equal(L.idx_keys[N - 1], numfmt.bf16_round_f64(r["new_entry"][1]))
        qc, qs = numfmt.quantize_e4m3_rows(inp["q_idx"].astype(np.float32))
        s4 = oracle.index_score_fp4(qc[None], (inp["w_idx"].astype(np.float32) * qs).astype(np.float32)[None],
                                    L.idx_codes[:N], L.idx_scales[:N])[0]
        np.testing.assert_array_equal(r["scores"], s4)
        exact = oracle.index_score(inp["q_idx"][None], inp["w_idx"][None], L.idx_keys[:N])[0]
        want, wc = oracle.rescored_topk(s4[None], exact[None], 3, 6)
        np.testing.assert_array_equal(r["idx"], want[0])
        assert r["count"] == wc[0]
    assert L.n_comp == 10


# ---------------------------------------------------------------------------
# recall (page 1, ARCHITECTURE_AND_MEMORY_AUDIT.md, Tier 1 gate 4)
# ---------------------------------------------------------------------------

def _fp4_workload_scores(seed, n):
    g = synth.rng(seed)
    f = numfmt.bf16_bits_to_f64
    K = f(synth.to_bf16_bits(g.standard_normal((n, 128), dtype=np.float32)))
    q = f(synth.to_bf16_bits(g.standard_normal((64, 128), dtype=np.float32) / np.float32(np.sqrt(128))))
    w = g.standard_normal(64).astype(np.float32)
    exact = oracle.index_score(q[None], w[None].astype(np.float64), K)[0]
    kc, ks = numfmt.quantize_mxfp4_rows(K.astype(np.float32))
    qc, qs = numfmt.quantize_e4m3_rows(q.astype(np.float32))
    s4 = oracle.index_score_fp4(qc[None], (w * qs).astype(np.float32)[None], kc, ks)[0]
    return exact, s4


def _recall(sel, exact, k):
    ref = set(oracle.topk(exact[None], k)[0][0].tolist())
    return len(ref & set(sel[:k].tolist())) / k


def test_fp4_recall_study_at_1m_context():
    """FP4 keys alone miss the gate by far; the 1024 best by FP4 score do
    not hold enough of the exact top-512 either; the 2048 best do."""
    exact, s4 = _fp4_workload_scores(4100, 250_000)
    plain = _recall(oracle.topk(s4[None], 512)[0][0], exact, 512)
    r1k = _recall(oracle.rescored_topk(s4[None], exact[None], 512, 1024)[0][0], exact, 512)
    r2k = _recall(oracle.rescored_topk(s4[None], exact[None], 512, 2048)[0][0], exact, 512)
    print(f"top-512 recall at n=250000, FP4 keys: plain {plain:.4f}; top-1024 then exact {r1k:.4f}; "
          f"top-2048 then exact {r2k:.4f}")
    assert plain < 0.9
    assert r1k < 0.99
    assert r2k >= 0.99


def test_fp4_recall_small_n_gate():
    for seed, n in ((4101, 1024), (4102, 4096)):
        exact, s4 = _fp4_workload_scores(seed, n)
        assert _recall(oracle.rescored_topk(s4[None], exact[None], 512, 2048)[0][0], exact, 512) >= 0.99
