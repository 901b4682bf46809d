"""Pins for the CPU oracle: every oracle function checked against something
other than itself — hand-derived closed forms (tests/golden/), invariants the
mathematics fixes, special cases that reduce to a textbook formula, and brute
force on tiny inputs.  Each pin is chosen so a plausible mistake (a dropped
term, a wrong sign or index, the wrong softmax axis, the bias leaking into C)
fails it; the ``test_mutation_*`` tests plant such mistakes in wrapped copies
of the oracle and check that the pins reject them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import numfmt
from tests.conftest import GOLDEN

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _num(x):
    if isinstance(x, str):
        return float(x)  # "-inf", "-0.0"
    if isinstance(x, list):
        return [_num(v) for v in x]
    return x


def _g(seed):
    return np.random.Generator(np.random.PCG64(seed))


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def test_bf16_decode_known_patterns():
    bits = np.array([0x3F80, 0xC000, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x3FC0, 0x7F80, 0xFF80],
                    dtype=np.uint16)
    v = numfmt.bf16_bits_to_f64(bits)
    exp = [1.0, -2.0, 0.0, -0.0, (2 - 2 ** -7) * 2.0 ** 127, 2.0 ** -133, 1.5, math.inf, -math.inf]
    assert list(v) == exp
    assert math.copysign(1.0, v[3]) == -1.0


def test_bf16_decode_matches_torch():
    import torch
    bits = _g(1).integers(0, 1 << 16, size=4096, dtype=np.uint16)
    exp_mask = (bits >> 7) & 0xFF
    bits = bits[exp_mask != 0xFF]  # drop inf/NaN patterns
    ours = numfmt.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(ours, ref)


def test_f32_to_bf16_matches_torch_rne():
    import torch
    g = _g(2)
    x = np.concatenate([g.standard_normal(4096).astype(np.float32) * 10,
                        # exact halfway cases: 1 + 2^-8 (tie -> even 1.0), 1 + 3*2^-8 (tie -> up)
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8)], dtype=np.float32)])
    ours = numfmt.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    assert numfmt.bf16_bits_to_f64(ours[-3:]).tolist() == [1.0, 1 + 2 ** -6, -1.0]


def test_f64_to_bf16_single_rounding():
    # just above a bf16 halfway point, below float32 resolution: one rounding
    # from float64 goes up; a float32 detour would land on the tie and go to even
    x = 1.0 + 2.0 ** -8 + 2.0 ** -30
    assert numfmt.bf16_round_f64(np.array([x]))[0] == 1.0 + 2.0 ** -7
    assert numfmt.bf16_round_f64(np.array([1.0 + 2.0 ** -8]))[0] == 1.0          # tie -> even
    assert numfmt.bf16_round_f64(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6
    assert numfmt.bf16_round_f64(np.array([2.0 ** -134 * 1.5]))[0] == 2.0 ** -133  # subnormal
    assert numfmt.bf16_round_f64(np.array([3.0e38 * 1.2]))[0] == math.inf
    b = numfmt.f64_to_bf16_bits(np.array([1.0, -2.0]))
    assert b.tolist() == [0x3F80, 0xC000]


# ---------------------------------------------------------------------------
# (1) compressor reduce
# ---------------------------------------------------------------------------

def _check_compress_golden(fn):
    for c in _load("compress_hand.json")["cases"]:
        y = fn(np.array(c["Z"]), np.array(c["C"]), np.array(c["B"]), c["m"], overlap=c["overlap"])
        np.testing.assert_allclose(y, np.array(c["expect"]), rtol=0, atol=1e-13, err_msg=c["name"])


def _check_compress_weights(fn, m=4, D=6, seed=3):
    """Extract the softmax weights through one-hot C and check the closed form."""
    g = _g(seed)
    Z = g.standard_normal((m, D)) * 3
    B = g.standard_normal((m, D)) * 0.5
    w = np.empty((m, D))
    for t in range(m):
        C = np.zeros((m, D))
        C[t] = 1.0
        w[t] = fn(Z, C, B, m)[0]
    np.testing.assert_allclose(w.sum(axis=0), 1.0, rtol=0, atol=1e-15)
    for c in range(D):
        for t in range(1, m):
            # p_t / p_0 = exp(l_t - l_0) with l = Z + B (bias on the logits)
            r = w[t, c] / w[0, c]
            e = math.exp((Z[t, c] + B[t, c]) - (Z[0, c] + B[0, c]))
            assert abs(r - e) <= 1e-12 * e


def _check_compress_bias_leak(fn, m=4, D=8, seed=4):
    """C constant per channel => output is that constant, whatever Z and B."""
    g = _g(seed)
    Z = g.standard_normal((3 * m, D)) * 4
    B = g.standard_normal((m, D)) * 2
    const = g.standard_normal(D)
    C = np.tile(const, (3 * m, 1))
    np.testing.assert_allclose(fn(Z, C, B, m), np.tile(const, (3, 1)), rtol=0, atol=1e-14)


def test_compress_golden():
    _check_compress_golden(oracle.compress)


def test_compress_weights_are_softmax_of_z_plus_b():
    _check_compress_weights(oracle.compress)


def test_compress_bias_never_reaches_c():
    _check_compress_bias_leak(oracle.compress)


def test_compress_shift_invariance():
    g = _g(5)
    m, D = 4, 16
    Z = g.standard_normal((2 * m, D))
    C = g.standard_normal((2 * m, D))
    B = g.standard_normal((m, D)) * 0.1
    y0 = oracle.compress(Z, C, B, m)
    sz = g.standard_normal(D) * 7
    sb = g.standard_normal(D) * 7
    np.testing.assert_allclose(oracle.compress(Z + sz, C, B, m), y0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.compress(Z, C, B + sb, m), y0, rtol=0, atol=1e-13)
    # a per-row shift is NOT an invariance: it changes the weights
    shifted = Z.copy()
    shifted[0] += 1.0
    assert np.abs(oracle.compress(shifted, C, B, m) - y0).max() > 1e-3


def test_compress_special_cases():
    g = _g(6)
    D = 10
    # m = 1: the softmax over one row is 1, so the output is C itself
    Z, C, B = g.standard_normal((5, D)), g.standard_normal((5, D)), g.standard_normal((1, D))
    np.testing.assert_allclose(oracle.compress(Z, C, B, 1), C, rtol=0, atol=0)
    # equal logits and zero bias: the block mean
    C = g.standard_normal((4, D))
    np.testing.assert_allclose(oracle.compress(np.ones((4, D)) * 0.3, C, np.zeros((4, D)), 4),
                               C.mean(axis=0, keepdims=True), rtol=0, atol=1e-15)
    # one logit 50 above the rest takes (almost) all the weight
    Z = np.zeros((4, D))
    Z[2] = 50.0
    y = oracle.compress(Z, C, np.zeros((4, D)), 4)
    np.testing.assert_allclose(y[0], C[2], rtol=0, atol=8 * math.exp(-50) * np.abs(C).max())
    # huge logits stay finite (max subtraction)
    Z = g.standard_normal((4, D)) + 900.0
    y = oracle.compress(Z, C, np.zeros((4, D)), 4)
    np.testing.assert_allclose(y, oracle.compress(Z - 900.0, C, np.zeros((4, D)), 4), rtol=1e-12, atol=1e-12)


def test_compress_tail_rows_ignored():
    g = _g(7)
    Z, C = g.standard_normal((11, 4)), g.standard_normal((11, 4))
    B = g.standard_normal((4, 4))
    y = oracle.compress(Z, C, B, 4)
    assert y.shape == (2, 4)
    Z2, C2 = Z.copy(), C.copy()
    Z2[8:] += 100.0
    C2[8:] -= 100.0
    np.testing.assert_array_equal(oracle.compress(Z2, C2, B, 4), y)


def test_compress_overlap_reduces_to_plain_blocks():
    """Overlapped block 0 is the plain reduce of the b half; block i>0 is the plain
    reduce (ratio 2m) of [a half of block i-1 ; b half of block i]."""
    g = _g(8)
    m, D, nb = 4, 6, 4
    Z = g.standard_normal((nb * m, 2 * D))
    C = g.standard_normal((nb * m, 2 * D))
    B = g.standard_normal((m, 2 * D)) * 0.3
    y = oracle.compress(Z, C, B, m, overlap=True)
    a, b = slice(0, D), slice(D, 2 * D)
    np.testing.assert_allclose(y[0], oracle.compress(Z[:m, b], C[:m, b], B[:, b], m)[0], rtol=0, atol=1e-15)
    for i in range(1, nb):
        Zi = np.concatenate([Z[(i - 1) * m:i * m, a], Z[i * m:(i + 1) * m, b]])
        Ci = np.concatenate([C[(i - 1) * m:i * m, a], C[i * m:(i + 1) * m, b]])
        Bi = np.concatenate([B[:, a], B[:, b]])
        np.testing.assert_allclose(y[i], oracle.compress(Zi, Ci, Bi, 2 * m)[0], rtol=0, atol=1e-15)
    # the a half of the last block is never used
    Z2, C2 = Z.copy(), C.copy()
    Z2[(nb - 1) * m:, a] = 77.0
    C2[(nb - 1) * m:, a] = -77.0
    np.testing.assert_array_equal(oracle.compress(Z2, C2, B, m, overlap=True), y)


def test_kv_norm_closed_forms():
    w = np.array([1.0, 2.0, -1.0, 0.5])
    a = 3.0
    y = oracle.kv_norm(np.full((1, 4), a), w)
    np.testing.assert_allclose(y[0], a / math.sqrt(a * a + 1e-6) * w, rtol=1e-15)
    g = _g(9)
    x = g.standard_normal((3, 64))
    y1 = oracle.kv_norm(x, np.ones(64))
    ms = (y1 ** 2).mean(axis=1)
    np.testing.assert_allclose(ms, (x ** 2).mean(axis=1) / ((x ** 2).mean(axis=1) + 1e-6), rtol=1e-14)


def test_mutation_compress_pins_catch_planted_mistakes():
    def bias_on_c(Z, C, B, m, overlap=False):  # the bug the pages fixed
        reps = np.asarray(Z).shape[0] // m
        Cb = np.asarray(C, dtype=float).copy()
        Cb[:reps * m] += np.tile(B, (reps, 1))
        return oracle.compress(Z, Cb, B, m, overlap)

    def wrong_axis(Z, C, B, m, overlap=False):  # softmax across channels, not rows
        Z, C = np.asarray(Z, float), np.asarray(C, float)
        out = []
        for i in range(Z.shape[0] // m):
            L = Z[i * m:(i + 1) * m] + B
            p = np.exp(L - L.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            out.append((p * C[i * m:(i + 1) * m]).sum(axis=0))
        return np.array(out)

    def no_bias(Z, C, B, m, overlap=False):
        return oracle.compress(Z, C, np.zeros_like(np.asarray(B, dtype=float)), m, overlap)

    with pytest.raises(AssertionError):
        _check_compress_bias_leak(bias_on_c)
    with pytest.raises(AssertionError):
        _check_compress_golden(bias_on_c)
    with pytest.raises(AssertionError):
        _check_compress_weights(wrong_axis, m=4, D=6)
    with pytest.raises(AssertionError):
        _check_compress_weights(no_bias)


# ---------------------------------------------------------------------------
# (2) lightning-indexer score
# ---------------------------------------------------------------------------

def _check_index_golden(fn):
    for c in _load("index_score_hand.json")["cases"]:
        got = fn(np.array(c["q"]), np.array(c["w"]), np.array(c["K"]),
                 q_pos=c.get("q_pos"))
        np.testing.assert_array_equal(got, np.array(_num(c["expect"])), err_msg=c["name"])


def test_index_score_golden():
    _check_index_golden(oracle.index_score)


def test_index_score_single_head_is_relu_matvec():
    g = _g(10)
    q = g.standard_normal((1, 1, 7))
    K = g.standard_normal((9, 7))
    got = oracle.index_score(q, np.ones((1, 1)), K)[0]
    for s in range(9):
        dot = 0.0
        for d in range(7):
            dot += q[0, 0, d] * K[s, d]
        assert abs(got[s] - max(dot, 0.0)) <= 1e-14


def test_index_score_linear_in_w_and_relu_split():
    g = _g(11)
    T, H, d, N = 2, 8, 16, 30
    q = g.standard_normal((T, H, d))
    K = g.standard_normal((N, d))
    w1, w2 = g.standard_normal((T, H)), g.standard_normal((T, H))
    I1, I2 = oracle.index_score(q, w1, K), oracle.index_score(q, w2, K)
    np.testing.assert_allclose(oracle.index_score(q, 2 * w1 - 3 * w2, K), 2 * I1 - 3 * I2, rtol=1e-12, atol=1e-12)
    # ReLU(x) - ReLU(-x) = x  =>  I(q) - I(-q) = K @ (sum_h w_h q_h)
    lin = np.einsum("th,thd->td", w1, q) @ K.T
    np.testing.assert_allclose(I1 - oracle.index_score(-q, w1, K), lin, rtol=1e-12, atol=1e-12)
    # non-negative weights give non-negative scores
    assert (oracle.index_score(q, np.abs(w1), K) >= 0).all()


def test_index_score_key_is_shared_across_heads():
    """F3: the stored key is [N, d_I]; a per-head [N, H, d_I] key is rejected."""
    g = _g(12)
    q = g.standard_normal((1, 4, 8))
    with pytest.raises(ValueError):
        oracle.index_score(q, np.ones((1, 4)), g.standard_normal((5, 4, 8)))


def test_index_score_causal_visible_counts():
    q = np.ones((1, 1, 1))
    K = np.ones((40, 1))
    for p in range(0, 150, 7):
        row = oracle.index_score(q, np.ones((1, 1)), K, q_pos=[p])[0]
        visible = int(np.isfinite(row).sum())
        assert visible == min(40, (p + 1) // 4)
        assert np.isfinite(row[:visible]).all() and not np.isfinite(row[visible:]).any()


def test_mutation_index_pins_catch_planted_mistakes():
    def no_relu(q, w, K, q_pos=None, ratio=4):
        q = np.asarray(q, float)
        return np.einsum("th,thn->tn", np.asarray(w, float), q @ np.asarray(K, float).T)

    def off_by_one_mask(q, w, K, q_pos=None, ratio=4):
        out = oracle.index_score(q, w, K)
        if q_pos is not None:
            ends = ratio * np.arange(out.shape[1]) + ratio - 1
            out[(ends - 1)[None, :] > np.asarray(q_pos)[:, None]] = -np.inf
        return out

    with pytest.raises(AssertionError):
        _check_index_golden(no_relu)
    with pytest.raises(AssertionError):
        _check_index_golden(off_by_one_mask)


# ---------------------------------------------------------------------------
# (3) top-k
# ---------------------------------------------------------------------------

def _check_topk_golden(fn):
    for c in _load("topk_hand.json")["cases"]:
        idx, cnt = fn(np.array([_num(c["scores"])]), c["k"])
        assert idx[0].tolist() == c["expect_idx"], c
        assert int(cnt[0]) == c["expect_count"], c


def test_topk_golden():
    _check_topk_golden(oracle.topk)


@pytest.mark.parametrize("seed", range(40))
def test_topk_brute_force(seed):
    g = _g(100 + seed)
    N = int(g.integers(1, 48))
    k = int(g.integers(1, 60))
    s = g.integers(-3, 4, size=N).astype(float)  # many ties
    s[g.random(N) < 0.2] = -np.inf
    idx, cnt = oracle.topk(s[None], k)
    valid = [i for i in range(N) if s[i] != -np.inf]
    ranked = sorted(valid, key=lambda i: (-s[i], i))[:k]
    assert idx[0, :len(ranked)].tolist() == ranked
    assert (idx[0, len(ranked):] == -1).all()
    assert cnt[0] == min(k, len(valid))


def test_topk_invariants_large():
    g = _g(13)
    s = g.standard_normal((3, 5000))
    k = 300
    idx, cnt = oracle.topk(s, k)
    for t in range(3):
        sel = idx[t]
        assert len(set(sel.tolist())) == k and cnt[t] == k
        mask = np.zeros(5000, bool)
        mask[sel] = True
        assert s[t, mask].min() >= s[t, ~mask].max()
        assert (np.diff(s[t, sel]) <= 0).all()


def test_mutation_topk_pins_catch_planted_mistakes():
    def higher_index_wins(scores, k):
        s = np.asarray(scores, float)
        idx, cnt = oracle.topk(s[:, ::-1], k)
        N = s.shape[1]
        return np.where(idx >= 0, N - 1 - idx, -1), cnt

    def signed_zero_order(scores, k):
        s = np.asarray(scores, float)
        s = np.where((s == 0) & np.signbit(s), -1e-300, s)
        return oracle.topk(s, k)

    with pytest.raises(AssertionError):
        _check_topk_golden(higher_index_wins)
    with pytest.raises(AssertionError):
        _check_topk_golden(signed_zero_order)


# ---------------------------------------------------------------------------
# (4) gather
# ---------------------------------------------------------------------------

def test_gather_golden():
    for c in _load("gather_hand.json")["cases"]:
        rows, nv = oracle.gather(np.array(c["comp_kv"]), np.array(c["idx"]), c["count"],
                                 np.array(c["swa"]), c["swa_head"], c["swa_len"])
        assert rows.tolist() == c["expect_rows"] and nv == c["expect_n_valid"]


def test_gather_wrap_is_chronological():
    W, D = 8, 3
    g = _g(14)
    ring = oracle.SwaRing(np.zeros((W, D)))
    history = []
    for p in range(29):  # wraps three times and ends with head = 29 % 8 = 5
        row = g.standard_normal(D)
        ring.append(row)
        history.append(row)
    assert ring.head == 29 % W and ring.length == W
    rows, nv = oracle.gather(np.zeros((1, D)), np.array([-1]), 0, ring.rows, ring.head, ring.length)
    np.testing.assert_array_equal(rows, np.stack(history[-W:]))
    assert nv == W


# ---------------------------------------------------------------------------
# (5) sparse attention with a sink
# ---------------------------------------------------------------------------

def _check_attn_golden(fn):
    for c in _load("attn_hand.json")["cases"]:
        q = np.array(c["q"], dtype=float)
        kv = np.array(c["kv"], dtype=float).reshape(-1, q.shape[1])
        out, lse = fn(q, kv, None if c["sink"] is None else np.array(c["sink"]), c["scale"])
        np.testing.assert_allclose(out, np.array(c["expect_out"]), rtol=1e-14, atol=1e-15, err_msg=c["name"])
        np.testing.assert_allclose(lse, np.array(c["expect_lse"]), rtol=1e-14, err_msg=c["name"])


def test_attn_golden():
    _check_attn_golden(oracle.sparse_attn)


def test_attn_sink_to_minus_inf_is_plain_softmax():
    g = _g(15)
    q, kv = g.standard_normal((4, 16)), g.standard_normal((9, 16))
    o1, l1 = oracle.sparse_attn(q, kv, np.full(4, -np.inf))
    o2, l2 = oracle.sparse_attn(q, kv, None)
    np.testing.assert_array_equal(o1, o2)
    # plain softmax attention, written as the textbook formula
    s = q @ kv.T / 4.0
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    np.testing.assert_allclose(o2, p @ kv, rtol=1e-13, atol=1e-14)


def test_attn_one_row_closed_form():
    g = _g(16)
    D = 8
    q, v = g.standard_normal((3, D)), g.standard_normal((1, D))
    sink = g.standard_normal(3)
    out, lse = oracle.sparse_attn(q, v, sink)
    s = q @ v[0] / math.sqrt(D)
    sig = 1.0 / (1.0 + np.exp(-(s - sink)))
    np.testing.assert_allclose(out, sig[:, None] * v, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, np.log(np.exp(s) + np.exp(sink)), rtol=1e-13)


def test_attn_identical_rows_closed_form():
    g = _g(17)
    D, n = 8, 5
    q, v = g.standard_normal((2, D)), g.standard_normal(D)
    sink = np.array([0.3, -1.2])
    out, _ = oracle.sparse_attn(q, np.tile(v, (n, 1)), sink)
    s = q @ v / math.sqrt(D)
    np.testing.assert_allclose(out, (n / (n + np.exp(sink - s)))[:, None] * v, rtol=1e-13, atol=1e-15)


def test_attn_permutation_invariance_and_weights():
    g = _g(18)
    q, kv = g.standard_normal((4, 32)), g.standard_normal((20, 32))
    sink = g.standard_normal(4)
    o1, l1, w, ws = oracle.sparse_attn(q, kv, sink, return_weights=True)
    perm = g.permutation(20)
    o2, l2 = oracle.sparse_attn(q, kv[perm], sink)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(l1, l2, rtol=1e-14)
    np.testing.assert_allclose(w.sum(1) + ws, 1.0, rtol=0, atol=1e-14)
    s = q @ kv.T / math.sqrt(32)
    np.testing.assert_allclose(w[:, 3] / w[:, 7], np.exp(s[:, 3] - s[:, 7]), rtol=1e-12)
    np.testing.assert_allclose(ws / w[:, 0], np.exp(sink - s[:, 0]), rtol=1e-12)


def test_attn_large_logits_stable():
    q = np.full((1, 4), 30.0)
    kv = np.array([[30.0] * 4, [29.0] * 4])
    out, lse = oracle.sparse_attn(q, kv, np.array([0.0]))
    assert np.isfinite(out).all() and np.isfinite(lse).all()


def test_mutation_attn_pins_catch_planted_mistakes():
    def sink_in_numerator(q, kv, sink=None, scale=None):  # sink given a value row of ones
        if sink is None or len(kv) == 0:
            return oracle.sparse_attn(q, kv, sink, scale)
        out, lse, w, ws = oracle.sparse_attn(q, kv, sink, scale, return_weights=True)
        return out + ws[:, None], lse

    def sink_scaled_again(q, kv, sink=None, scale=None):
        sc = 1.0 / math.sqrt(np.asarray(q).shape[1]) if scale is None else scale
        return oracle.sparse_attn(q, kv, None if sink is None else np.asarray(sink) * sc + 0.5, scale)

    with pytest.raises(AssertionError):
        _check_attn_golden(sink_in_numerator)
    with pytest.raises(AssertionError):
        _check_attn_golden(sink_scaled_again)


# ---------------------------------------------------------------------------
# (6) decode step
# ---------------------------------------------------------------------------

def _empty_state(g, D=16, di=8, H=4, W=8, max_comp=64, m=4):
    return oracle.LayerState(
        comp_kv=np.zeros((max_comp, D)), idx_keys=np.zeros((max_comp, di)), n_comp=0,
        swa=oracle.SwaRing(np.zeros((W, D))), main_bias=g.standard_normal((m, D)) * 0.1,
        idx_bias=g.standard_normal((m, di)) * 0.1, sink=g.standard_normal(H), m=m)


def _step_inputs(g, D=16, di=8, H=4, Hi=4, m=4):
    return dict(q=g.standard_normal((H, D)), q_idx=g.standard_normal((Hi, di)),
                w_idx=g.standard_normal(Hi), kv_new=g.standard_normal(D),
                z_main=g.standard_normal((m, D)), c_main=g.standard_normal((m, D)),
                z_idx=g.standard_normal((m, di)), c_idx=g.standard_normal((m, di)))


def test_decode_step_state_advances():
    g = _g(19)
    L = _empty_state(g)
    for pos in range(23):
        r = oracle.decode_step(L, pos=pos, top_k=3, **_step_inputs(g))
        assert L.n_comp == (pos + 1) // 4
        assert L.swa.length == min(pos + 1, 8) and L.swa.head == (pos + 1) % 8
        assert r["count"] == min(3, L.n_comp)
        assert r["n_valid"] == r["count"] + L.swa.length
        assert (r["new_entry"] is not None) == (pos % 4 == 3)


def test_decode_step_sees_new_token_and_new_block():
    g = _g(20)
    L = _empty_state(g)
    L.sink = None
    inp = _step_inputs(g)
    r = oracle.decode_step(L, pos=0, top_k=2, **inp)
    # one SWA row, nothing compressed, no sink: attention returns that row
    np.testing.assert_allclose(r["out"], np.tile(inp["kv_new"], (4, 1)), rtol=1e-15)
    for pos in (1, 2):
        oracle.decode_step(L, pos=pos, top_k=2, **_step_inputs(g))
    inp = _step_inputs(g)
    r = oracle.decode_step(L, pos=3, top_k=2, **inp)
    assert L.n_comp == 1 and r["count"] == 1 and r["idx"].tolist() == [0, -1]
    np.testing.assert_allclose(r["rows"][0], oracle.compress(inp["z_main"], inp["c_main"], L.main_bias, 4)[0])


def test_decode_step_sparse_equals_dense_when_k_covers_all():
    """top_k >= n_comp: sparse attention equals dense attention over [comp_kv; SWA]."""
    g = _g(21)
    L = _empty_state(g)
    for pos in range(30):
        oracle.decode_step(L, pos=pos, top_k=64, **_step_inputs(g))
    inp = _step_inputs(_g(999))
    q = inp["q"]
    r = oracle.decode_step(L, pos=30, top_k=64, **inp)
    dense_rows = np.concatenate([L.comp_kv[:L.n_comp],
                                 np.stack([L.swa.rows[(L.swa.head - L.swa.length + j) % 8]
                                           for j in range(L.swa.length)])])
    out_d, lse_d = oracle.sparse_attn(q, dense_rows, L.sink)
    np.testing.assert_allclose(r["out"], out_d, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(r["lse"], lse_d, rtol=1e-13)


def test_decode_step_cache_rounding_applies():
    g = _g(22)
    L = _empty_state(g)
    L.round_cache = numfmt.bf16_round_f64
    inp = _step_inputs(g)
    for pos in range(3):
        oracle.decode_step(L, pos=pos, top_k=2, **_step_inputs(g))
    oracle.decode_step(L, pos=3, top_k=2, **inp)
    exact = oracle.compress(inp["z_main"], inp["c_main"], L.main_bias, 4)[0]
    np.testing.assert_array_equal(L.comp_kv[0], numfmt.bf16_round_f64(exact))


def _e4m3_codes(g, shape):
    """Random finite E4M3 codes of either sign (0x7F / 0xFF are NaN)."""
    mag = g.integers(0, 0x7F, size=shape).astype(np.uint8)
    return mag | (g.integers(0, 2, size=shape).astype(np.uint8) << 7)


def test_decode_step_fp8_keys_equal_exact_keys_when_representable():
    """E4M3 indexer keys lose nothing when every key is an E4M3 value times a
    power of two and carries +-448 times that power (so max|row| / 448 is the
    power itself): with ratio 1 the compressed key is the content row, its
    quantisation is exact, and a step over E4M3 keys must match the step over
    the same keys in float64 — scores, selection and output — as must the
    stored codes and scales."""
    g = _g(26)
    D, di, H, W = 16, 8, 4, 6
    Lp = _empty_state(g, D=D, di=di, H=H, W=W, m=1)
    Lf = _empty_state(g, D=D, di=di, H=H, W=W, m=1)
    Lf.main_bias, Lf.idx_bias, Lf.sink = Lp.main_bias, Lp.idx_bias, Lp.sink
    Lf.idx_codes = np.zeros((64, di), dtype=np.uint8)
    Lf.idx_scales = np.zeros(64, dtype=np.float32)
    for pos in range(20):
        inp = _step_inputs(g, D=D, di=di, H=H, m=1)
        kc = _e4m3_codes(g, (1, di))
        kc[0, pos % di] = 0x7E | (0x80 if pos % 3 == 0 else 0)   # +-448
        inp["c_idx"] = numfmt.e4m3_decode(kc) * 0.125
        qc = _e4m3_codes(g, (4, di))
        rp = oracle.decode_step(Lp, pos=pos, top_k=5, **{**inp, "q_idx": numfmt.e4m3_decode(qc)})
        rf = oracle.decode_step(Lf, pos=pos, top_k=5, **{**inp, "q_idx": qc})
        np.testing.assert_array_equal(Lf.idx_codes[pos], kc[0])
        assert Lf.idx_scales[pos] == np.float32(0.125)
        np.testing.assert_allclose(rf["scores"], rp["scores"], rtol=1e-13, atol=1e-300)
        np.testing.assert_array_equal(rf["idx"], rp["idx"])
        np.testing.assert_allclose(rf["out"], rp["out"], rtol=1e-12, atol=1e-13)
    assert Lf.n_comp == Lp.n_comp == 20


def test_decode_step_fp8_key_within_e4m3_rounding():
    """General compressor inputs: each stored E4M3 key decodes to within half
    a unit of E4M3's last place of the float32 compressed key (3 significand
    bits: relative 2^-4 in the normal range, absolute 2^-10 times the scale
    below 2^-6), and the key's largest magnitude is stored as +-448."""
    g = _g(27)
    di = 32
    L = _empty_state(g, di=di)
    L.idx_codes = np.zeros((64, di), dtype=np.uint8)
    L.idx_scales = np.zeros(64, dtype=np.float32)
    for pos in range(16):
        inp = _step_inputs(g, di=di)
        inp["q_idx"] = _e4m3_codes(g, (4, di))
        r = oracle.decode_step(L, pos=pos, **inp, top_k=3)
        if r["new_entry"] is None:
            continue
        y = np.asarray(r["new_entry"][1], dtype=np.float32).astype(np.float64)
        j = L.n_comp - 1
        sc = float(L.idx_scales[j])
        dec = numfmt.e4m3_decode(L.idx_codes[j]) * sc
        assert sc == pytest.approx(np.abs(y).max() / 448, rel=1e-6)
        bound = np.maximum(np.abs(y) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6)
        assert (np.abs(dec - y) <= bound).all()
        assert (L.idx_codes[j][np.argmax(np.abs(y))] & 0x7F) == 0x7E
    assert L.n_comp == 4


def test_decode_step_fp8_float_query_quantised_and_folded():
    """Over E4M3 keys a real-valued query is quantised per head row and each
    row's scale folded into its head weight (reading R20).  Head rows that are
    E4M3 values times a power of two p_h, with +-448 present, quantise exactly
    (codes = those values, scale = p_h): the step must equal the step given
    those codes and w * p_h.  And doubling the query doubles every score (a
    step that dropped the scale would not move)."""
    g = _g(29)
    D, di, H, W, Hi = 16, 8, 4, 6, 4
    states = []
    for _ in range(3):
        L = _empty_state(g, D=D, di=di, H=H, W=W)
        L.idx_codes = np.zeros((64, di), dtype=np.uint8)
        L.idx_scales = np.zeros(64, dtype=np.float32)
        states.append(L)
    for L in states[1:]:
        L.main_bias, L.idx_bias, L.sink = states[0].main_bias, states[0].idx_bias, states[0].sink
    La, Lb, Lc = states
    for pos in range(14):
        inp = _step_inputs(g, D=D, di=di, H=H, Hi=Hi)
        qc = _e4m3_codes(g, (Hi, di))
        qc[np.arange(Hi), (pos + np.arange(Hi)) % di] = 0x7E | (0x80 * (np.arange(Hi) % 2)).astype(np.uint8)
        p = np.float32(2.0) ** g.integers(-6, 3, size=Hi).astype(np.float32)
        qv = numfmt.e4m3_decode(qc) * p[:, None].astype(np.float64)
        w = inp["w_idx"].astype(np.float32)
        ra = oracle.decode_step(La, pos=pos, top_k=5, **{**inp, "q_idx": qv, "w_idx": w})
        rb = oracle.decode_step(Lb, pos=pos, top_k=5, **{**inp, "q_idx": qc, "w_idx": (w * p).astype(np.float32)})
        rc = oracle.decode_step(Lc, pos=pos, top_k=5, **{**inp, "q_idx": 2 * qv, "w_idx": w})
        np.testing.assert_array_equal(ra["scores"], rb["scores"])
        np.testing.assert_array_equal(rc["scores"], 2 * ra["scores"])
        np.testing.assert_array_equal(ra["idx"], rb["idx"])
        if La.n_comp:
            assert np.abs(ra["scores"]).max() > 0
    assert La.n_comp == 3


def _rope_tables(n_pos, rd, base=10000.0, offset=0.0):
    """cos / sin rows of angle (p + offset) * base^(-2j/rd) (a test table)."""
    ang = (np.arange(n_pos)[:, None] + offset) * base ** (-2.0 * np.arange(rd // 2)[None, :] / rd)
    return np.cos(ang), np.sin(ang)


def test_rope_rotation_closed_forms():
    """The printed inverse, and the forward as its inverse: a quarter turn
    maps the pair (e, o) to (-o, e); inverse(forward(x)) = x; the NoPE part is
    untouched; pair norms are kept; and the score of two rotated vectors
    depends only on the difference of their positions."""
    g = _g(28)
    x = g.standard_normal((3, 24))
    c, s = np.zeros(4), np.ones(4)
    f = oracle.rope_rotate(x, c, s)
    np.testing.assert_array_equal(f[:, :16], x[:, :16])
    np.testing.assert_allclose(f[:, 16::2], -x[:, 17::2], atol=0)
    np.testing.assert_allclose(f[:, 17::2], x[:, 16::2], atol=0)
    inv = oracle.rope_rotate(x, c, s, inverse=True)
    np.testing.assert_allclose(inv[:, 16::2], x[:, 17::2], atol=0)
    np.testing.assert_allclose(inv[:, 17::2], -x[:, 16::2], atol=0)
    cos, sin = _rope_tables(50, 8)
    for p in (0, 7, 49):
        y = oracle.rope_rotate(x, cos[p], sin[p])
        np.testing.assert_allclose(oracle.rope_rotate(y, cos[p], sin[p], inverse=True), x, rtol=1e-14, atol=1e-14)
        pn = lambda a: a[:, 16::2] ** 2 + a[:, 17::2] ** 2
        np.testing.assert_allclose(pn(y), pn(x), rtol=1e-13)
    q, k = g.standard_normal(24), g.standard_normal(24)
    dots = [oracle.rope_rotate(q, cos[p + 5], sin[p + 5]) @ oracle.rope_rotate(k, cos[p], sin[p]) for p in (0, 9, 30)]
    np.testing.assert_allclose(dots, dots[0], rtol=1e-12)
    np.testing.assert_allclose(dots[0], oracle.rope_rotate(q, cos[5], sin[5]) @ k, rtol=1e-12)


def test_mixed_kv_row_exact_and_bounded():
    """A row whose NoPE part is E4M3 values times a power of two (carrying
    +-448 times it) and whose RoPE part is bfloat16 comes back exactly with a
    zero rotation; a general row within E4M3 / bfloat16 rounding."""
    g = _g(29)
    codes = _e4m3_codes(g, (1, 28))
    codes[0, 3] = 0x7E
    rope = numfmt.bf16_round_f64(g.standard_normal(4))
    y = np.concatenate([numfmt.e4m3_decode(codes[0]) * 0.25, rope])
    c, sc, rp, row = oracle.mixed_kv_row(y, 4, np.ones(2), np.zeros(2))
    np.testing.assert_array_equal(c, codes[0])
    assert sc == np.float32(0.25)
    np.testing.assert_array_equal(row, y)
    y = g.standard_normal(32)
    _, sc, _, row = oracle.mixed_kv_row(y, 8)
    yf = y.astype(np.float32).astype(np.float64)
    bound = np.maximum(np.abs(yf[:24]) * 2.0 ** -4, sc * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(row[:24] - yf[:24]) <= bound).all()
    assert (np.abs(row[24:] - yf[24:]) <= np.abs(yf[24:]) * 2.0 ** -8).all()


def test_decode_step_mixed_kv_equals_plain_step_when_exact():
    """Mixed storage loses nothing when every stored value is representable
    (E4M3 NoPE times a power of two, bfloat16 RoPE) and every rotation is the
    identity: the mixed step then matches the float64 step — scores,
    selection and output (ratio 1: each compressed entry is its content row)."""
    g = _g(30)
    D, di, H, W, rd = 16, 8, 4, 6, 4
    Lp = _empty_state(g, D=D, di=di, H=H, W=W, m=1)
    Lm = _empty_state(g, D=D, di=di, H=H, W=W, m=1)
    Lm.main_bias, Lm.idx_bias, Lm.sink = Lp.main_bias, Lp.idx_bias, Lp.sink
    Lm.kv_mixed, Lm.rope_dim = True, rd
    one, zero = np.ones((64, rd // 2)), np.zeros((64, rd // 2))
    Lm.rope_cos, Lm.rope_sin, Lm.comp_rope_cos, Lm.comp_rope_sin = one, zero, one, zero

    def exact_row():
        c = _e4m3_codes(g, (1, D - rd))
        c[0, 0] = 0x7E
        return np.concatenate([numfmt.e4m3_decode(c[0]) * 0.5, numfmt.bf16_round_f64(g.standard_normal(rd))])

    for pos in range(12):
        inp = _step_inputs(g, D=D, di=di, H=H, m=1)
        inp["kv_new"] = exact_row()
        inp["c_main"] = exact_row()[None]
        rp = oracle.decode_step(Lp, pos=pos, top_k=4, **inp)
        rm = oracle.decode_step(Lm, pos=pos, top_k=4, **inp)
        np.testing.assert_array_equal(Lm.comp_kv[:Lm.n_comp], Lp.comp_kv[:Lp.n_comp])
        np.testing.assert_array_equal(Lm.swa.rows, Lp.swa.rows)
        np.testing.assert_array_equal(rm["idx"], rp["idx"])
        np.testing.assert_allclose(rm["out"], rp["out"], rtol=1e-13, atol=1e-14)


def test_decode_step_mixed_kv_rotations():
    """Each compressed entry's RoPE part is rotated at its block index with
    the comp tables, and the output gets the inverse rotation at the token's
    position: with a sink-free first block attended alone, the output is the
    entry itself rotated back."""
    g = _g(31)
    D, H, W, rd = 16, 4, 1, 4
    L = _empty_state(g, D=D, H=H, W=W, m=2)
    L.sink = None
    L.kv_mixed, L.rope_dim = True, rd
    L.rope_cos, L.rope_sin = _rope_tables(16, rd)
    L.comp_rope_cos, L.comp_rope_sin = _rope_tables(8, rd, base=7.0, offset=0.5)
    for pos in range(4):
        inp = _step_inputs(g, D=D, H=H, m=2)
        r = oracle.decode_step(L, pos=pos, top_k=4, **inp)
    # position 3 completed block 1 (positions 2, 3)
    ym = oracle.compress(inp["z_main"], inp["c_main"], L.main_bias, 2)[0]
    _, _, _, want = oracle.mixed_kv_row(ym, rd, L.comp_rope_cos[1], L.comp_rope_sin[1])
    np.testing.assert_array_equal(L.comp_kv[1], want)
    rows = r["rows"]
    o, _ = oracle.sparse_attn(inp["q"], rows, None)
    np.testing.assert_allclose(r["out"], oracle.rope_rotate(o, L.rope_cos[3], L.rope_sin[3], inverse=True),
                               rtol=1e-13, atol=1e-14)
    # the RoPE part of the stored entry is not the unrotated one
    assert not np.allclose(L.comp_kv[1][-rd:], numfmt.bf16_round_f64(ym[-rd:].astype(np.float32)))


# ---------------------------------------------------------------------------
# (6b) HCA step: the dense special case of the CSA step
# ---------------------------------------------------------------------------

def test_hca_step_equals_csa_step_with_top_k_covering_all():
    """An HCA step attends to every compressed entry and the window; a CSA
    step whose top-k covers every entry selects the same rows in another
    order, and attention does not depend on the order — so both give the same
    output for any indexer keys (ratio 8, four block completions, ring wrap)."""
    g = _g(24)
    m, W, D, H = 8, 6, 16, 4
    Lh = _empty_state(g, D=D, W=W, H=H, m=m)
    Lc = _empty_state(g, D=D, W=W, H=H, m=m)
    Lc.main_bias, Lc.sink = Lh.main_bias, Lh.sink
    for pos in range(37):
        inp = _step_inputs(g, D=D, H=H, m=m)
        rh = oracle.hca_decode_step(Lh, q=inp["q"], kv_new=inp["kv_new"], pos=pos,
                                    z_main=inp["z_main"], c_main=inp["c_main"])
        rc = oracle.decode_step(Lc, pos=pos, top_k=64, **inp)
        assert Lh.n_comp == Lc.n_comp == (pos + 1) // m
        assert rh["n_valid"] == rc["n_valid"] == Lh.n_comp + min(pos + 1, W)
        np.testing.assert_allclose(rh["out"], rc["out"], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(rh["lse"], rc["lse"], rtol=1e-13)


def test_hca_step_mixed_kv_equals_csa_step_mixed_kv_with_top_k_covering_all():
    """With mixed main KV too, an HCA step equals a CSA step whose top-k
    covers every entry: the same stored rows, rotations and output."""
    g = _g(32)
    m, W, D, H, rd = 8, 6, 16, 4, 4
    Lh = _empty_state(g, D=D, W=W, H=H, m=m)
    Lc = _empty_state(g, D=D, W=W, H=H, m=m)
    Lc.main_bias, Lc.sink = Lh.main_bias, Lh.sink
    cos, sin = _rope_tables(64, rd)
    ccos, csin = _rope_tables(16, rd, base=9.0, offset=0.5)
    for L in (Lh, Lc):
        L.kv_mixed, L.rope_dim = True, rd
        L.rope_cos, L.rope_sin, L.comp_rope_cos, L.comp_rope_sin = cos, sin, ccos, csin
    for pos in range(27):
        inp = _step_inputs(g, D=D, H=H, m=m)
        rh = oracle.hca_decode_step(Lh, q=inp["q"], kv_new=inp["kv_new"], pos=pos,
                                    z_main=inp["z_main"], c_main=inp["c_main"])
        rc = oracle.decode_step(Lc, pos=pos, top_k=64, **inp)
        np.testing.assert_array_equal(Lh.comp_kv[:Lh.n_comp], Lc.comp_kv[:Lc.n_comp])
        np.testing.assert_allclose(rh["out"], rc["out"], rtol=1e-12, atol=1e-13)


def test_hca_step_rows_are_cache_then_window():
    g = _g(25)
    L = _empty_state(g, W=4, m=2)
    L.sink = None
    for pos in range(7):
        inp = _step_inputs(g, m=2)
        r = oracle.hca_decode_step(L, q=inp["q"], kv_new=inp["kv_new"], pos=pos, z_main=inp["z_main"],
                                   c_main=inp["c_main"])
    # three entries (positions 1, 3, 5 complete blocks 0..2; position 6 does not), then window 3..6
    assert L.n_comp == 3 and r["n_valid"] == 3 + 4
    np.testing.assert_array_equal(r["rows"][:3], L.comp_kv[:3])
    np.testing.assert_array_equal(r["rows"][3], L.swa.rows[(L.swa.head - 4) % 4])


# ---------------------------------------------------------------------------
# (7) prefill chunk: the same as one decode step per token
# ---------------------------------------------------------------------------

def _prefill_vs_decode_steps(pos0, T, top_k, W=8, seed=23, prefill=oracle.prefill_chunk):
    """Run decode steps for positions 0 .. pos0+T-1 and the prefill chunk for
    the last T of them on the final caches; both must agree token by token."""
    g = _g(seed)
    L = _empty_state(g, W=W)
    per_token = []
    kv_rows = []
    for pos in range(pos0 + T):
        inp = _step_inputs(g)
        kv_rows.append(inp["kv_new"])
        r = oracle.decode_step(L, pos=pos, top_k=top_k, **inp)
        if pos >= pos0:
            per_token.append((inp, r))
    first = pos0 - W + 1
    win = np.stack([kv_rows[x] if x >= 0 else np.full(16, np.nan) for x in range(first, pos0 + T)])
    N = L.n_comp
    got = prefill(q=np.stack([i["q"] for i, _ in per_token]), q_idx=np.stack([i["q_idx"] for i, _ in per_token]),
                  w_idx=np.stack([i["w_idx"] for i, _ in per_token]), idx_keys=L.idx_keys[:N],
                  comp_kv=L.comp_kv[:N], win_kv=win, pos0=pos0, top_k=top_k, window=W, sink=L.sink)
    for t, (_, r) in enumerate(per_token):
        assert got["count"][t] == r["count"]
        assert got["idx"][t].tolist() == r["idx"].tolist()
        np.testing.assert_allclose(got["out"][t], r["out"], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(got["lse"][t], r["lse"], rtol=1e-13)


@pytest.mark.parametrize("pos0,T,top_k", [(21, 9, 3), (2, 10, 2), (13, 6, 64), (0, 5, 1)])
def test_prefill_chunk_equals_decode_steps(pos0, T, top_k):
    """Each query of the chunk gets exactly what a decode step at its position
    gets: causal mask = blocks complete by then, window = the last W tokens
    (clipped at position 0), top_k >= n_comp = dense attention."""
    _prefill_vs_decode_steps(pos0, T, top_k)


def test_mutation_prefill_pins_catch_planted_mistakes():
    def window_one_late(**kw):  # window rows shifted by one position
        kw = dict(kw)
        kw["win_kv"] = np.concatenate([kw["win_kv"][1:], kw["win_kv"][-1:]])
        return oracle.prefill_chunk(**kw)

    def positions_one_early(**kw):  # every query one position early (mask and window)
        return oracle.prefill_chunk(**dict(kw, pos0=kw["pos0"] - 1))

    for bad in (window_one_late, positions_one_early):
        with pytest.raises(AssertionError):
            _prefill_vs_decode_steps(21, 9, 3, prefill=bad)


# ---------------------------------------------------------------------------
# workload shapes against the pages' printed sizes
# ---------------------------------------------------------------------------

def test_workload_shapes_match_printed_sizes():
    import synth
    ps = _load("page_sizes.json")
    s = synth.SHAPES["ctx1m"]
    assert s.d_i == ps["indexer_key_width"] and s.h_i == ps["indexer_heads"]
    assert s.d_i * 2 == ps["indexer_bytes_per_block"]
    assert s.ctx // s.m == ps["blocks_at_1m"] == s.n_comp
    assert s.n_comp * s.d_i * 2 == ps["indexer_bytes_per_layer_at_1m"]
    assert s.n_comp * s.d * 2 == ps["main_bytes_per_layer_at_1m"]
    assert s.w * s.d * 2 == ps["swa_bytes_per_layer"] and s.w == ps["swa_window"]
    assert s.top_k + s.w == ps["gather_buf_rows"]
    assert 2 * s.d_i == ps["indexer_compressor_kv_dim"] and 2 * s.d == ps["main_compressor_kv_dim"]
    assert [s.m, 2 * s.d_i] == ps["indexer_position_bias_shape"]


def test_synth_inputs_deterministic_and_shaped():
    import synth
    sh = synth.SHAPES["tiny"]
    a = synth.make_decode_inputs(sh, 1001)
    b = synth.make_decode_inputs(sh, 1001)
    for k in a:
        np.testing.assert_array_equal(np.asarray(a[k]), np.asarray(b[k]))
    assert a["idx_keys"].shape == (1, 256, 128) and a["comp_kv"].shape == (1, 256, 128)
    assert a["n_comp"] == 255 and a["swa_head"] == 1023 % 128 and a["swa_len"] == 128
    sh2 = synth.SHAPES["ctx8k"]
    c = synth.make_decode_inputs(synth.with_(sh2, n_comp=64, ctx=256), 5)
    assert c["comp_kv"].dtype == np.uint16 and c["q"].shape == (1, 64, 512)


# ---------------------------------------------------------------------------
# FP8 E4M3 codec, row quantiser and the FP8 index score
# ---------------------------------------------------------------------------

def test_e4m3_decode_closed_forms():
    """Spot values fixed by the format's definition (bias 7, 3 mantissa bits,
    exponent field 0 = subnormals m/8 * 2^-6, S.1111.111 = NaN, no inf)."""
    d = lambda c: float(numfmt.e4m3_decode(np.array([c], dtype=np.uint8))[0])  # noqa: E731
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    assert d(0x01) == 2.0 ** -9 and d(0x07) == 7 * 2.0 ** -9
    assert d(0x08) == 2.0 ** -6                      # smallest normal
    assert d(0x38) == 1.0 and d(0x39) == 1.125 and d(0x3F) == 1.875 and d(0x40) == 2.0
    assert d(0x7E) == 448.0 and d(0xFE) == -448.0    # largest finite
    assert d(0xB8) == -1.0
    assert math.isnan(d(0x7F)) and math.isnan(d(0xFF))
    vals = numfmt.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert np.isnan(vals).sum() == 2 and np.isinf(vals).sum() == 0
    # the non-negative codes are monotone in value
    assert np.all(np.diff(vals[:0x7F]) > 0)


def test_e4m3_encode_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = numfmt.e4m3_decode(codes)
    np.testing.assert_array_equal(numfmt.e4m3_encode(vals), codes)


def test_e4m3_encode_ties_to_even_and_saturation():
    enc = lambda x: int(numfmt.e4m3_encode(np.array([x]))[0])  # noqa: E731
    assert enc(1.0625) == 0x38       # midway 1 and 1.125: even mantissa
    assert enc(1.1875) == 0x3A       # midway 1.125 and 1.25: even mantissa
    assert enc(1.9375) == 0x40       # midway 1.875 and 2: carries into the exponent
    assert enc(2.0 ** -10) == 0x00   # midway 0 and the smallest subnormal
    assert enc(3 * 2.0 ** -10) == 0x02
    assert enc(1.07) == 0x39 and enc(1.05) == 0x38
    assert enc(449.0) == 0x7E and enc(1e9) == 0x7E and enc(-1e9) == 0xFE
    assert enc(-0.0) == 0x80 and enc(0.0) == 0x00


def test_e4m3_encode_is_nearest_by_brute_force():
    rng = np.random.default_rng(11)
    x = np.concatenate([rng.standard_normal(2000) * 50, rng.standard_normal(500) * 2.0 ** -7,
                        rng.uniform(-448, 448, 500)])
    got = numfmt.e4m3_decode(numfmt.e4m3_encode(x))
    grid = numfmt.e4m3_decode(np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8))
    best = np.abs(x[:, None] - grid[None, :]).min(axis=1)
    np.testing.assert_array_equal(np.abs(x - got), best)
    assert np.all(np.sign(got[got != 0]) == np.sign(x[got != 0]))


def test_quantize_e4m3_rows():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((40, 128)).astype(np.float32)
    x[3] = 0.0
    x[5, 17] = -9.5            # a negative row maximum
    codes, scale = numfmt.quantize_e4m3_rows(x)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    assert scale[3] == 1.0 and not codes[3].any()
    for r in (0, 5, 39):
        j = int(np.argmax(np.abs(x[r])))
        assert codes[r, j] in (0x7E, 0xFE)                          # the row maximum maps to +-448
        assert scale[r] == np.float32(np.abs(x[r]).max()) / np.float32(448.0)
    deq = numfmt.e4m3_decode(codes) * scale[:, None].astype(np.float64)
    # relative error of a normal e4m3 value is at most 2^-4 (half of 2^-3)
    big = np.abs(x) > 2.0 ** -6 * scale[:, None]
    assert np.all(np.abs(deq - x)[big] <= np.abs(x)[big] * 2.0 ** -4 + 1e-12)


def test_index_score_fp8_integer_brute_force():
    """Codes of small integers and k_scale values that are powers of two give
    exactly known scores, summed by hand in integers."""
    enc = {0: 0x00, 1: 0x38, 2: 0x40, -1: 0xB8, -2: 0xC0, 3: 0x44}
    rng = np.random.default_rng(13)
    H, D, N = 4, 8, 6
    qi = rng.choice([0, 1, 2, -1, -2, 3], size=(1, H, D))
    ki = rng.choice([0, 1, 2, -1, -2, 3], size=(N, D))
    q = np.vectorize(enc.get)(qi).astype(np.uint8)
    k = np.vectorize(enc.get)(ki).astype(np.uint8)
    ks = np.array([1.0, 2.0, 0.5, 4.0, 0.25, 1.0])
    w = np.array([[1.0, -2.0, 0.5, 3.0]])
    got = oracle.index_score_fp8(q, w, k, ks)
    for s in range(N):
        ref = 0.0
        for h in range(H):
            dot = sum(int(qi[0, h, d]) * int(ki[s, d]) for d in range(D))
            ref += w[0, h] * max(0.0, ks[s] * dot)
        assert got[0, s] == ref
    # the causal form hides blocks past the position
    masked = oracle.index_score_fp8(q, w, k, ks, q_pos=[9], ratio=4)
    assert np.isneginf(masked[0, 3:]).all() and np.array_equal(masked[0, :2], got[0, :2])
