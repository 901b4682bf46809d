"""GPU parity of the mixed main-KV path (E4M3 NoPE codes + bfloat16 RoPE
part per row, RoPE on compressed entries, inverse RoPE on the output)
against the float64 CPU oracle.

* csa_pack_kv_mixed: records bit-exact against the oracle's mixed rows;
* csa_decode_step with kv_dtype = CSA_FP8_E4M3: the appended ring record
  bit-exact, the compressed entry within E4M3 / one bfloat16 ulp of the
  oracle's (then adopted), top-k as for bf16 caches, gather_buf records
  bit-exact, output within 2e-2 relative (the attention decodes the records
  to bfloat16: 2^-9 relative per value on top of the bf16 path's rounding),
  lse within 1e-2.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import numfmt
from tests.gpu_util import (assert_lse_close, DEV, as_f64, assert_topk_gap_rule, dev_bf16, dev_f32, host_f64, rel_err)

pytestmark = pytest.mark.gpu

REC, NOPE, ROPE = 592, 448, 64


@pytest.fixture(scope="module")
def csa():
    import compressed_sparse_attention_reduce_amd as pkg
    pkg.lib()
    return pkg


def _g(seed):
    return np.random.Generator(np.random.PCG64(seed))


def rope_tables(rows, offset=0.5, base=10000.0):
    """float32 cos / sin [rows, 32] of the angles (p + offset) * base^(-2j/64)."""
    ang = (np.arange(rows)[:, None] + offset) * base ** (-2.0 * np.arange(ROPE // 2)[None, :] / ROPE)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def record_of(codes, scale, rope):
    """The 592 bytes of one record from the oracle's (codes, scale, rope values)."""
    r = np.zeros(REC, dtype=np.uint8)
    r[:NOPE] = codes
    r[NOPE:NOPE + 2 * ROPE] = numfmt.f64_to_bf16_bits(rope).view(np.uint8)
    r[576:580] = np.array([scale], dtype=np.float32).view(np.uint8)
    return r


def decode_records(rec):
    """float64 rows [..., 512] that records [..., 592] hold."""
    rec = np.ascontiguousarray(rec)
    codes = rec[..., :NOPE]
    scale = rec[..., 576:580].copy().view(np.float32)[..., 0].astype(np.float64)
    rope = numfmt.bf16_bits_to_f64(rec[..., NOPE:NOPE + 2 * ROPE].copy().view(np.uint16))
    return np.concatenate([numfmt.e4m3_decode(codes) * scale[..., None], rope], axis=-1)


def oracle_records(rows):
    """Records and their values for float rows [n, 512] (no rotation)."""
    recs, vals = [], []
    for y in rows:
        c, s, rp, v = oracle.mixed_kv_row(y, ROPE)
        recs.append(record_of(c, s, rp))
        vals.append(v)
    return np.stack(recs), np.stack(vals)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_pack_kv_mixed_bit_exact(csa, dt):
    g = _g(71 if dt == "bf16" else 72)
    x = g.standard_normal((300, 512), dtype=np.float32) * np.float32(3.0)
    x[5] = 0.0                     # all-zero row: scale 1
    x[6, :NOPE] = 0.0              # zero NoPE part
    x[7, 17] = 1e-30               # a subnormal E4M3 code after scaling
    if dt == "bf16":
        xb = synth.to_bf16_bits(x)
        xd, xs = dev_bf16(xb), numfmt.bf16_bits_to_f64(xb)
    else:
        xd, xs = dev_f32(x), x.astype(np.float64)
    rec = torch.full((300, REC), 0xAB, dtype=torch.uint8, device=DEV)
    csa.csa_pack_kv_mixed(xd, rec)
    torch.cuda.synchronize()
    want, _ = oracle_records(xs)
    np.testing.assert_array_equal(rec.cpu().numpy(), want)


def _mixed_layer(csa, x, shape, g, max_comp, rope_rows, comp_rows):
    """Device layer with mixed caches built from the oracle's records of the
    synthetic bf16 rows; the oracle state holds the same values."""
    f = numfmt.bf16_bits_to_f64
    comp_rec, comp_val = oracle_records(f(x["comp_kv"][0]))
    swa_rec, swa_val = oracle_records(f(x["swa"][0]))
    comp = torch.from_numpy(comp_rec[None].copy()).to(DEV)
    swa = torch.from_numpy(swa_rec[None].copy()).to(DEV)
    rc, rs = rope_tables(rope_rows)
    cc, cs = rope_tables(comp_rows, offset=0.25, base=500.0)
    rope = (dev_f32(rc), dev_f32(rs))
    comp_rope = (dev_f32(cc), dev_f32(cs))
    keys = dev_bf16(x["idx_keys"])
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=keys, swa=swa, main_bias=dev_f32(x["main_bias"]),
                            idx_bias=dev_f32(x["idx_bias"]), sink=dev_f32(x["sink"]), n_comp=x["n_comp"],
                            swa_head=x["swa_head"], swa_len=x["swa_len"], h=shape.h, h_i=shape.h_i,
                            top_k=shape.top_k, rope=rope, comp_rope=comp_rope)
    assert L.kv_dtype == csa.CSA_FP8_E4M3 and L.d == 512
    ost = oracle.LayerState(comp_kv=comp_val, idx_keys=f(x["idx_keys"][0]), n_comp=x["n_comp"],
                            swa=oracle.SwaRing(swa_val, x["swa_head"], x["swa_len"]),
                            main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"],
                            round_cache=numfmt.bf16_round_f64, kv_mixed=True, rope_dim=ROPE,
                            rope_cos=rc.astype(np.float64), rope_sin=rs.astype(np.float64),
                            comp_rope_cos=cc.astype(np.float64), comp_rope_sin=cs.astype(np.float64))
    return L, ost, comp, swa, keys


def _assert_entry_close(got_rec, want_vals):
    """A GPU-packed compressed entry against the oracle's values: NoPE within
    half an E4M3 unit (plus float32 slack), RoPE within one bfloat16 ulp."""
    got = decode_records(got_rec)
    scale = float(got_rec[576:580].copy().view(np.float32)[0])
    nope_w = want_vals[:NOPE]
    assert scale == pytest.approx(np.abs(nope_w).max() / 448, rel=1e-5)
    bound = np.maximum(np.abs(nope_w) * 2.0 ** -4, scale * 2.0 ** -10) + 1e-5 * np.abs(nope_w).max()
    assert (np.abs(got[:NOPE] - nope_w) <= bound).all()
    assert (np.abs(got[NOPE:] - want_vals[NOPE:]) <= np.abs(want_vals[NOPE:]) * 2.0 ** -7 + 1e-30).all()


def test_decode_steps_in_sequence_mixed_kv(csa):
    """Nine consecutive steps over mixed caches (two block completions, ring
    wrap), each against the oracle's evolving state."""
    shape = synth.with_(synth.SHAPES["ctx8k"], ctx=600, n_comp=150, top_k=64, w=8)
    x = synth.make_decode_inputs(shape, 7101, max_comp=200)
    g = _g(7102)
    L, ost, comp, swa, keys = _mixed_layer(csa, x, shape, g, 200, 1000, 300)
    f = numfmt.bf16_bits_to_f64
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    for pos in range(x["pos"], x["pos"] + 9):
        q = synth.to_bf16_bits(g.standard_normal((1, 64, 512), dtype=np.float32))
        qi = synth.to_bf16_bits(g.standard_normal((1, 64, 128), dtype=np.float32) / np.float32(np.sqrt(128)))
        wi = g.standard_normal((1, 64), dtype=np.float32)
        kvn = synth.to_bf16_bits(g.standard_normal((1, 512), dtype=np.float32))
        zm, cm = g.standard_normal((2, 1, 4, 512), dtype=np.float32)
        zi, ci = g.standard_normal((2, 1, 4, 128), dtype=np.float32)
        outs = dict(scores=torch.empty(1, 200, device=DEV), topk_idx=torch.empty(1, 64, dtype=torch.int32, device=DEV),
                    topk_count=torch.empty(1, dtype=torch.int32, device=DEV),
                    gather_buf=torch.zeros(1, 72, REC, dtype=torch.uint8, device=DEV),
                    n_valid=torch.empty(1, dtype=torch.int32, device=DEV),
                    out=torch.empty(1, 64, 512, dtype=torch.bfloat16, device=DEV),
                    lse=torch.empty(1, 64, device=DEV))
        io = csa.make_step_io(pos=pos, q=dev_bf16(q), q_idx=dev_bf16(qi), w_idx=dev_f32(wi), kv_new=dev_bf16(kvn),
                              z_main=dev_f32(zm), c_main=dev_f32(cm), z_idx=dev_f32(zi), c_idx=dev_f32(ci), **outs)
        print(f"mixed-KV step pos={pos}", flush=True)
        slot = L.swa_head
        csa.csa_decode_step(L, io, ws)
        csa.csa_layer_advance(L, pos)
        torch.cuda.synchronize()
        completes = pos % 4 == 3
        n0 = ost.n_comp
        oracle.decode_step(ost, q=f(q[0]), q_idx=f(qi[0]), w_idx=wi[0], kv_new=f(kvn[0]), pos=pos, top_k=64,
                           z_main=zm[0], c_main=cm[0], z_idx=zi[0], c_idx=ci[0], scale=1 / np.sqrt(512))
        assert (L.n_comp, L.swa_head, L.swa_len) == (ost.n_comp, ost.swa.head, ost.swa.length)
        N = ost.n_comp
        # a. the ring record of the new token: bit-exact
        c_, s_, rp_, _ = oracle.mixed_kv_row(f(kvn[0]), ROPE)
        np.testing.assert_array_equal(swa[0, slot].cpu().numpy(), record_of(c_, s_, rp_))
        # b. the compressed entry and its indexer key, then adopt the GPU's
        if completes:
            ym = oracle.compress(zm[0], cm[0], x["main_bias"], 4)[0]
            blk = pos // 4
            _, _, _, want = oracle.mixed_kv_row(ym, ROPE, ost.comp_rope_cos[blk], ost.comp_rope_sin[blk])
            _assert_entry_close(comp[0, n0].cpu().numpy(), want)
        ost.comp_kv[:N] = decode_records(comp[0, :N].cpu().numpy())
        ost.idx_keys[:N] = host_f64(keys[0, :N])
        # c, d. scores and top-k (bf16 indexer keys)
        ref_s = oracle.index_score(f(qi[0])[None], wi[0][None], ost.idx_keys[:N])[0]
        got_s = outs["scores"][0, :N].cpu().numpy().astype(np.float64)
        assert rel_err(got_s, ref_s) <= 1e-4
        gi, gc = outs["topk_idx"][0].cpu().numpy(), int(outs["topk_count"][0])
        np.testing.assert_array_equal(gi, oracle.topk(got_s[None], 64)[0][0])
        assert_topk_gap_rule(gi, gc, ref_s, 64)
        # e. gather_buf: the selected records then the window's, bit-exact
        recs = comp[0].cpu().numpy()
        ring = swa[0].cpu().numpy()
        want_buf = [recs[i] for i in gi[:gc]] + [ring[(ost.swa.head - ost.swa.length + j) % 8]
                                                 for j in range(ost.swa.length)]
        nv = int(outs["n_valid"][0])
        assert nv == len(want_buf)
        np.testing.assert_array_equal(outs["gather_buf"][0, :nv].cpu().numpy(), np.stack(want_buf))
        # f. attention over the decoded rows, then the inverse rotation
        rows = decode_records(np.stack(want_buf))
        ro, rl = oracle.sparse_attn(f(q[0]), rows, x["sink"], 1 / np.sqrt(512))
        ro = oracle.rope_rotate(ro, ost.rope_cos[pos], ost.rope_sin[pos], inverse=True)
        assert rel_err(host_f64(outs["out"][0]), ro) <= 2e-2
        assert_lse_close(outs["lse"][0].cpu().numpy(), rl)


def test_mixed_step_decodes_every_code(csa):
    """The first token of a layer with nothing before it: the attention sees
    one row (the token's own record), so with no sink and identity tables
    every head's output is that row exactly.  Its NoPE part holds every
    finite E4M3 code times 1/8 (with +-448/8 setting the scale to 1/8), so
    the attention's decoding of every code is checked bit for bit."""
    g = _g(7301)
    finite = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    codes = np.resize(finite, NOPE)
    codes[0] = 0x7E
    vals = np.concatenate([numfmt.e4m3_decode(codes) * 0.125,
                           numfmt.bf16_round_f64(g.standard_normal(ROPE))])
    kvn = numfmt.f64_to_bf16_bits(vals)[None]
    assert np.array_equal(numfmt.bf16_bits_to_f64(kvn[0]), vals)
    H, K, W, max_comp = 16, 8, 4, 8
    comp = torch.zeros(1, max_comp, REC, dtype=torch.uint8, device=DEV)
    swa = torch.zeros(1, W, REC, dtype=torch.uint8, device=DEV)
    keys = torch.zeros(1, max_comp, 128, dtype=torch.bfloat16, device=DEV)
    ones, zeros = torch.ones(4, 32, device=DEV), torch.zeros(4, 32, device=DEV)
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=keys, swa=swa, main_bias=torch.zeros(4, 512, device=DEV),
                            idx_bias=torch.zeros(4, 128, device=DEV), sink=None, n_comp=0, swa_head=0, swa_len=0,
                            h=H, h_i=64, top_k=K, rope=(ones, zeros), comp_rope=(ones, zeros))
    q = dev_bf16(synth.to_bf16_bits(g.standard_normal((1, H, 512), dtype=np.float32)))
    qi = dev_bf16(synth.to_bf16_bits(g.standard_normal((1, 64, 128), dtype=np.float32)))
    out = torch.empty(1, H, 512, dtype=torch.bfloat16, device=DEV)
    io = csa.make_step_io(pos=0, q=q, q_idx=qi, w_idx=torch.ones(1, 64, device=DEV), kv_new=dev_bf16(kvn),
                          z_main=torch.zeros(1, 4, 512, device=DEV), c_main=torch.zeros(1, 4, 512, device=DEV),
                          z_idx=torch.zeros(1, 4, 128, device=DEV), c_idx=torch.zeros(1, 4, 128, device=DEV),
                          scores=torch.empty(1, max_comp, device=DEV),
                          topk_idx=torch.empty(1, K, dtype=torch.int32, device=DEV),
                          topk_count=torch.empty(1, dtype=torch.int32, device=DEV),
                          gather_buf=torch.zeros(1, K + W, REC, dtype=torch.uint8, device=DEV),
                          n_valid=torch.empty(1, dtype=torch.int32, device=DEV), out=out)
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    csa.csa_decode_step(L, io, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(swa[0, 0, :NOPE].cpu().numpy(), codes)
    got = host_f64(out[0])
    for h in range(H):
        np.testing.assert_array_equal(got[h], vals)


def test_decode_step_ctx1m_mixed_kv_full_size(csa):
    """One layer of the 1M-context workload over mixed caches packed on the
    GPU (csa_pack_kv_mixed, bit-exact above) from the bf16 caches: gather_buf
    records bit-exact, output against the oracle's attention over the
    decoded rows with the inverse rotation."""
    shape = synth.SHAPES["ctx1m"]
    x = synth.make_decode_inputs_torch(shape, seed=None, device=DEV, layers=1)[0]
    B, K, W = shape.batch, shape.top_k, shape.w
    comp = torch.empty(B, shape.max_comp, REC, dtype=torch.uint8, device=DEV)
    swa = torch.empty(B, W, REC, dtype=torch.uint8, device=DEV)
    csa.csa_pack_kv_mixed(x["comp_kv"], comp)
    csa.csa_pack_kv_mixed(x["swa"], swa)
    rc, rs = rope_tables(shape.ctx + 8)
    cc, cs = rope_tables(shape.max_comp + 1, offset=0.25, base=500.0)
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=x["idx_keys"], swa=swa, main_bias=x["main_bias"],
                            idx_bias=x["idx_bias"], sink=x["sink"], n_comp=x["n_comp"], swa_head=x["swa_head"],
                            swa_len=x["swa_len"], h=shape.h, h_i=shape.h_i, top_k=K,
                            rope=(dev_f32(rc), dev_f32(rs)), comp_rope=(dev_f32(cc), dev_f32(cs)))
    outs = dict(scores=torch.empty(B, shape.max_comp, device=DEV),
                topk_idx=torch.empty(B, K, dtype=torch.int32, device=DEV),
                topk_count=torch.empty(B, dtype=torch.int32, device=DEV),
                gather_buf=torch.zeros(B, K + W, REC, dtype=torch.uint8, device=DEV),
                n_valid=torch.empty(B, dtype=torch.int32, device=DEV),
                out=torch.empty(B, shape.h, 512, dtype=torch.bfloat16, device=DEV),
                lse=torch.empty(B, shape.h, device=DEV))
    io = csa.make_step_io(pos=x["pos"], q=x["q"], q_idx=x["q_idx"], w_idx=x["w_idx"], kv_new=x["kv_new"],
                          z_main=x["z_main"], c_main=x["c_main"], z_idx=x["z_idx"], c_idx=x["c_idx"], **outs)
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    csa.csa_decode_step(L, io, ws)
    torch.cuda.synchronize()
    N = shape.n_comp
    pos = x["pos"]
    ym = oracle.compress(host_f64(x["z_main"][0]), host_f64(x["c_main"][0]), host_f64(x["main_bias"]), 4)[-1]
    _, _, _, want = oracle.mixed_kv_row(ym, ROPE, cc[pos // 4].astype(np.float64), cs[pos // 4].astype(np.float64))
    _assert_entry_close(comp[0, N - 1].cpu().numpy(), want)
    gi = outs["topk_idx"][0].cpu().numpy()
    gc = int(outs["topk_count"][0])
    assert gc == K
    sel = comp[0, torch.from_numpy(gi).to(DEV).long()].cpu().numpy()
    ring = swa[0].cpu().numpy()
    head = (x["swa_head"] + 1) % W
    win = np.stack([ring[(head - W + j) % W] for j in range(W)])
    want_buf = np.concatenate([sel, win])
    assert int(outs["n_valid"][0]) == K + W
    np.testing.assert_array_equal(outs["gather_buf"][0].cpu().numpy(), want_buf)
    rows = decode_records(want_buf)
    ro, rl = oracle.sparse_attn(host_f64(x["q"][0]), rows, host_f64(x["sink"]), 1.0 / np.sqrt(512))
    ro = oracle.rope_rotate(ro, rc[pos].astype(np.float64), rs[pos].astype(np.float64), inverse=True)
    assert rel_err(host_f64(outs["out"][0]), ro) <= 2e-2
    assert_lse_close(outs["lse"][0].cpu().numpy(), rl)


@pytest.mark.parametrize("B", [3, 5, 8])
def test_decode_step_mixed_kv_fp8_keys_batched(csa, B):
    """Several sequences, E4M3 indexer keys and mixed main KV together, a step
    that completes a block: each sequence's new records, scores, selection,
    gather_buf and output against the oracle.  Three sequences take the fused
    top-k + attention (240 workgroups, all resident on 256 compute units);
    five and eight take one top-k launch per sequence and the separate
    attention (eight: 640 attention workgroups)."""
    shape = synth.with_(synth.SHAPES["ctx8k"], batch=B, ctx=4000, n_comp=999)
    x = synth.make_decode_inputs(shape, 7401, max_comp=1000)
    g = _g(7402)
    f = numfmt.bf16_bits_to_f64
    pos = x["pos"]
    assert pos % 4 == 3
    comp_recs, comp_vals, swa_recs, swa_vals = [], [], [], []
    for b in range(B):
        r, v = oracle_records(f(x["comp_kv"][b]))
        comp_recs.append(r); comp_vals.append(v)
        r, v = oracle_records(f(x["swa"][b]))
        swa_recs.append(r); swa_vals.append(v)
    comp = torch.from_numpy(np.stack(comp_recs)).to(DEV)
    swa = torch.from_numpy(np.stack(swa_recs)).to(DEV)
    kc0, ks0 = numfmt.quantize_e4m3_rows(f(x["idx_keys"].reshape(-1, 128)).astype(np.float32))
    kc0, ks0 = kc0.reshape(B, 1000, 128), ks0.reshape(B, 1000)
    kc, ks = torch.from_numpy(kc0.copy()).to(DEV), dev_f32(ks0)
    # the step takes the bf16 query and quantises it; the oracle's codes and folded weights from the host
    qi = synth.to_bf16_bits(g.standard_normal((B, 64, 128), dtype=np.float32) / np.float32(np.sqrt(128)))
    qc, qs = numfmt.quantize_e4m3_rows(f(qi).reshape(-1, 128).astype(np.float32))
    qc = qc.reshape(B, 64, 128)
    w8 = (x["w_idx"] * qs.reshape(B, 64)).astype(np.float32)
    rc, rs = rope_tables(pos + 4)
    cc, cs = rope_tables(1001, offset=0.25, base=500.0)
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=kc, idx_scales=ks, swa=swa, main_bias=dev_f32(x["main_bias"]),
                            idx_bias=dev_f32(x["idx_bias"]), sink=dev_f32(x["sink"]), n_comp=x["n_comp"],
                            swa_head=x["swa_head"], swa_len=x["swa_len"], h=64, h_i=64, top_k=shape.top_k,
                            rope=(dev_f32(rc), dev_f32(rs)), comp_rope=(dev_f32(cc), dev_f32(cs)))
    K, W = shape.top_k, shape.w
    outs = dict(scores=torch.empty(B, 1000, device=DEV), topk_idx=torch.empty(B, K, dtype=torch.int32, device=DEV),
                topk_count=torch.empty(B, dtype=torch.int32, device=DEV),
                gather_buf=torch.zeros(B, K + W, REC, dtype=torch.uint8, device=DEV),
                n_valid=torch.empty(B, dtype=torch.int32, device=DEV),
                out=torch.empty(B, 64, 512, dtype=torch.bfloat16, device=DEV), lse=torch.empty(B, 64, device=DEV))
    io = csa.make_step_io(pos=pos, q=dev_bf16(x["q"]), q_idx=dev_bf16(qi), w_idx=dev_f32(x["w_idx"]),
                          kv_new=dev_bf16(x["kv_new"]), z_main=dev_f32(x["z_main"]), c_main=dev_f32(x["c_main"]),
                          z_idx=dev_f32(x["z_idx"]), c_idx=dev_f32(x["c_idx"]), **outs)
    ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    csa.csa_decode_step(L, io, ws)
    torch.cuda.synchronize()
    N = x["n_comp"] + 1
    for b in range(B):
        ost = oracle.LayerState(comp_kv=comp_vals[b].copy(), idx_keys=np.zeros((1000, 128)), n_comp=x["n_comp"],
                                swa=oracle.SwaRing(swa_vals[b].copy(), x["swa_head"], x["swa_len"]),
                                main_bias=x["main_bias"], idx_bias=x["idx_bias"], sink=x["sink"],
                                idx_codes=kc0[b].copy(), idx_scales=ks0[b].copy(), kv_mixed=True, rope_dim=ROPE,
                                rope_cos=rc.astype(np.float64), rope_sin=rs.astype(np.float64),
                                comp_rope_cos=cc.astype(np.float64), comp_rope_sin=cs.astype(np.float64))
        oracle.decode_step(ost, q=f(x["q"][b]), q_idx=f(qi[b]), w_idx=x["w_idx"][b], kv_new=f(x["kv_new"][b]), pos=pos,
                           top_k=K, z_main=x["z_main"][b], c_main=x["c_main"][b], z_idx=x["z_idx"][b],
                           c_idx=x["c_idx"][b], scale=1 / np.sqrt(512))
        # the new records: the ring one bit-exact, the entry within rounding; the key within E4M3 rounding
        c_, s_, rp_, _ = oracle.mixed_kv_row(f(x["kv_new"][b]), ROPE)
        np.testing.assert_array_equal(swa[b, x["swa_head"]].cpu().numpy(), record_of(c_, s_, rp_))
        _assert_entry_close(comp[b, N - 1].cpu().numpy(), ost.comp_kv[N - 1])
        gk, gs = kc[b, N - 1].cpu().numpy(), float(ks[b, N - 1])
        yi = oracle.compress(x["z_idx"][b], x["c_idx"][b], x["idx_bias"], 4)[-1]
        assert gs == pytest.approx(np.abs(yi).max() / 448, rel=1e-5)
        ost.comp_kv[:N] = decode_records(comp[b, :N].cpu().numpy())
        ost.idx_codes[:N], ost.idx_scales[:N] = kc[b, :N].cpu().numpy(), ks[b, :N].cpu().numpy()
        ref_s = oracle.index_score_fp8(qc[b][None], w8[b][None], ost.idx_codes[:N], ost.idx_scales[:N])[0]
        got_s = outs["scores"][b, :N].cpu().numpy().astype(np.float64)
        assert rel_err(got_s, ref_s) <= 1e-4
        gi, gc = outs["topk_idx"][b].cpu().numpy(), int(outs["topk_count"][b])
        np.testing.assert_array_equal(gi, oracle.topk(got_s[None], K)[0][0])
        assert_topk_gap_rule(gi, gc, ref_s, K)
        recs, ring = comp[b].cpu().numpy(), swa[b].cpu().numpy()
        head, ln = (x["swa_head"] + 1) % W, min(x["swa_len"] + 1, W)
        want_buf = np.stack([recs[i] for i in gi[:gc]] + [ring[(head - ln + j) % W] for j in range(ln)])
        nv = int(outs["n_valid"][b])
        assert nv == len(want_buf)
        np.testing.assert_array_equal(outs["gather_buf"][b, :nv].cpu().numpy(), want_buf)
        ro, rl = oracle.sparse_attn(f(x["q"][b]), decode_records(want_buf), x["sink"], 1 / np.sqrt(512))
        ro = oracle.rope_rotate(ro, rc[pos].astype(np.float64), rs[pos].astype(np.float64), inverse=True)
        assert rel_err(host_f64(outs["out"][b]), ro) <= 2e-2
        assert_lse_close(outs["lse"][b].cpu().numpy(), rl)


HCA_MIXED_CASES = [
    # name, ratio m, heads, entries before, cache capacity, window
    ("ratio8_h64", 8, 64, 37, 48, 8),           # a short block, folded since its scale spans every channel
    ("ratio64_h16_fold", 64, 16, 5, 40, 8),     # the block folded into the one attention workgroup
    ("ratio32_h32_fold", 32, 32, 20, 300, 16),  # folded over workgroups of empty splits too
]


@pytest.mark.parametrize("case", HCA_MIXED_CASES, ids=[c[0] for c in HCA_MIXED_CASES])
def test_hca_steps_in_sequence_mixed_kv(csa, case):
    """Twenty HCA steps over mixed caches (block completions, ring wrap),
    each against the oracle's evolving state: the ring record bit-exact, the
    compressed entry within E4M3 / bfloat16 rounding of the oracle's (then
    adopted), output and lse over every entry and the window."""
    name, m, H, n0, max_comp, W = case
    D = 512
    g = _g(7501 + m)
    f = numfmt.bf16_bits_to_f64
    pos0 = n0 * m + (5 if m == 8 else m - 10)
    comp_rec, comp_val = oracle_records(f(synth.to_bf16_bits(g.standard_normal((max_comp, D), dtype=np.float32))))
    swa_rec, swa_val = oracle_records(f(synth.to_bf16_bits(g.standard_normal((W, D), dtype=np.float32))))
    comp = torch.from_numpy(comp_rec[None].copy()).to(DEV)
    swa = torch.from_numpy(swa_rec[None].copy()).to(DEV)
    mb = g.standard_normal((m, D), dtype=np.float32) * np.float32(0.1)
    sink = g.standard_normal(H, dtype=np.float32)
    rc, rs = rope_tables(pos0 + 20)
    cc, cs = rope_tables((pos0 + 20) // m + 1, offset=0.25, base=500.0)
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=None, swa=swa, main_bias=dev_f32(mb), idx_bias=None,
                            sink=dev_f32(sink), n_comp=n0, swa_head=pos0 % W, swa_len=W, h=H, h_i=0, m=m, top_k=0,
                            rope=(dev_f32(rc), dev_f32(rs)), comp_rope=(dev_f32(cc), dev_f32(cs)))
    assert L.kv_dtype == csa.CSA_FP8_E4M3
    ost = oracle.LayerState(comp_kv=comp_val, idx_keys=np.zeros((max_comp, 1)), n_comp=n0,
                            swa=oracle.SwaRing(swa_val, pos0 % W, W), main_bias=mb.astype(np.float64),
                            idx_bias=np.zeros((m, 1)), sink=sink.astype(np.float64), m=m,
                            round_cache=numfmt.bf16_round_f64, kv_mixed=True, rope_dim=ROPE,
                            rope_cos=rc.astype(np.float64), rope_sin=rs.astype(np.float64),
                            comp_rope_cos=cc.astype(np.float64), comp_rope_sin=cs.astype(np.float64))
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
        print(f"mixed-KV HCA {name} pos={pos}", flush=True)
        slot = L.swa_head
        csa.csa_hca_decode_step(L, io, ws)
        csa.csa_layer_advance(L, pos)
        torch.cuda.synchronize()
        nprev = ost.n_comp
        r = oracle.hca_decode_step(ost, q=f(q[0]), kv_new=f(kvn[0]), pos=pos, z_main=zm[0], c_main=cm[0],
                                   scale=1 / np.sqrt(D))
        assert (L.n_comp, L.swa_head, L.swa_len) == (ost.n_comp, ost.swa.head, ost.swa.length)
        c_, s_, rp_, _ = oracle.mixed_kv_row(f(kvn[0]), ROPE)
        np.testing.assert_array_equal(swa[0, slot].cpu().numpy(), record_of(c_, s_, rp_))
        if pos % m == m - 1:  # the new entry within rounding, then adopt the GPU's record
            _assert_entry_close(comp[0, nprev].cpu().numpy(), ost.comp_kv[nprev])
            ost.comp_kv[nprev] = decode_records(comp[0, nprev].cpu().numpy())
            ro, rl = oracle.sparse_attn(f(q[0]), np.concatenate([ost.comp_kv[:ost.n_comp], r["rows"][ost.n_comp:]]),
                                        sink.astype(np.float64), 1 / np.sqrt(D))
            ro = oracle.rope_rotate(ro, ost.rope_cos[pos], ost.rope_sin[pos], inverse=True)
            r = {"out": ro, "lse": rl, "n_valid": ost.n_comp + ost.swa.length}
        assert int(n_valid[0]) == r["n_valid"]
        assert rel_err(host_f64(out[0]), r["out"]) <= 2e-2
        assert_lse_close(lse[0].cpu().numpy(), r["lse"])


def test_hca_step_full_size_mixed_kv(csa):
    """One HCA layer at 1M context (ratio 128: 7812 entries + the one this
    step completes, window 128 with wrap) over mixed caches packed on the
    GPU: the entry's record within rounding, output and lse against the
    oracle's attention over all 7941 decoded rows with the inverse rotation."""
    shape = synth.SHAPES["hca1m"]
    x = synth.make_decode_inputs_torch(shape, seed=None, device=DEV, layers=1)[0]
    H, W, m = shape.h, shape.w, shape.m
    comp = torch.empty(1, shape.max_comp, REC, dtype=torch.uint8, device=DEV)
    swa = torch.empty(1, W, REC, dtype=torch.uint8, device=DEV)
    csa.csa_pack_kv_mixed(x["comp_kv"], comp)
    csa.csa_pack_kv_mixed(x["swa"], swa)
    pos = x["pos"]
    rc, rs = rope_tables(pos + 1)
    cc, cs = rope_tables(shape.max_comp + 1, offset=0.25, base=500.0)
    L = csa.make_layer_desc(comp_kv=comp, idx_keys=None, swa=swa, main_bias=x["main_bias"], idx_bias=None,
                            sink=x["sink"], n_comp=x["n_comp"], swa_head=x["swa_head"], swa_len=x["swa_len"],
                            h=H, h_i=0, m=m, top_k=0, rope=(dev_f32(rc), dev_f32(rs)),
                            comp_rope=(dev_f32(cc), dev_f32(cs)))
    out = torch.empty(1, H, 512, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(1, H, device=DEV)
    n_valid = torch.empty(1, dtype=torch.int32, device=DEV)
    io = csa.make_step_io(pos=pos, q=x["q"], kv_new=x["kv_new"], z_main=x["z_main"], c_main=x["c_main"], out=out,
                          lse=lse, n_valid=n_valid)
    ws = torch.empty(csa.csa_hca_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
    slot = x["swa_head"]
    csa.csa_hca_decode_step(L, io, ws)
    torch.cuda.synchronize()
    N = x["n_comp"] + 1
    assert N == shape.n_comp and pos % m == m - 1
    ym = oracle.compress(host_f64(x["z_main"][0]), host_f64(x["c_main"][0]), host_f64(x["main_bias"]), m)[-1]
    blk = pos // m
    _, _, _, want = oracle.mixed_kv_row(ym, ROPE, cc[blk].astype(np.float64), cs[blk].astype(np.float64))
    _assert_entry_close(comp[0, N - 1].cpu().numpy(), want)
    c_, s_, rp_, _ = oracle.mixed_kv_row(host_f64(x["kv_new"][0]), ROPE)
    np.testing.assert_array_equal(swa[0, slot].cpu().numpy(), record_of(c_, s_, rp_))
    ring = swa[0].cpu().numpy()
    head = (x["swa_head"] + 1) % W
    rows = decode_records(np.concatenate([comp[0, :N].cpu().numpy(),
                                          np.stack([ring[(head - W + j) % W] for j in range(W)])]))
    assert int(n_valid[0]) == N + W
    ro, rl = oracle.sparse_attn(host_f64(x["q"][0]), rows, host_f64(x["sink"]), 1 / np.sqrt(512))
    ro = oracle.rope_rotate(ro, rc[pos].astype(np.float64), rs[pos].astype(np.float64), inverse=True)
    assert rel_err(host_f64(out[0]), ro) <= 2e-2
    assert_lse_close(lse[0].cpu().numpy(), rl)


PREFILL_MIXED_CASES = [
    # name, t, h, n_comp, k, window, pos0, sink, bf16 out, counts all k
    ("h64_ragged_counts", 40, 64, 300, 64, 16, 700, True, True, False),
    ("h32_f32_from_position0", 24, 32, 50, 40, 8, 0, False, False, True),
    ("h64_k512_window128", 6, 64, 2000, 512, 128, 9000, True, True, True),
]


@pytest.mark.parametrize("case", PREFILL_MIXED_CASES, ids=[c[0] for c in PREFILL_MIXED_CASES])
def test_prefill_attn_mixed_kv(csa, case):
    """csa_prefill_attn_mixed against the oracle: per query row, the softmax
    over the decoded records of its selected rows then its window rows, and
    the inverse rotation of the RoPE dims at the row's position."""
    name, t, h, n_comp, k, window, pos0, use_sink, out_bf16, full = case
    g = _g(7601 + t + h + n_comp)
    f = numfmt.bf16_bits_to_f64
    qn = synth.to_bf16_bits(g.standard_normal((t, h, 512), dtype=np.float32))
    comp_rec, comp_val = oracle_records(f(synth.to_bf16_bits(g.standard_normal((n_comp, 512), dtype=np.float32))))
    win_rec, win_val = oracle_records(f(synth.to_bf16_bits(g.standard_normal((t + window - 1, 512),
                                                                            dtype=np.float32))))
    sink = g.standard_normal(h, dtype=np.float32) if use_sink else None
    idx = np.stack([g.choice(n_comp, size=k, replace=False) for _ in range(t)]).astype(np.int32)
    cnt = np.full(t, k, dtype=np.int32) if full else g.integers(0, k + 1, size=t).astype(np.int32)
    for r in range(t):
        idx[r, cnt[r]:] = -1
    rc, rs = rope_tables(pos0 + t)
    out = torch.full((t, h, 512), 7.0, dtype=torch.bfloat16 if out_bf16 else torch.float32, device=DEV)
    lse = torch.empty(t, h, device=DEV)
    scale = 1.0 / np.sqrt(512)
    print(f"prefill mixed {name}", flush=True)
    csa.csa_prefill_attn_mixed(dev_bf16(qn), torch.from_numpy(comp_rec).to(DEV), torch.from_numpy(idx).to(DEV),
                               torch.from_numpy(cnt).to(DEV), torch.from_numpy(win_rec).to(DEV), window, pos0,
                               (dev_f32(rc), dev_f32(rs)), None if sink is None else dev_f32(sink), scale, out,
                               lse=lse)
    torch.cuda.synchronize()
    got, got_lse = host_f64(out), lse.cpu().numpy()
    for r in range(t):
        p = pos0 + r
        first = max(0, p - window + 1)
        wrows = [win_val[x - (pos0 - window + 1)] for x in range(first, p + 1)]
        rows = np.stack([comp_val[i] for i in idx[r, :cnt[r]]] + wrows)
        ro, rl = oracle.sparse_attn(f(qn[r]), rows, None if sink is None else sink.astype(np.float64), scale)
        ro = oracle.rope_rotate(ro, rc[p].astype(np.float64), rs[p].astype(np.float64), inverse=True)
        assert rel_err(got[r], ro) <= 2e-2, r
        assert_lse_close(got_lse[r], rl)
