"""GPU: the decode step with its counters on the device (csa_decode_step_dev)
captured once in a HIP graph and replayed step after step.  Every replay is
checked against the float64 oracle's evolving layer state (the compressed
entry and key within rounding of the oracle's, then adopted; scores, the
top-k by the gap rule, gather_buf and the attention output within the
stated tolerances), and, bit for bit, against the host-counter step
(csa_decode_step) on the same inputs: the two run the same kernels, only
where the counters come from differs.  Eager work and synchronisations run
between replays."""

import numpy as np
import pytest
import torch

import oracle
import synth
from oracle import numfmt
from tests.gpu_util import (DEV, assert_bf16_close, assert_fp4_key_close, assert_topk_gap_rule, dev_bf16, dev_f32,
                            host_bits, host_f64, rel_err)
from tests.test_gpu_mixed_kv import _assert_entry_close, decode_records, oracle_records, record_of
from tests.test_gpu_parity import _assert_e4m3_key_close

pytestmark = pytest.mark.gpu

REC = 592
ROPE = 64


@pytest.fixture(scope="module")
def csa():
    import compressed_sparse_attention_reduce_amd as pkg
    pkg.lib()
    return pkg


def _g(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _tables_np(rows, offset, base):
    ang = (np.arange(rows)[:, None] + offset) * base ** (-2.0 * np.arange(32)[None, :] / 64)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def _run(csa, *, mixed, overlap, B, n0, pos0, max_comp, steps, seed, W=8, K=64, fp8=False, fp4=False):
    fp8 = fp8 or fp4  # fp4: E2M1 keys, the E4M3 step's paths otherwise
    g = _g(seed)
    D, Di, H = 512, 128, 64
    m = 4
    f = numfmt.bf16_bits_to_f64
    scale = 1 / np.sqrt(D)
    wm, wi = (2 * D, 2 * Di) if overlap else (D, Di)
    comp_bits = synth.to_bf16_bits(g.standard_normal((B, max_comp, D), dtype=np.float32))
    keys_bits = synth.to_bf16_bits(g.standard_normal((B, max_comp, Di), dtype=np.float32))
    swa_bits = synth.to_bf16_bits(g.standard_normal((B, W, D), dtype=np.float32))
    mb_np = g.standard_normal((m, wm), dtype=np.float32) * np.float32(0.1)
    ib_np = g.standard_normal((m, wi), dtype=np.float32) * np.float32(0.1)
    sink_np = g.standard_normal(H, dtype=np.float32)
    mb, ib, sink = dev_f32(mb_np), dev_f32(ib_np), dev_f32(sink_np)
    rope_np = _tables_np(pos0 + steps + 4, 0.5, 10000.0) if mixed else None
    comp_rope_np = _tables_np(max_comp + 2, 0.25, 500.0) if mixed else None
    rope = tuple(dev_f32(t) for t in rope_np) if mixed else None
    comp_rope = tuple(dev_f32(t) for t in comp_rope_np) if mixed else None

    if fp4:
        c4, s4 = numfmt.quantize_mxfp4_rows(f(keys_bits).reshape(-1, Di).astype(np.float32))
        kc0 = numfmt.pack_e2m1(c4).reshape(B, max_comp, Di // 2)
        ks0 = s4.reshape(B, max_comp, Di // 32)
        oc0 = c4.reshape(B, max_comp, Di)              # the oracle's codes, one per element
    elif fp8:
        kc0, ks0 = numfmt.quantize_e4m3_rows(f(keys_bits).reshape(-1, Di).astype(np.float32))
        kc0, ks0 = kc0.reshape(B, max_comp, Di), ks0.reshape(B, max_comp)
        oc0 = kc0

    def caches():
        if fp4:
            keys = (torch.from_numpy(kc0.copy()).to(DEV), torch.from_numpy(ks0.copy()).to(DEV))
        else:
            keys = (torch.from_numpy(kc0.copy()).to(DEV), dev_f32(ks0)) if fp8 else dev_bf16(keys_bits)
        if mixed:
            comp = torch.empty(B, max_comp, REC, dtype=torch.uint8, device=DEV)
            swa = torch.empty(B, W, REC, dtype=torch.uint8, device=DEV)
            csa.csa_pack_kv_mixed(dev_bf16(comp_bits), comp)
            csa.csa_pack_kv_mixed(dev_bf16(swa_bits), swa)
        else:
            comp, swa = dev_bf16(comp_bits), dev_bf16(swa_bits)
        return comp, keys, swa

    def layer(comp, keys, swa):
        keys, scales = keys if fp8 else (keys, None)
        return csa.make_layer_desc(comp_kv=comp, idx_keys=keys, idx_scales=scales, swa=swa, main_bias=mb,
                                   idx_bias=ib, sink=sink,
                                   n_comp=n0, swa_head=pos0 % W, swa_len=min(pos0, W), h=H, h_i=64, top_k=K,
                                   overlap=overlap, rope=rope, comp_rope=comp_rope)

    def outs():
        return dict(scores=torch.zeros(B, max_comp, device=DEV),
                    topk_idx=torch.zeros(B, K, dtype=torch.int32, device=DEV),
                    topk_count=torch.zeros(B, dtype=torch.int32, device=DEV),
                    gather_buf=torch.zeros(B, K + W, REC if mixed else D,
                                           dtype=torch.uint8 if mixed else torch.bfloat16, device=DEV),
                    n_valid=torch.zeros(B, dtype=torch.int32, device=DEV),
                    out=torch.zeros(B, H, D, dtype=torch.bfloat16, device=DEV),
                    lse=torch.zeros(B, H, device=DEV))

    # one oracle layer state per sequence, from the same cache values
    osts = []
    for b in range(B):
        if mixed:
            comp_rec, comp_val = oracle_records(f(comp_bits[b]))
            _, swa_val = oracle_records(f(swa_bits[b]))
        else:
            comp_val, swa_val = f(comp_bits[b]), f(swa_bits[b])
        osts.append(oracle.LayerState(
            comp_kv=comp_val.copy(), idx_keys=np.zeros((max_comp, Di)) if fp8 else f(keys_bits[b]), n_comp=n0,
            swa=oracle.SwaRing(swa_val.copy(), pos0 % W, min(pos0, W)), main_bias=mb_np.astype(np.float64),
            idx_bias=ib_np.astype(np.float64), sink=sink_np.astype(np.float64), overlap=bool(overlap),
            round_cache=numfmt.bf16_round_f64,
            idx_codes=oc0[b].copy() if fp8 else None, idx_scales=ks0[b].copy() if fp8 else None, idx_fp4=fp4,
            kv_mixed=mixed, rope_dim=ROPE,
            rope_cos=rope_np[0].astype(np.float64) if mixed else None,
            rope_sin=rope_np[1].astype(np.float64) if mixed else None,
            comp_rope_cos=comp_rope_np[0].astype(np.float64) if mixed else None,
            comp_rope_sin=comp_rope_np[1].astype(np.float64) if mixed else None))

    ch, kh, sh = caches()
    Lh = layer(ch, kh, sh)
    cd, kd, sd = caches()
    Ld = layer(cd, kd, sd)
    if mixed:  # the library packs the caches as the oracle does
        np.testing.assert_array_equal(cd[0].cpu().numpy(), oracle_records(f(comp_bits[0]))[0])
    # static inputs of the captured step (the E4M3 step takes the bf16 query too)
    st_in = dict(q=torch.zeros(B, H, D, dtype=torch.bfloat16, device=DEV),
                 q_idx=torch.zeros(B, 64, Di, dtype=torch.bfloat16, device=DEV),
                 w_idx=torch.zeros(B, 64, device=DEV),
                 kv_new=torch.zeros(B, D, dtype=torch.bfloat16, device=DEV),
                 z_main=torch.zeros(B, wm, device=DEV), c_main=torch.zeros(B, wm, device=DEV),
                 z_idx=torch.zeros(B, wi, device=DEV), c_idx=torch.zeros(B, wi, device=DEV))
    od = outs()
    iod = csa.make_step_io(pos=0, **st_in, **od)
    state = torch.tensor([pos0, n0, pos0 % W, min(pos0, W), 0], dtype=torch.int32, device=DEV)
    ring = torch.zeros(csa.csa_decode_step_dev_ring_size(Ld) // 4, device=DEV)
    wsd = torch.empty(csa.csa_decode_step_workspace_size(Ld), dtype=torch.uint8, device=DEV)
    wsh = torch.empty(csa.csa_decode_step_workspace_size(Lh), dtype=torch.uint8, device=DEV)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            csa.csa_decode_step_dev(Ld, iod, state, ring, wsd, stream=stream)
    torch.cuda.synchronize()

    hist_z = {k: [] for k in ("z_main", "c_main", "z_idx", "c_idx")}
    for pos in range(pos0, pos0 + steps):
        x = dict(q=synth.to_bf16_bits(g.standard_normal((B, H, D), dtype=np.float32)),
                 q_idx=synth.to_bf16_bits(g.standard_normal((B, 64, Di), dtype=np.float32) / np.float32(np.sqrt(Di))),
                 w_idx=g.standard_normal((B, 64), dtype=np.float32),
                 kv_new=synth.to_bf16_bits(g.standard_normal((B, D), dtype=np.float32)),
                 z_main=g.standard_normal((B, wm), dtype=np.float32), c_main=g.standard_normal((B, wm), dtype=np.float32),
                 z_idx=g.standard_normal((B, wi), dtype=np.float32), c_idx=g.standard_normal((B, wi), dtype=np.float32))
        for k in hist_z:
            hist_z[k].append(x[k])
        # the captured step: new inputs into its static buffers, one replay
        dev_in = {k: (dev_bf16(v) if v.dtype == np.uint16 else dev_f32(v)) for k, v in x.items()}
        for k, v in dev_in.items():
            st_in[k].copy_(v)
        print(f"dev step pos={pos}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        # the host-counter step on the same inputs (block rows from the history)
        completes = pos % m == m - 1
        blk_np = {}
        for k in hist_z:
            rows = np.stack(hist_z[k][-m:], axis=1)                   # [B, m, w]
            if overlap and pos // m > 0:
                rows = np.stack(hist_z[k][-2 * m:], axis=1)           # previous block then this one
            blk_np[k] = np.ascontiguousarray(rows)
        blk = {k: dev_f32(v) if completes else dev_f32(np.zeros((B, m, v.shape[2]), np.float32))
               for k, v in blk_np.items()}
        oh = outs()
        ioh = csa.make_step_io(pos=pos, q=dev_in["q"], q_idx=dev_in["q_idx"], w_idx=dev_in["w_idx"],
                               kv_new=dev_in["kv_new"], **blk, **oh)
        slot = Lh.swa_head
        csa.csa_decode_step(Lh, ioh, wsh)
        csa.csa_layer_advance(Lh, pos)
        torch.cuda.synchronize()
        N = Lh.n_comp
        sv = state.cpu().numpy()
        assert (sv[0], sv[1], sv[2], sv[3], sv[4]) == (pos + 1, N, Lh.swa_head, Lh.swa_len, 0)

        # 1. against the oracle, sequence by sequence
        for b in range(B):
            ost = osts[b]
            nb = ost.n_comp
            r = oracle.decode_step(ost, q=f(x["q"][b]), q_idx=f(x["q_idx"][b]), w_idx=x["w_idx"][b],
                                   kv_new=f(x["kv_new"][b]), pos=pos, top_k=K,
                                   **{k: v[b] for k, v in blk_np.items()}, scale=scale)
            assert (ost.n_comp, ost.swa.head, ost.swa.length) == (N, Lh.swa_head, Lh.swa_len)
            # the new token's ring row
            if mixed:
                c_, s_, rp_, _ = oracle.mixed_kv_row(f(x["kv_new"][b]), ROPE)
                np.testing.assert_array_equal(sd[b, slot].cpu().numpy(), record_of(c_, s_, rp_))
            else:
                np.testing.assert_array_equal(host_bits(sd[b, slot]), x["kv_new"][b])
            # the compressed entry and key within rounding of the oracle's, then the GPU's adopted
            if completes:
                ym, yi = r["new_entry"]
                if mixed:
                    _assert_entry_close(cd[b, nb].cpu().numpy(), ost.comp_kv[nb])
                else:
                    assert_bf16_close(host_bits(cd[b, nb]), ym)
                if fp4:
                    assert_fp4_key_close(kd[0][b, nb].cpu().numpy(), kd[1][b, nb].cpu().numpy(), yi)
                elif fp8:
                    _assert_e4m3_key_close(kd[0][b, nb].cpu().numpy(), float(kd[1][b, nb]), yi)
                else:
                    assert_bf16_close(host_bits(kd[b, nb]), yi)
            ost.comp_kv[:N] = decode_records(cd[b, :N].cpu().numpy()) if mixed else host_f64(cd[b, :N])
            if fp8:
                gcodes = kd[0][b, :N].cpu().numpy()
                ost.idx_codes[:N] = numfmt.unpack_e2m1(gcodes) if fp4 else gcodes
                ost.idx_scales[:N] = kd[1][b, :N].cpu().numpy()
                qc, qs = numfmt.quantize_e4m3_rows(f(x["q_idx"][b]).astype(np.float32))
                w8 = (x["w_idx"][b] * qs).astype(np.float32)
                score_fn = oracle.index_score_fp4 if fp4 else oracle.index_score_fp8
                ref_s = score_fn(qc[None], w8[None], ost.idx_codes[:N], ost.idx_scales[:N])[0]
            else:
                ost.idx_keys[:N] = host_f64(kd[b, :N])
                ref_s = oracle.index_score(f(x["q_idx"][b])[None], x["w_idx"][b][None], ost.idx_keys[:N])[0]
            got_s = od["scores"][b, :N].cpu().numpy().astype(np.float64)
            assert rel_err(got_s, ref_s) <= 1e-4, (pos, b)
            gi, gc = od["topk_idx"][b].cpu().numpy(), int(od["topk_count"][b])
            np.testing.assert_array_equal(gi, oracle.topk(got_s[None], K)[0][0])
            assert_topk_gap_rule(gi, gc, ref_s, K)
            nv = int(od["n_valid"][b])
            if mixed:
                recs, ringr = cd[b].cpu().numpy(), sd[b].cpu().numpy()
                want_buf = np.stack([recs[i] for i in gi[:gc]] +
                                    [ringr[(ost.swa.head - ost.swa.length + j) % W] for j in range(ost.swa.length)])
                assert nv == len(want_buf)
                np.testing.assert_array_equal(od["gather_buf"][b, :nv].cpu().numpy(), want_buf)
                rows = decode_records(want_buf)
                np.testing.assert_array_equal(rows[gc:], oracle.gather(ost.comp_kv[:N], gi, gc, ost.swa.rows,
                                                                       ost.swa.head, ost.swa.length)[0][gc:])
            else:
                rows, n_valid = oracle.gather(ost.comp_kv[:N], gi, gc, ost.swa.rows, ost.swa.head, ost.swa.length)
                assert nv == n_valid
                np.testing.assert_array_equal(host_f64(od["gather_buf"][b, :nv]), rows)
            ro, rl = oracle.sparse_attn(f(x["q"][b]), rows, ost.sink, scale)
            if mixed:
                ro = oracle.rope_rotate(ro, ost.rope_cos[pos], ost.rope_sin[pos], inverse=True)
            assert rel_err(host_f64(od["out"][b]), ro) <= 2e-2, (pos, b)
            gl = od["lse"][b].cpu().numpy()
            assert rel_err(gl, rl) <= 2e-2 and np.abs(gl - rl).max() <= 1e-2, (pos, b)

        # 2. bit for bit against the host-counter step
        assert torch.equal(od["scores"][:, :N], oh["scores"][:, :N])
        for k in ("topk_idx", "topk_count", "n_valid", "out", "lse"):
            assert torch.equal(od[k], oh[k]), (pos, k)
        nv = int(oh["n_valid"].min())
        assert torch.equal(od["gather_buf"][:, :nv], oh["gather_buf"][:, :nv])
        if fp8:
            assert torch.equal(kd[0][:, :N], kh[0][:, :N]) and torch.equal(kd[1][:, :N], kh[1][:, :N])
        else:
            assert torch.equal(kd[:, :N], kh[:, :N])
        assert torch.equal(cd[:, :N], ch[:, :N]) and torch.equal(sd, sh)
    return state, cd, ch


def test_dev_step_graph_replays_match_host_steps(csa):
    """Ten replays from a block start (two completions, ring wrap), batch 2."""
    _run(csa, mixed=False, overlap=0, B=2, n0=150, pos0=600, max_comp=200, steps=10, seed=8101)


def test_dev_step_overlap_and_mixed_kv(csa):
    """The overlapped compressor (the ring keeps the previous block) and mixed
    main KV (RoPE rows from the device position), from the first token."""
    _run(csa, mixed=True, overlap=1, B=1, n0=0, pos0=0, max_comp=16, steps=13, seed=8102)


def test_dev_step_fp8_keys(csa):
    """E4M3 indexer keys (the new key quantised in the step), batch 2."""
    _run(csa, mixed=False, overlap=0, B=2, n0=150, pos0=600, max_comp=200, steps=9, seed=8104, fp8=True)


def test_dev_step_fp4_keys(csa):
    """E2M1 indexer keys with E8M0 block scales (the new key quantised in the
    step), batch 2."""
    _run(csa, mixed=False, overlap=0, B=2, n0=150, pos0=600, max_comp=200, steps=9, seed=8105, fp4=True)


def test_dev_step_fp4_keys_overlap_and_mixed_kv(csa):
    """E2M1 indexer keys with the overlapped compressor and mixed main KV,
    from the first token (the new key quantised from the overlapped block's
    compression), batch 2."""
    _run(csa, mixed=True, overlap=1, B=2, n0=0, pos0=0, max_comp=16, steps=13, seed=8106, fp4=True)


def test_dev_step_batched_separate_topk(csa):
    """Batch 4 at top_k 512, window 128: 4 x 80 fused workgroups would not all
    be resident, so the device-counter step takes one top-k launch per
    sequence (entry count from the device state, candidate lists from the
    scan) and the 256-thread attention; five replays from a block start, one
    block completion."""
    _run(csa, mixed=False, overlap=0, B=4, n0=8000, pos0=32000, max_comp=8200, steps=5, seed=8105, W=128, K=512)


def test_dev_step_full_cache_sets_flag(csa):
    """A block completing into a full cache writes nothing, keeps n_comp and
    sets bit 0 of the flags; the step's attention is the one of a step that
    completes nothing (the host step one position earlier, same state)."""
    g = _g(8103)
    B, D, Di, H, W, K, m = 1, 512, 128, 64, 8, 64, 4
    max_comp = n0 = 20
    pos = 79  # completes block 19, but the cache is full
    comp = dev_bf16(synth.to_bf16_bits(g.standard_normal((B, max_comp, D), dtype=np.float32)))
    keys = dev_bf16(synth.to_bf16_bits(g.standard_normal((B, max_comp, Di), dtype=np.float32)))
    swa_bits = synth.to_bf16_bits(g.standard_normal((B, W, D), dtype=np.float32))
    mb = dev_f32(g.standard_normal((m, D), dtype=np.float32))
    ib = dev_f32(g.standard_normal((m, Di), dtype=np.float32))
    sink = dev_f32(g.standard_normal(H, dtype=np.float32))
    x = dict(q=dev_bf16(synth.to_bf16_bits(g.standard_normal((B, H, D), dtype=np.float32))),
             q_idx=dev_bf16(synth.to_bf16_bits(g.standard_normal((B, 64, Di), dtype=np.float32))),
             w_idx=dev_f32(g.standard_normal((B, 64), dtype=np.float32)),
             kv_new=dev_bf16(synth.to_bf16_bits(g.standard_normal((B, D), dtype=np.float32))))
    res = []
    for dev in (True, False):
        swa = dev_bf16(swa_bits)
        L = csa.make_layer_desc(comp_kv=comp, idx_keys=keys, swa=swa, main_bias=mb, idx_bias=ib, sink=sink,
                                n_comp=n0, swa_head=3, swa_len=W, h=H, h_i=64, top_k=K)
        o = dict(scores=torch.zeros(B, max_comp, device=DEV), topk_idx=torch.zeros(B, K, dtype=torch.int32, device=DEV),
                 topk_count=torch.zeros(B, dtype=torch.int32, device=DEV),
                 gather_buf=torch.zeros(B, K + W, D, dtype=torch.bfloat16, device=DEV),
                 n_valid=torch.zeros(B, dtype=torch.int32, device=DEV),
                 out=torch.zeros(B, H, D, dtype=torch.bfloat16, device=DEV), lse=torch.zeros(B, H, device=DEV))
        zc = dict(z_main=torch.ones(B, m, D, device=DEV), c_main=torch.ones(B, m, D, device=DEV),
                  z_idx=torch.ones(B, m, Di, device=DEV), c_idx=torch.ones(B, m, Di, device=DEV))
        ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
        before = comp.clone()
        if dev:
            io = csa.make_step_io(pos=0, **x, **{k: v[:, 0].contiguous() for k, v in zc.items()}, **o)
            state = torch.tensor([pos, n0, 3, W, 0], dtype=torch.int32, device=DEV)
            ring = torch.zeros(csa.csa_decode_step_dev_ring_size(L) // 4, device=DEV)
            csa.csa_decode_step_dev(L, io, state, ring, ws)
            torch.cuda.synchronize()
            assert state.cpu().tolist() == [pos + 1, n0, 4, W, 1]
        else:
            io = csa.make_step_io(pos=pos - 1, **x, **zc, **o)
            csa.csa_decode_step(L, io, ws)
            torch.cuda.synchronize()
        assert torch.equal(comp, before)
        res.append((o, swa))
    (od, sd), (oh, sh) = res
    for k in ("scores", "topk_idx", "topk_count", "n_valid", "gather_buf", "out", "lse"):
        assert torch.equal(od[k], oh[k]), k
    assert torch.equal(sd, sh)


# ---------------------------------------------------------------------------
# HCA layers with device counters (csa_hca_decode_step_dev)
# ---------------------------------------------------------------------------

HCA_DEV_CASES = [
    # name, ratio m, heads, entries before, capacity, window, batch, mixed KV, main norm, replays
    ("ratio128_bf16_batch2", 128, 64, 20, 40, 16, 2, False, False, 130),
    ("ratio8_mixed", 8, 16, 10, 60, 8, 1, True, False, 30),
    ("ratio16_norm", 16, 32, 5, 30, 8, 1, False, True, 40),
]


@pytest.mark.parametrize("case", HCA_DEV_CASES, ids=[c[0] for c in HCA_DEV_CASES])
def test_hca_dev_step_graph_replays(csa, case):
    """One captured graph of csa_hca_decode_step_dev replayed step after step
    from a block's first token across a block boundary (ratio 128: 130
    replays, the block completing at the 128th); each replay against
    oracle.hca_decode_step over the evolving state (the new entry within
    rounding, then adopted; output and lse within the stated tolerances) and
    bit for bit against csa_hca_decode_step with host counters."""
    name, m, H, n0, max_comp, W, B, mixed, norm, steps = case
    D = 512
    g = _g(8201 + m + B)
    f = numfmt.bf16_bits_to_f64
    scale = 1 / np.sqrt(D)
    pos0 = n0 * m  # a block's first token
    comp_bits = synth.to_bf16_bits(g.standard_normal((B, max_comp, D), dtype=np.float32))
    swa_bits = synth.to_bf16_bits(g.standard_normal((B, W, D), dtype=np.float32))
    mb_np = g.standard_normal((m, D), dtype=np.float32) * np.float32(0.1)
    sink_np = g.standard_normal(H, dtype=np.float32)
    norm_np = (1 + 0.1 * g.standard_normal(D)).astype(np.float32) if norm else None
    rope_np = _tables_np(pos0 + steps + 4, 0.5, 10000.0) if mixed else None
    comp_rope_np = _tables_np(max_comp + 2, 0.25, 500.0) if mixed else None
    rope = tuple(dev_f32(t) for t in rope_np) if mixed else None
    comp_rope = tuple(dev_f32(t) for t in comp_rope_np) if mixed else None

    def caches():
        if mixed:
            comp = torch.empty(B, max_comp, REC, dtype=torch.uint8, device=DEV)
            swa = torch.empty(B, W, REC, dtype=torch.uint8, device=DEV)
            csa.csa_pack_kv_mixed(dev_bf16(comp_bits), comp)
            csa.csa_pack_kv_mixed(dev_bf16(swa_bits), swa)
            return comp, swa
        return dev_bf16(comp_bits), dev_bf16(swa_bits)

    def layer(comp, swa):
        return csa.make_layer_desc(comp_kv=comp, idx_keys=None, swa=swa, main_bias=dev_f32(mb_np), idx_bias=None,
                                   sink=dev_f32(sink_np), n_comp=n0, swa_head=pos0 % W, swa_len=min(pos0, W), h=H,
                                   h_i=0, m=m, top_k=0, main_norm=None if norm_np is None else dev_f32(norm_np),
                                   rope=rope, comp_rope=comp_rope)

    def outs():
        return dict(out=torch.zeros(B, H, D, dtype=torch.bfloat16, device=DEV), lse=torch.zeros(B, H, device=DEV),
                    n_valid=torch.zeros(B, dtype=torch.int32, device=DEV))

    osts = []
    for b in range(B):
        if mixed:
            _, comp_val = oracle_records(f(comp_bits[b]))
            _, swa_val = oracle_records(f(swa_bits[b]))
        else:
            comp_val, swa_val = f(comp_bits[b]), f(swa_bits[b])
        osts.append(oracle.LayerState(
            comp_kv=comp_val.copy(), idx_keys=np.zeros((max_comp, 1)), n_comp=n0,
            swa=oracle.SwaRing(swa_val.copy(), pos0 % W, min(pos0, W)), main_bias=mb_np.astype(np.float64),
            idx_bias=np.zeros((m, 1)), sink=sink_np.astype(np.float64), m=m, round_cache=numfmt.bf16_round_f64,
            main_norm=None if norm_np is None else norm_np.astype(np.float64), kv_mixed=mixed, rope_dim=ROPE,
            rope_cos=rope_np[0].astype(np.float64) if mixed else None,
            rope_sin=rope_np[1].astype(np.float64) if mixed else None,
            comp_rope_cos=comp_rope_np[0].astype(np.float64) if mixed else None,
            comp_rope_sin=comp_rope_np[1].astype(np.float64) if mixed else None))

    ch, sh = caches()
    Lh = layer(ch, sh)
    cd, sd = caches()
    Ld = layer(cd, sd)
    st_in = dict(q=torch.zeros(B, H, D, dtype=torch.bfloat16, device=DEV),
                 kv_new=torch.zeros(B, D, dtype=torch.bfloat16, device=DEV),
                 z_main=torch.zeros(B, D, device=DEV), c_main=torch.zeros(B, D, device=DEV))
    od = outs()
    iod = csa.make_step_io(pos=0, **st_in, **od)
    state = torch.tensor([pos0, n0, pos0 % W, min(pos0, W), 0], dtype=torch.int32, device=DEV)
    ring = torch.zeros(csa.csa_hca_decode_step_dev_ring_size(Ld) // 4, device=DEV)
    wsd = torch.empty(csa.csa_hca_decode_step_workspace_size(Ld), dtype=torch.uint8, device=DEV)
    wsh = torch.empty(csa.csa_hca_decode_step_workspace_size(Lh), dtype=torch.uint8, device=DEV)
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            csa.csa_hca_decode_step_dev(Ld, iod, state, ring, wsd, stream=stream)
    torch.cuda.synchronize()

    hist = {"z_main": [], "c_main": []}
    completions = 0
    for pos in range(pos0, pos0 + steps):
        x = dict(q=synth.to_bf16_bits(g.standard_normal((B, H, D), dtype=np.float32)),
                 kv_new=synth.to_bf16_bits(g.standard_normal((B, D), dtype=np.float32)),
                 z_main=g.standard_normal((B, D), dtype=np.float32), c_main=g.standard_normal((B, D), dtype=np.float32))
        for k in hist:
            hist[k].append(x[k])
        dev_in = {k: (dev_bf16(v) if v.dtype == np.uint16 else dev_f32(v)) for k, v in x.items()}
        for k, v in dev_in.items():
            st_in[k].copy_(v)
        if pos % 16 == 0 or pos % m >= m - 2:
            print(f"hca dev step {name} pos={pos}", flush=True)
        graph.replay()
        torch.cuda.synchronize()
        completes = pos % m == m - 1
        blk_np = {k: np.ascontiguousarray(np.stack(hist[k][-m:], axis=1)) for k in hist}   # [B, <=m, D]
        blk = {k: dev_f32(v) if completes else dev_f32(np.zeros((B, m, D), np.float32)) for k, v in blk_np.items()}
        oh = outs()
        ioh = csa.make_step_io(pos=pos, q=dev_in["q"], kv_new=dev_in["kv_new"], **blk, **oh)
        slot = Lh.swa_head
        csa.csa_hca_decode_step(Lh, ioh, wsh)
        csa.csa_layer_advance(Lh, pos)
        torch.cuda.synchronize()
        N = Lh.n_comp
        sv = state.cpu().numpy()
        assert (sv[0], sv[1], sv[2], sv[3], sv[4]) == (pos + 1, N, Lh.swa_head, Lh.swa_len, 0), (pos, sv)
        completions += int(completes)
        for b in range(B):
            ost = osts[b]
            nb = ost.n_comp
            r = oracle.hca_decode_step(ost, q=f(x["q"][b]), kv_new=f(x["kv_new"][b]), pos=pos,
                                       z_main=blk_np["z_main"][b], c_main=blk_np["c_main"][b], scale=scale)
            assert ost.n_comp == N
            if mixed:
                c_, s_, rp_, _ = oracle.mixed_kv_row(f(x["kv_new"][b]), ROPE)
                np.testing.assert_array_equal(sd[b, slot].cpu().numpy(), record_of(c_, s_, rp_))
            else:
                np.testing.assert_array_equal(host_bits(sd[b, slot]), x["kv_new"][b])
            if completes:  # the new entry within rounding of the oracle's, then the GPU's adopted
                if mixed:
                    _assert_entry_close(cd[b, nb].cpu().numpy(), ost.comp_kv[nb])
                    ost.comp_kv[nb] = decode_records(cd[b, nb].cpu().numpy())
                else:
                    assert_bf16_close(host_bits(cd[b, nb]), r["new_entry"])  # (normalised when there is a norm)
                    ost.comp_kv[nb] = host_f64(cd[b, nb])
            win = r["rows"][nb + (1 if completes else 0):]
            rows = np.concatenate([ost.comp_kv[:N], win])
            ro, rl = oracle.sparse_attn(f(x["q"][b]), rows, ost.sink, scale)
            if mixed:
                ro = oracle.rope_rotate(ro, ost.rope_cos[pos], ost.rope_sin[pos], inverse=True)
            assert int(od["n_valid"][b]) == rows.shape[0]
            assert rel_err(host_f64(od["out"][b]), ro) <= 2e-2, (pos, b)
            gl = od["lse"][b].cpu().numpy()
            assert rel_err(gl, rl) <= 2e-2 and np.abs(gl - rl).max() <= 1e-2, (pos, b)
        for k in ("out", "lse", "n_valid"):
            assert torch.equal(od[k], oh[k]), (pos, k)
        assert torch.equal(cd[:, :N], ch[:, :N]) and torch.equal(sd, sh)
    assert completions >= 1


def test_hca_dev_step_full_cache_sets_flag(csa):
    """A ratio-8 block completing into a full cache writes nothing, keeps
    n_comp and sets bit 0 of the flags; the attention is the host step's that
    completes nothing (position one earlier, same state)."""
    g = _g(8301)
    B, D, H, W, m = 1, 512, 16, 8, 8
    max_comp = n0 = 12
    pos = n0 * m + m - 1
    comp = dev_bf16(synth.to_bf16_bits(g.standard_normal((B, max_comp, D), dtype=np.float32)))
    swa_bits = synth.to_bf16_bits(g.standard_normal((B, W, D), dtype=np.float32))
    mb = dev_f32(g.standard_normal((m, D), dtype=np.float32))
    sink = dev_f32(g.standard_normal(H, dtype=np.float32))
    x = dict(q=dev_bf16(synth.to_bf16_bits(g.standard_normal((B, H, D), dtype=np.float32))),
             kv_new=dev_bf16(synth.to_bf16_bits(g.standard_normal((B, D), dtype=np.float32))))
    res = []
    for dev in (True, False):
        swa = dev_bf16(swa_bits)
        L = csa.make_layer_desc(comp_kv=comp, idx_keys=None, swa=swa, main_bias=mb, idx_bias=None, sink=sink,
                                n_comp=n0, swa_head=3, swa_len=W, h=H, h_i=0, m=m, top_k=0)
        o = dict(out=torch.zeros(B, H, D, dtype=torch.bfloat16, device=DEV), lse=torch.zeros(B, H, device=DEV),
                 n_valid=torch.zeros(B, dtype=torch.int32, device=DEV))
        ws = torch.empty(csa.csa_hca_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
        before = comp.clone()
        if dev:
            io = csa.make_step_io(pos=0, **x, z_main=torch.ones(B, D, device=DEV), c_main=torch.ones(B, D, device=DEV),
                                  **o)
            state = torch.tensor([pos, n0, 3, W, 0], dtype=torch.int32, device=DEV)
            ring = torch.zeros(csa.csa_hca_decode_step_dev_ring_size(L) // 4, device=DEV)
            csa.csa_hca_decode_step_dev(L, io, state, ring, ws)
            torch.cuda.synchronize()
            assert state.cpu().tolist() == [pos + 1, n0, 4, W, 1]
        else:
            io = csa.make_step_io(pos=pos - 1, **x, z_main=torch.ones(B, m, D, device=DEV),
                                  c_main=torch.ones(B, m, D, device=DEV), **o)
            csa.csa_hca_decode_step(L, io, ws)
            torch.cuda.synchronize()
        assert torch.equal(comp, before)
        res.append((o, swa))
    (od, sd), (oh, sh) = res
    for k in ("out", "lse", "n_valid"):
        assert torch.equal(od[k], oh[k]), k
    assert torch.equal(sd, sh)
