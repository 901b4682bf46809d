"""GPU: csa_decode_step_noalloc (the decode step with the library's own fixed
device scratch, for callers that cannot allocate) against csa_decode_step
with a caller workspace, through the C ABI.  The two run the same kernels,
so every output and every cache write must match bit for bit.  Two calls in
a row share the scratch: the second, smaller one must not see anything the
first left behind."""

import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import DEV, dev_bf16, dev_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def csa():
    import compressed_sparse_attention_reduce_amd as pkg
    pkg.lib()
    return pkg


def _step(csa, x, shape, noalloc):
    B, K, W, D = shape.batch, shape.top_k, shape.w, shape.d
    caches = dict(comp_kv=dev_bf16(x["comp_kv"]), idx_keys=dev_bf16(x["idx_keys"]), swa=dev_bf16(x["swa"]))
    L = csa.make_layer_desc(**caches, main_bias=dev_f32(x["main_bias"]), idx_bias=dev_f32(x["idx_bias"]),
                            sink=dev_f32(x["sink"]), n_comp=x["n_comp"], swa_head=x["swa_head"],
                            swa_len=x["swa_len"], h=shape.h, h_i=shape.h_i, top_k=K)
    outs = dict(scores=torch.full((B, shape.max_comp), -7.0, device=DEV),
                topk_idx=torch.full((B, K), -9, dtype=torch.int32, device=DEV),
                topk_count=torch.full((B,), -9, dtype=torch.int32, device=DEV),
                gather_buf=torch.zeros(B, K + W, D, dtype=torch.bfloat16, device=DEV),
                n_valid=torch.full((B,), -9, dtype=torch.int32, device=DEV),
                out=torch.zeros(B, shape.h, D, dtype=torch.bfloat16, device=DEV),
                lse=torch.zeros(B, shape.h, device=DEV))
    io = csa.make_step_io(pos=x["pos"], q=dev_bf16(x["q"]), q_idx=dev_bf16(x["q_idx"]), w_idx=dev_f32(x["w_idx"]),
                          kv_new=dev_bf16(x["kv_new"]), z_main=dev_f32(x["z_main"]), c_main=dev_f32(x["c_main"]),
                          z_idx=dev_f32(x["z_idx"]), c_idx=dev_f32(x["c_idx"]), **outs)
    if noalloc:
        csa.csa_decode_step_noalloc(L, io)
    else:
        ws = torch.empty(csa.csa_decode_step_workspace_size(L), dtype=torch.uint8, device=DEV)
        csa.csa_decode_step(L, io, ws)
    torch.cuda.synchronize()
    return outs, caches


def _compare(got, want, shape):
    (og, cg), (ow, cw) = got, want
    N = shape.n_comp
    assert torch.equal(og["scores"][:, :N], ow["scores"][:, :N])
    for k in ("topk_idx", "topk_count", "n_valid", "out", "lse"):
        assert torch.equal(og[k], ow[k]), k
    nv = int(ow["n_valid"].min())
    assert nv == min(shape.top_k, shape.n_comp) + shape.w
    assert torch.equal(og["gather_buf"][:, :nv], ow["gather_buf"][:, :nv])
    for k in ("comp_kv", "idx_keys", "swa"):
        assert torch.equal(cg[k], cw[k]), k


def test_noalloc_matches_workspace_step_twice(csa):
    """First 8 sequences at 16K context (the split top-k + attention path,
    about 25 MB of scratch), then one sequence at 1200 context (the short-row
    exact path): each bit-identical to csa_decode_step."""
    need = []
    for name, shape, seed in (
            ("batch8", synth.with_(synth.SHAPES["batch128k"], n_comp=4096, ctx=16384), 9201),
            ("batch1", synth.with_(synth.SHAPES["ctx8k"], n_comp=300, ctx=1200), 9202)):
        x = synth.make_decode_inputs(shape, seed)
        print(f"no-alloc step {name}: batch {shape.batch} n_comp {shape.n_comp}", flush=True)
        got = _step(csa, x, shape, noalloc=True)
        want = _step(csa, x, shape, noalloc=False)
        _compare(got, want, shape)
        L = csa.make_layer_desc(comp_kv=got[1]["comp_kv"], idx_keys=got[1]["idx_keys"], swa=got[1]["swa"],
                                main_bias=dev_f32(x["main_bias"]), idx_bias=dev_f32(x["idx_bias"]), sink=None,
                                n_comp=x["n_comp"], swa_head=0, swa_len=0, h=shape.h, h_i=64, top_k=shape.top_k)
        need.append(csa.csa_decode_step_workspace_size(L))
    assert need[0] > need[1] and need[0] <= csa.csa_decode_step_noalloc_max_bytes()
