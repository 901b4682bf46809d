"""CPU-only checks of the C-ABI library: it loads, exports every symbol that
include/csa.h declares, lays out its structs as the C compiler does, and
rejects bad host-known arguments before anything is enqueued (no GPU call is
made by any test here)."""

import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from tests.conftest import ROOT

HEADER = os.path.join(ROOT, "include", "csa.h")
FAKE = 0x10000  # never dereferenced: validation fails before any device work


@pytest.fixture(scope="module")
def csa():
    import compressed_sparse_attention_reduce_amd as pkg
    from compressed_sparse_attention_reduce_amd import binding
    if not os.path.exists(binding.LIB_PATH):
        from compressed_sparse_attention_reduce_amd.build import build
        build()
    pkg.lib()
    return pkg


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(csa):
    names = _declared_functions()
    assert {"csa_compress", "csa_index_score", "csa_topk", "csa_gather", "csa_sparse_attn",
            "csa_decode_step"} <= set(names)
    lib = csa.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", csa.binding.LIB_PATH], capture_output=True, text=True)
    exported = set(re.findall(r" T (\w+)", out.stdout))
    missing = [n for n in names if n not in exported]
    assert not missing, f"not exported: {missing}"
    for n in names:
        assert hasattr(lib, n)


def test_struct_layout_matches_c(csa):
    from compressed_sparse_attention_reduce_amd.binding import LayerDesc, StepIO
    fields = {"csa_layer_desc": LayerDesc, "csa_step_io": StepIO}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void){"]
    for cname, cls in fields.items():
        lines.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        exe = os.path.join(d, "t")
        open(src, "w").write("\n".join(lines))
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", src, "-o", exe], check=True)
        res = dict(l.split() for l in subprocess.run([exe], capture_output=True, text=True).stdout.splitlines())
    for cname, cls in fields.items():
        assert int(res[cname]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(res[f"{cname}.{f}"]) == getattr(cls, f).offset, f"{cname}.{f}"


def test_compress_rejects_bad_args(csa):
    lib = csa.lib()
    ok_args = [FAKE, FAKE, FAKE, None, FAKE, 0, 1, 1, 4, 128, 0, 0, 0, 0, None]

    def call(**kw):
        a = list(ok_args)
        names = ["z", "c", "bias", "norm", "out", "odt", "batch", "nb", "m", "d", "ov", "fb", "zs", "os", "s"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return lib.csa_compress(*a)

    assert call(z=None) == csa.binding.CSA_ERR_INVALID_ARG
    assert "null" in csa.csa_last_error()
    assert call(m=0) == csa.binding.CSA_ERR_INVALID_ARG
    assert call(d=5000) == csa.binding.CSA_ERR_INVALID_ARG
    assert call(ov=2) == csa.binding.CSA_ERR_INVALID_ARG
    assert call(odt=7) == csa.binding.CSA_ERR_INVALID_ARG
    assert call(batch=2) == csa.binding.CSA_ERR_INVALID_ARG  # zero batch strides with batch 2


def test_index_score_rejects_bad_args(csa):
    lib = csa.lib()
    B = csa.binding
    base = [FAKE, FAKE, FAKE, FAKE, B.CSA_BF16, 1, 1, 64, 128, 1000, None, 4, 0, 0, 0, 0, 1000, None]
    a = list(base); a[7] = 32
    assert lib.csa_index_score(*a) == B.CSA_ERR_UNSUPPORTED
    a = list(base); a[0] = None
    assert lib.csa_index_score(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[16] = 10  # ld_s < n
    assert lib.csa_index_score(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[0] = FAKE + 2  # misaligned bf16 q
    assert lib.csa_index_score(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[4] = B.CSA_F32; a[8] = 512
    assert lib.csa_index_score(*a) == B.CSA_ERR_UNSUPPORTED


def test_fp8_entry_points_reject_bad_args(csa):
    lib = csa.lib()
    B = csa.binding
    q = [FAKE, B.CSA_F32, FAKE, FAKE, 10, 128, None]
    a = list(q); a[1] = B.CSA_FP8_E4M3          # input must be float32 or bf16
    assert lib.csa_quantize_fp8(*a) == B.CSA_ERR_INVALID_ARG
    a = list(q); a[5] = 0
    assert lib.csa_quantize_fp8(*a) == B.CSA_ERR_INVALID_ARG
    a = list(q); a[2] = None
    assert lib.csa_quantize_fp8(*a) == B.CSA_ERR_INVALID_ARG
    a = list(q); a[0] = None; a[2] = None; a[3] = None; a[4] = 0   # nothing to do
    assert lib.csa_quantize_fp8(*a) == B.CSA_OK
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 128, 1000, None, 4, 0, 0, 0, 0, 0, 1000, None]
    a = list(base); a[8] = 64
    assert lib.csa_index_score_fp8(*a) == B.CSA_ERR_UNSUPPORTED
    a = list(base); a[3] = None                 # no key scales
    assert lib.csa_index_score_fp8(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[17] = 999                 # ld_s < n
    assert lib.csa_index_score_fp8(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[2] = FAKE + 8             # misaligned keys
    assert lib.csa_index_score_fp8(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[5] = 2; a[14] = 8         # batch stride that breaks alignment
    assert lib.csa_index_score_fp8(*a) == B.CSA_ERR_INVALID_ARG


def test_fp4_entry_points_reject_bad_args(csa):
    lib = csa.lib()
    B = csa.binding
    q = [FAKE, B.CSA_F32, FAKE, FAKE, 10, 128, None]
    a = list(q); a[1] = B.CSA_FP4_E2M1          # input must be float32 or bf16
    assert lib.csa_quantize_fp4(*a) == B.CSA_ERR_INVALID_ARG
    for d in (0, 16, 48, 100):                  # whole 32-element blocks only
        a = list(q); a[5] = d
        assert lib.csa_quantize_fp4(*a) == B.CSA_ERR_INVALID_ARG
    a = list(q); a[3] = None                    # no scales
    assert lib.csa_quantize_fp4(*a) == B.CSA_ERR_INVALID_ARG
    a = list(q); a[0] = None; a[2] = None; a[3] = None; a[4] = 0   # nothing to do
    assert lib.csa_quantize_fp4(*a) == B.CSA_OK
    base = [FAKE, FAKE, FAKE, FAKE, FAKE, 1, 1, 64, 128, 1000, None, 4, 0, 0, 0, 0, 0, 1000, None]
    a = list(base); a[8] = 64
    assert lib.csa_index_score_fp4(*a) == B.CSA_ERR_UNSUPPORTED
    a = list(base); a[3] = None                 # no block scales
    assert lib.csa_index_score_fp4(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[17] = 999                 # ld_s < n
    assert lib.csa_index_score_fp4(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[2] = FAKE + 8             # misaligned keys
    assert lib.csa_index_score_fp4(*a) == B.CSA_ERR_INVALID_ARG
    # the chunk selections over FP4 keys: the E4M3 forms' rules
    tk = [FAKE, FAKE, FAKE, FAKE, 16, 64, 128, 1000, 0, 4, 64, FAKE, FAKE, FAKE, 1 << 30, None]
    a = list(tk); a[3] = None                   # no block scales
    assert lib.csa_index_topk_fp4(*a) == B.CSA_ERR_INVALID_ARG
    a = list(tk); a[5] = 32
    assert lib.csa_index_topk_fp4(*a) == B.CSA_ERR_UNSUPPORTED
    a = list(tk); a[14] = 16                    # short workspace
    assert lib.csa_index_topk_fp4(*a) == B.CSA_ERR_WORKSPACE
    rs = [FAKE, FAKE, FAKE, FAKE, FAKE, 16, 64, 128, 1000, 0, 4, 64, 256, FAKE, FAKE, FAKE, 1 << 30, None]
    a = list(rs); a[4] = None                   # no bfloat16 keys
    assert lib.csa_index_topk_fp4_rescored(*a) == B.CSA_ERR_INVALID_ARG
    a = list(rs); a[12] = 32                    # k_cand < top_k
    assert lib.csa_index_topk_fp4_rescored(*a) == B.CSA_ERR_INVALID_ARG
    a = list(rs); a[16] = 16
    assert lib.csa_index_topk_fp4_rescored(*a) == B.CSA_ERR_WORKSPACE


def test_calib_symbols_are_exported_by_their_own_library(csa):
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "csa_calib.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(csa_\w+)\s*\(", text)))
    assert names == ["csa_handoff_probe", "csa_mfma_probe", "csa_probe_workgroups", "csa_queue_probe",
                     "csa_read_probe"]
    out = subprocess.run(["nm", "-D", "--defined-only", csa.binding.CALIB_LIB_PATH], capture_output=True, text=True)
    exported = set(re.findall(r" T (\w+)", out.stdout))
    assert set(names) <= exported
    # and they are not part of the CSA library itself
    out = subprocess.run(["nm", "-D", "--defined-only", csa.binding.LIB_PATH], capture_output=True, text=True)
    assert not set(names) & set(re.findall(r" T (\w+)", out.stdout))


def test_probes_reject_bad_args(csa):
    lib, B = csa.binding.calib_lib(), csa.binding
    sink = ctypes.c_void_p(16)  # never dereferenced: every call below fails validation
    assert lib.csa_mfma_probe(None, 1, 1, 0, None) == B.CSA_ERR_INVALID_ARG
    assert lib.csa_mfma_probe(sink, 0, 1, 0, None) == B.CSA_ERR_INVALID_ARG
    assert lib.csa_mfma_probe(sink, 9, 1, 0, None) == B.CSA_ERR_INVALID_ARG
    assert lib.csa_mfma_probe(sink, 1, 0, 0, None) == B.CSA_ERR_INVALID_ARG
    assert lib.csa_mfma_probe(sink, 1, 1, 4, None) == B.CSA_ERR_INVALID_ARG
    assert lib.csa_read_probe(None, 64, None, None) == B.CSA_ERR_INVALID_ARG
    # queue probe: no row, a ring depth it does not build, a misaligned row, no slices to read
    assert lib.csa_queue_probe(None, sink, 1 << 30, 4, sink, 1 << 20, sink, None) == B.CSA_ERR_INVALID_ARG
    assert lib.csa_queue_probe(sink, sink, 1 << 30, 3, sink, 1 << 20, sink, None) == B.CSA_ERR_INVALID_ARG
    assert lib.csa_queue_probe(ctypes.c_void_p(24), sink, 1 << 30, 4, sink, 1 << 20, sink, None) == \
        B.CSA_ERR_INVALID_ARG
    assert lib.csa_queue_probe(sink, None, 0, 4, sink, 1 << 20, sink, None) == B.CSA_ERR_INVALID_ARG
    # hand-off probe: no counter, no workgroups, too few floats for the grid
    assert lib.csa_handoff_probe(sink, 1 << 20, None, sink, 80, 1, None) == B.CSA_ERR_INVALID_ARG
    assert lib.csa_handoff_probe(sink, 1 << 20, sink, sink, 0, 1, None) == B.CSA_ERR_INVALID_ARG
    assert lib.csa_handoff_probe(sink, 255 * 80, sink, sink, 80, 1, None) == B.CSA_ERR_INVALID_ARG


def test_prefill_entry_points_reject_bad_args(csa):
    lib = csa.lib()
    B = csa.binding
    ws = lib.csa_index_topk_workspace_size(2048, 65536, 512)
    # 256 query rows of scores at a time, plus the top-k lists of those rows
    assert ws >= 256 * 65536 * 4
    assert lib.csa_index_topk_workspace_size(16, 65536, 512) < ws
    assert lib.csa_index_topk_workspace_size(0, 65536, 512) == 0
    base = [FAKE, FAKE, FAKE, 2048, 64, 128, 65536, 260096, 4, 512, FAKE, FAKE, FAKE, ws, None]
    a = list(base); a[5] = 64
    assert lib.csa_index_topk(*a) == B.CSA_ERR_UNSUPPORTED
    a = list(base); a[9] = 0
    assert lib.csa_index_topk(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[9] = 2049
    assert lib.csa_index_topk(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[13] = ws - 1
    assert lib.csa_index_topk(*a) == B.CSA_ERR_WORKSPACE
    a = list(base); a[2] = FAKE + 8
    assert lib.csa_index_topk(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[10] = None
    assert lib.csa_index_topk(*a) == B.CSA_ERR_INVALID_ARG
    a = list(base); a[8] = 0
    assert lib.csa_index_topk(*a) == B.CSA_ERR_INVALID_ARG
    # the E4M3 form: one more pointer (the key scales) after k
    b8 = base[:3] + [FAKE] + base[3:]
    a = list(b8); a[6] = 64
    assert lib.csa_index_topk_fp8(*a) == B.CSA_ERR_UNSUPPORTED
    a = list(b8); a[3] = None
    assert lib.csa_index_topk_fp8(*a) == B.CSA_ERR_INVALID_ARG
    a = list(b8); a[14] = ws - 1
    assert lib.csa_index_topk_fp8(*a) == B.CSA_ERR_WORKSPACE
    a = list(b8); a[10] = 2049
    assert lib.csa_index_topk_fp8(*a) == B.CSA_ERR_INVALID_ARG
    attn = [FAKE, FAKE, 65536, FAKE, FAKE, 512, FAKE, 128, 260096, FAKE, 0.04, FAKE, B.CSA_BF16, None,
            2048, 64, 512, None]
    a = list(attn); a[15] = 8                   # heads not a multiple of 16
    assert lib.csa_prefill_attn(*a) == B.CSA_ERR_UNSUPPORTED
    a = list(attn); a[16] = 384                 # unsupported width
    assert lib.csa_prefill_attn(*a) == B.CSA_ERR_UNSUPPORTED
    a = list(attn); a[7] = 0                    # empty window
    assert lib.csa_prefill_attn(*a) == B.CSA_ERR_INVALID_ARG
    a = list(attn); a[8] = -1                   # negative position
    assert lib.csa_prefill_attn(*a) == B.CSA_ERR_INVALID_ARG
    a = list(attn); a[5] = 4096                 # k above the top-k limit
    assert lib.csa_prefill_attn(*a) == B.CSA_ERR_INVALID_ARG
    a = list(attn); a[12] = B.CSA_FP8_E4M3
    assert lib.csa_prefill_attn(*a) == B.CSA_ERR_INVALID_ARG
    a = list(attn); a[6] = FAKE + 2             # misaligned window rows
    assert lib.csa_prefill_attn(*a) == B.CSA_ERR_INVALID_ARG
    a = list(attn); a[3] = None
    assert lib.csa_prefill_attn(*a) == B.CSA_ERR_INVALID_ARG
    # over mixed records: d is 512; the RoPE tables must cover every query position
    mixed = [FAKE, FAKE, 65536, FAKE, FAKE, 512, FAKE, 128, 260096, FAKE, FAKE, 262144, FAKE, 0.04, FAKE,
             B.CSA_BF16, None, 2048, 64, None]
    a = list(mixed); a[11] = 262143             # the last query's row missing
    assert lib.csa_prefill_attn_mixed(*a) == B.CSA_ERR_INVALID_ARG
    assert "RoPE" in csa.csa_last_error()
    a = list(mixed); a[10] = None
    assert lib.csa_prefill_attn_mixed(*a) == B.CSA_ERR_INVALID_ARG
    a = list(mixed); a[18] = 80                 # heads above 64
    assert lib.csa_prefill_attn_mixed(*a) == B.CSA_ERR_UNSUPPORTED
    a = list(mixed); a[1] = FAKE + 8            # misaligned records
    assert lib.csa_prefill_attn_mixed(*a) == B.CSA_ERR_INVALID_ARG
    a = list(mixed); a[7] = 0
    assert lib.csa_prefill_attn_mixed(*a) == B.CSA_ERR_INVALID_ARG


def test_topk_rejects_bad_args_and_sizes_workspace(csa):
    lib = csa.lib()
    B = csa.binding
    need = csa.csa_topk_workspace_size(1, 1, 250000, 512)
    assert need > 0 and need % 256 == 0
    assert csa.csa_topk_workspace_size(8, 1, 250000, 512) > need
    assert csa.csa_topk_workspace_size(1, 1, 0, 0) == 0
    args = [FAKE, 1, 1, 250000, 250000, 0, 512, FAKE, FAKE, FAKE, need, None]
    a = list(args); a[6] = 4096
    assert lib.csa_topk(*a) == B.CSA_ERR_INVALID_ARG
    a = list(args); a[10] = need - 1
    assert lib.csa_topk(*a) == B.CSA_ERR_WORKSPACE
    a = list(args); a[4] = 100
    assert lib.csa_topk(*a) == B.CSA_ERR_INVALID_ARG


def test_gather_rejects_bad_args(csa):
    lib = csa.lib()
    B = csa.binding
    args = [FAKE, 100, FAKE, FAKE, 512, FAKE, 0, 128, 128, FAKE, FAKE, B.CSA_BF16, 1, 512, 0, 0, 0, None]
    a = list(args); a[6] = 128  # head == w
    assert lib.csa_gather(*a) == B.CSA_ERR_INVALID_ARG
    a = list(args); a[7] = 129  # len > w
    assert lib.csa_gather(*a) == B.CSA_ERR_INVALID_ARG
    a = list(args); a[13] = 4  # 8-byte rows
    assert lib.csa_gather(*a) == B.CSA_ERR_INVALID_ARG


def test_attn_rejects_bad_args(csa):
    lib = csa.lib()
    B = csa.binding
    ws = csa.csa_sparse_attn_workspace_size(1, 64, 512, 640)
    assert ws >= 64 * 10 * 514 * 4  # ten 64-row splits of 640 rows
    args = [FAKE, FAKE, FAKE, None, 0.04, FAKE, None, B.CSA_BF16, B.CSA_BF16, 1, 64, 512, 640, 0, 0, 0, FAKE, ws, None]
    a = list(args); a[10] = 60
    assert lib.csa_sparse_attn(*a) == B.CSA_ERR_UNSUPPORTED
    a = list(args); a[17] = ws - 1
    assert lib.csa_sparse_attn(*a) == B.CSA_ERR_WORKSPACE
    a = list(args); a[2] = None
    assert lib.csa_sparse_attn(*a) == B.CSA_ERR_INVALID_ARG


def _desc(csa, **kw):
    L = csa.LayerDesc()
    L.batch, L.h, L.d, L.h_i, L.d_i, L.m, L.w, L.top_k = 1, 64, 512, 64, 128, 4, 128, 512
    L.dtype = L.out_dtype = csa.CSA_BF16
    L.comp_kv = L.idx_keys = L.swa = L.main_bias = L.idx_bias = FAKE
    L.max_comp, L.n_comp, L.swa_head, L.swa_len = 1000, 999, 5, 128
    L.scale = 0.044
    for k, v in kw.items():
        setattr(L, k, v)
    return L


def _io(csa, pos):
    io = csa.StepIO()
    for f, _ in io._fields_:
        if f.endswith("stride_b"):
            continue
        setattr(io, f, FAKE if f != "pos" else pos)
    return io


def test_decode_step_validation_and_advance(csa):
    B = csa.binding
    lib = csa.lib()
    L = _desc(csa)
    need = csa.csa_decode_step_workspace_size(L)
    assert need > csa.csa_topk_workspace_size(1, 1, 1000, 512)
    io = _io(csa, pos=3999)  # completes a block while the cache is full-but-one: fine
    L.n_comp = 1000          # now full
    assert lib.csa_decode_step(ctypes.byref(L), ctypes.byref(io), FAKE, need, None) == B.CSA_ERR_INVALID_ARG
    assert "full" in csa.csa_last_error()
    L.n_comp = 999
    assert lib.csa_decode_step(ctypes.byref(L), ctypes.byref(io), FAKE, need - 1, None) == B.CSA_ERR_WORKSPACE
    L2 = _desc(csa, top_k=4096)
    assert lib.csa_decode_step(ctypes.byref(L2), ctypes.byref(io), FAKE, need, None) == B.CSA_ERR_INVALID_ARG
    # host-side counter advance: block completion and ring wrap
    L3 = _desc(csa, n_comp=10, swa_head=127, swa_len=127)
    csa.csa_layer_advance(L3, 42)   # 42 % 4 != 3
    assert (L3.n_comp, L3.swa_head, L3.swa_len) == (10, 0, 128)
    csa.csa_layer_advance(L3, 43)
    assert (L3.n_comp, L3.swa_head, L3.swa_len) == (11, 1, 128)
    L4 = _desc(csa, n_comp=1000)
    with pytest.raises(csa.CsaError):
        csa.csa_layer_advance(L4, 3)


def test_decode_step_noalloc_rejects_oversize_scratch(csa):
    """The fixed-scratch step refuses layers whose scratch exceeds its array
    (before any device call), and validates like csa_decode_step."""
    B = csa.binding
    lib = csa.lib()
    cap = csa.csa_decode_step_noalloc_max_bytes()
    assert cap == 32 << 20
    io = _io(csa, pos=3999)
    big = _desc(csa, batch=16)
    assert csa.csa_decode_step_workspace_size(big) > cap
    assert lib.csa_decode_step_noalloc(ctypes.byref(big), ctypes.byref(io), None) == B.CSA_ERR_WORKSPACE
    assert "scratch" in csa.csa_last_error()
    assert lib.csa_decode_step_noalloc(None, ctypes.byref(io), None) == B.CSA_ERR_INVALID_ARG


def test_decode_step_fp8_keys_validation(csa):
    """E4M3 indexer keys: bfloat16 caches, 64 x 128 indexer, row scales given."""
    B = csa.binding
    lib = csa.lib()
    L = _desc(csa, idx_dtype=csa.CSA_FP8_E4M3)
    need = csa.csa_decode_step_workspace_size(L)
    io = _io(csa, pos=3999)

    def call(layer):
        return lib.csa_decode_step(ctypes.byref(layer), ctypes.byref(io), FAKE, need, None)

    assert call(L) == B.CSA_ERR_INVALID_ARG      # idx_scales missing
    assert "null" in csa.csa_last_error()
    L.idx_scales = FAKE
    L.h_i = 32
    assert call(L) == B.CSA_ERR_UNSUPPORTED
    L.h_i = 64
    L.dtype = csa.CSA_F32
    assert call(L) == B.CSA_ERR_UNSUPPORTED
    assert "bfloat16" in csa.csa_last_error()
    L.dtype = csa.CSA_BF16
    L.idx_scales_stride_b = -1
    assert call(L) == B.CSA_ERR_INVALID_ARG
    # a zero-filled descriptor keeps keys of the cache dtype
    assert _desc(csa).idx_dtype == csa.CSA_F32 and _desc(csa).idx_scales is None


def test_decode_step_fp4_keys_validation(csa):
    """E2M1 indexer keys: the E4M3 step's rules (bfloat16 caches, a 64 x 128
    indexer, block scales given)."""
    B = csa.binding
    lib = csa.lib()
    L = _desc(csa, idx_dtype=csa.CSA_FP4_E2M1)
    io = _io(csa, pos=3999)

    def call(layer):
        need = csa.csa_decode_step_workspace_size(layer)
        return lib.csa_decode_step(ctypes.byref(layer), ctypes.byref(io), FAKE, need, None)

    assert call(L) == B.CSA_ERR_INVALID_ARG      # idx_scales missing
    L.idx_scales = FAKE
    L.d_i = 64
    assert call(L) == B.CSA_ERR_UNSUPPORTED
    L.d_i = 128
    L.dtype = csa.CSA_F32
    assert call(L) == B.CSA_ERR_UNSUPPORTED
    assert "bfloat16" in csa.csa_last_error()
    L.dtype = csa.CSA_BF16
    L.idx_rescore = L.top_k - 1                  # a first stage smaller than top_k
    assert call(L) == B.CSA_ERR_INVALID_ARG


def test_mixed_kv_validation(csa):
    """Mixed main KV: bfloat16, d = 512, rope_dim = 64, both tables, table
    rows for the position and the block, 16-byte records; the same for the
    HCA step, which also takes no main norm."""
    B = csa.binding
    lib = csa.lib()
    L = _desc(csa, kv_dtype=csa.CSA_FP8_E4M3, rope_dim=64, rope_rows=5000, comp_rope_rows=1000)
    need = csa.csa_decode_step_workspace_size(L)
    io = _io(csa, pos=3999)

    def call(layer):
        return lib.csa_decode_step(ctypes.byref(layer), ctypes.byref(io), FAKE, need, None)

    assert call(L) == B.CSA_ERR_INVALID_ARG      # tables missing
    assert "RoPE" in csa.csa_last_error()
    L.rope_cos = L.rope_sin = L.comp_rope_cos = L.comp_rope_sin = FAKE
    L.rope_rows = 3999                           # the position's row missing
    assert call(L) == B.CSA_ERR_INVALID_ARG
    L.rope_rows = 5000
    L.comp_rope_rows = 999                       # block 999's row missing
    assert call(L) == B.CSA_ERR_INVALID_ARG
    L.comp_rope_rows = 1000
    L.rope_dim = 32
    assert call(L) == B.CSA_ERR_UNSUPPORTED
    L.rope_dim = 64
    L.swa_stride_b = 592 * 128 + 8               # records must stay 16-byte aligned
    assert call(L) == B.CSA_ERR_INVALID_ARG
    L.swa_stride_b = 0
    L.dtype = csa.CSA_F32
    assert call(L) == B.CSA_ERR_UNSUPPORTED
    L.dtype = csa.CSA_BF16
    # the HCA step over mixed records: no main norm, both tables, the position's row
    L.m = 128

    def hca():
        return lib.csa_hca_decode_step(ctypes.byref(L), ctypes.byref(io), FAKE, 1 << 40, None)

    L.main_norm = FAKE
    assert hca() == B.CSA_ERR_UNSUPPORTED
    L.main_norm = None
    L.comp_rope_sin = None
    assert hca() == B.CSA_ERR_INVALID_ARG
    L.comp_rope_sin = FAKE
    L.rope_rows = 3999
    assert hca() == B.CSA_ERR_INVALID_ARG
    L.rope_rows = 5000
    L.comp_kv_stride_b = 592 * 1000 + 4
    assert hca() == B.CSA_ERR_INVALID_ARG
    L.comp_kv_stride_b = 0
    assert lib.csa_pack_kv_mixed(FAKE, csa.CSA_BF16, FAKE, 10, 256, 64, None) == B.CSA_ERR_UNSUPPORTED
    assert lib.csa_pack_kv_mixed(FAKE, csa.CSA_FP8_E4M3, FAKE, 10, 512, 64, None) == B.CSA_ERR_INVALID_ARG
    assert lib.csa_pack_kv_mixed(FAKE + 8, csa.CSA_BF16, FAKE + 8, 10, 512, 64, None) == B.CSA_ERR_INVALID_ARG


def test_dev_step_validation(csa):
    """The device-counter step: state, ring of the stated size, Z/C rows,
    bfloat16 caches and keys; the ring size follows the block rows."""
    B = csa.binding
    lib = csa.lib()
    L = _desc(csa)
    ring = lib.csa_decode_step_dev_ring_size(ctypes.byref(L))
    assert ring == 4 * 1 * 4 * 4 * (512 + 128)  # floats x batch x arrays x 2 blocks x rows x widths
    L.overlap = 1
    assert lib.csa_decode_step_dev_ring_size(ctypes.byref(L)) == 2 * ring
    L.overlap = 0
    need = csa.csa_decode_step_workspace_size(L)
    io = _io(csa, pos=-5)  # ignored: the position is on the device

    def call(layer, state=FAKE, ring_ptr=FAKE, ring_bytes=ring):
        return lib.csa_decode_step_dev(ctypes.byref(layer), ctypes.byref(io), state, ring_ptr, ring_bytes, FAKE,
                                       need, None)

    assert call(L, state=None) == B.CSA_ERR_INVALID_ARG
    assert call(L, ring_bytes=ring - 4) == B.CSA_ERR_INVALID_ARG
    assert call(L, ring_ptr=None) == B.CSA_ERR_INVALID_ARG
    assert call(L, state=FAKE + 4) == B.CSA_ERR_INVALID_ARG
    L2 = _desc(csa, dtype=csa.CSA_F32)
    assert call(L2, ring_bytes=1 << 30) == B.CSA_ERR_UNSUPPORTED
    L3 = _desc(csa, idx_dtype=csa.CSA_FP8_E4M3, idx_scales=FAKE, h_i=32)
    assert call(L3) == B.CSA_ERR_UNSUPPORTED  # E4M3 keys need the 64 x 128 indexer
    io.z_idx = None
    assert call(L) == B.CSA_ERR_INVALID_ARG
    assert "Z/C" in csa.csa_last_error()


def test_hca_step_validation(csa):
    B = csa.binding
    L = B.LayerDesc()
    L.batch, L.h, L.d, L.m, L.w, L.overlap = 1, 64, 512, 128, 128, 0
    L.dtype = L.out_dtype = B.CSA_BF16
    L.comp_kv, L.swa, L.main_bias = FAKE, FAKE, FAKE
    L.max_comp, L.n_comp, L.swa_head, L.swa_len, L.scale = 7813, 7812, 64, 128, 0.04
    io = B.StepIO()
    io.pos, io.q, io.kv_new, io.out, io.z_main, io.c_main = 1000063, FAKE, FAKE, FAKE, FAKE, FAKE
    lib = csa.lib()
    need = lib.csa_hca_decode_step_workspace_size(ctypes.byref(L))
    assert need >= 64 * 63 * 514 * 4  # partials of every 128-row split of 7941 rows
    def call(ws_bytes=need):
        return lib.csa_hca_decode_step(ctypes.byref(L), ctypes.byref(io), FAKE, ws_bytes, None)
    assert call(need - 1) == B.CSA_ERR_WORKSPACE
    L.dtype = B.CSA_F32
    assert call() == B.CSA_ERR_UNSUPPORTED
    L.dtype = B.CSA_BF16
    L.overlap = 1
    assert call() == B.CSA_ERR_INVALID_ARG
    L.overlap = 0
    L.n_comp = 7813  # cache full and the step completes a block
    assert call() == B.CSA_ERR_INVALID_ARG
    L.n_comp = 7812
    io.z_main = None
    assert call() == B.CSA_ERR_INVALID_ARG
    io.z_main = FAKE
    L.max_comp = 9000  # max_comp + w above the attention's row limit
    assert lib.csa_hca_decode_step(ctypes.byref(L), ctypes.byref(io), FAKE, 1 << 40, None) == B.CSA_ERR_UNSUPPORTED


def test_descriptors_keep_their_tensors_alive(csa):
    """make_layer_desc / make_step_io store raw pointers; the returned structs
    must keep the tensors alive, or temporaries passed in would be freed and
    their memory reused before the step runs."""
    import gc
    import weakref

    import torch

    bias = torch.zeros(4, 128)
    ref = weakref.ref(bias)
    L = csa.make_layer_desc(comp_kv=torch.zeros(1, 8, 128), idx_keys=torch.zeros(1, 8, 128),
                            swa=torch.zeros(1, 16, 128), main_bias=torch.zeros(4, 128), idx_bias=bias,
                            sink=torch.zeros(16), n_comp=3, swa_head=0, swa_len=3, h=16, h_i=64, top_k=4)
    del bias
    gc.collect()
    assert ref() is not None and L.idx_bias == ref().data_ptr()
    q = torch.zeros(1, 16, 128)
    rq = weakref.ref(q)
    io = csa.make_step_io(pos=3, q=q, q_idx=torch.zeros(1, 64, 128), w_idx=torch.zeros(1, 64),
                          kv_new=torch.zeros(1, 128), z_main=torch.zeros(1, 4, 128), c_main=torch.zeros(1, 4, 128),
                          z_idx=torch.zeros(1, 4, 128), c_idx=torch.zeros(1, 4, 128), scores=torch.zeros(1, 8),
                          topk_idx=torch.zeros(1, 4, dtype=torch.int32), topk_count=torch.zeros(1, dtype=torch.int32),
                          gather_buf=torch.zeros(1, 20, 128), n_valid=torch.zeros(1, dtype=torch.int32),
                          out=torch.zeros(1, 16, 128))
    del q
    gc.collect()
    assert rq() is not None and io.q == rq().data_ptr()
    del L, io
    gc.collect()
    assert ref() is None and rq() is None
