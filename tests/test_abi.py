"""CPU-side checks of the C ABI: the library loads, exports every declared symbol,
and rejects bad arguments on the host (before any device work); with no GPU the
device check fails cleanly.  No compute call is made."""

import ctypes as C
import os
import re

import pytest

from helpers import ROOT, ensure_built


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "csa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(csa_\w+|hca_\w+)\s*\(", text)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    return ensure_built()


def test_every_declared_symbol_is_exported(L):
    from compressed_sparse_attention_07_amd import EXPORTS
    declared = _declared_symbols()
    assert set(declared) == set(EXPORTS), (declared, EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_abi_version(L):
    assert L.csa_abi_version() == 4


def test_struct_layouts_match_the_header(tmp_path):
    """The ctypes mirrors of csa_layer_desc / csa_forward_io have the C sizes and
    field offsets (the header compiled by the host C compiler)."""
    import shutil
    import subprocess
    from compressed_sparse_attention_07_amd._lib import (csa_decode_desc, csa_decode_io, csa_forward_io,
                                                         csa_layer_desc)
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    fields = {"csa_layer_desc": csa_layer_desc, "csa_forward_io": csa_forward_io, "csa_decode_desc": csa_decode_desc,
              "csa_decode_io": csa_decode_io}
    lines = ["#include <stddef.h>", "#include <stdio.h>", '#include "csa.h"', "int main(void) {"]
    for sname, cls in fields.items():
        lines.append(f'  printf("{sname} %zu\\n", sizeof({sname}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{sname}.{f} %zu\\n", offsetof({sname}, {f}));')
    lines.append("  return 0;\n}")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = str(tmp_path / "layout")
    subprocess.run([cc, "-I" + os.path.join(ROOT, "include"), str(src), "-o", exe], check=True)
    got = dict(line.split() for line in subprocess.run([exe], capture_output=True, text=True, check=True)
               .stdout.splitlines())
    for sname, cls in fields.items():
        assert int(got[sname]) == C.sizeof(cls), sname
        for f, _ in cls._fields_:
            assert int(got[f"{sname}.{f}"]) == getattr(cls, f).offset, (sname, f)


def _buf(dtype=1, data=0x100000):
    from compressed_sparse_attention_07_amd._lib import csa_buf
    return csa_buf(data, 0, 0, dtype, 0)


def test_compress_rejects_bad_arguments(L):
    out = _buf()
    p = 0x100000
    # NULL input
    st = L.csa_compress(None, p, p, p, 1, None, None, None, None, 1, 8, 16, 4, 1, 0, 0, 10000.0, 0, C.byref(out), 2, None)
    assert st == 1 and b"required" in L.csa_last_error()
    # T not a multiple of ratio
    st = L.csa_compress(p, p, p, p, 1, None, None, None, None, 1, 9, 16, 4, 1, 0, 0, 10000.0, 0, C.byref(out), 3, None)
    assert st == 2
    # odd rope dims
    st = L.csa_compress(p, p, p, p, 1, None, None, None, None, 1, 8, 16, 4, 1, 0, 3, 10000.0, 0, C.byref(out), 2, None)
    assert st == 2
    # more than 128 RoPE dims (D = 512, R = 256)
    st = L.csa_compress(p, p, p, p, 1, None, None, None, None, 1, 8, 512, 4, 1, 0, 256, 10000.0, 0, C.byref(out), 2,
                        None)
    assert st == 6 and b"128" in L.csa_last_error()
    # t0 > 0 without the previous block
    st = L.csa_compress(p, p, p, p, 1, None, None, None, None, 1, 8, 16, 4, 1, 4, 0, 10000.0, 0, C.byref(out), 3, None)
    assert st == 1
    # unsupported input dtype
    st = L.csa_compress(p, p, p, p, 2, None, None, None, None, 1, 8, 16, 4, 1, 0, 0, 10000.0, 0, C.byref(out), 2, None)
    assert st == 3
    # output too short
    st = L.csa_compress(p, p, p, p, 1, None, None, None, None, 1, 8, 16, 4, 1, 0, 0, 10000.0, 0, C.byref(out), 1, None)
    assert st == 2
    # misaligned pointer
    st = L.csa_compress(p + 2, p, p, p, 1, None, None, None, None, 1, 8, 16, 4, 1, 0, 0, 10000.0, 0, C.byref(out), 2, None)
    assert st == 2
    # MXFP4 output needs D % 32 == 0 and a scale pointer
    mx = _buf(3)
    st = L.csa_compress(p, p, p, p, 1, None, None, None, None, 1, 8, 16, 4, 1, 0, 0, 10000.0, 0, C.byref(mx), 2, None)
    assert st == 1


def test_norm_and_projection_reject_bad_arguments(L):
    p = 0x100000
    x, out = _buf(), _buf()
    # RMSNorm: no weight, D not a multiple of 8, mixed dtypes, negative eps
    assert L.csa_rmsnorm(C.byref(x), 4, 512, None, C.c_float(1e-6), C.byref(out), None) == 1
    assert L.csa_rmsnorm(C.byref(x), 4, 500, p, C.c_float(1e-6), C.byref(out), None) == 2
    assert L.csa_rmsnorm(C.byref(x), 4, 4096, p, C.c_float(1e-6), C.byref(out), None) == 2
    f32 = _buf(0)
    assert L.csa_rmsnorm(C.byref(x), 4, 512, p, C.c_float(1e-6), C.byref(f32), None) == 3
    assert L.csa_rmsnorm(C.byref(x), 4, 512, p, C.c_float(-1.0), C.byref(out), None) == 2
    # compress with a norm weight: misaligned weight, bad eps
    st = L.csa_compress_norm(p, p, p, p, 1, None, None, None, None, 1, 8, 16, 4, 1, 0, 0, 10000.0, 0, p + 4,
                             C.c_float(1e-6), C.byref(out), 2, None)
    assert st == 2
    st = L.csa_compress_norm(p, p, p, p, 1, None, None, None, None, 1, 8, 16, 4, 1, 0, 0, 10000.0, 0, p,
                             C.c_float(float("nan")), C.byref(out), 2, None)
    assert st == 2
    # grouped projection: g not dividing n_h, contraction not a multiple of 32, f32 input,
    # missing workspace
    o = _buf()
    assert L.csa_grouped_out_proj(C.byref(o), p, p, 16, 128, 512, 12, 1024, 7168, C.byref(out), p, 1 << 30, None) == 2
    assert L.csa_grouped_out_proj(C.byref(o), p, p, 16, 4, 12, 4, 1024, 7168, C.byref(out), p, 1 << 30, None) == 6
    assert L.csa_grouped_out_proj(C.byref(f32), p, p, 16, 128, 512, 16, 1024, 7168, C.byref(out), p, 1 << 30,
                                  None) == 3
    assert L.csa_grouped_out_proj(C.byref(o), p, p, 16, 128, 512, 16, 1024, 7168, C.byref(out), None, 0, None) == 4
    # sizes: mid (bf16) plus fp32 split partials for few rows; none for T = 0
    assert L.csa_grouped_out_proj_workspace_size(0, 128, 512, 16, 1024, 7168) == 0
    assert L.csa_grouped_out_proj_workspace_size(16, 128, 512, 16, 1024, 7168) >= 16 * 16 * 1024 * 2
    assert L.csa_grouped_out_proj_workspace_size(16, 128, 512, 12, 1024, 7168) == 0


def test_forward_norm_flag_needs_weights(L):
    from compressed_sparse_attention_07_amd import CSA_FLAG_QKV_NORM, layer_desc
    from compressed_sparse_attention_07_amd._lib import csa_forward_io
    d = layer_desc(mode=0, B=16, T=0, t0=4096, Tq=1, cache_rows=1024, Tw=128, D=512, H=128, HI=64, DI=128, ratio=4,
                   topk=512, n_win=128, rope_dims=64, rope_base=10000.0, softmax_scale=1.0, stream_dtype=1,
                   flags=CSA_FLAG_QKV_NORM, norm_eps=1e-6)
    plain = layer_desc(mode=0, B=16, T=0, t0=4096, Tq=1, cache_rows=1024, Tw=128, D=512, H=128, HI=64, DI=128,
                       ratio=4, topk=512, n_win=128, rope_dims=64, rope_base=10000.0, softmax_scale=1.0,
                       stream_dtype=1)
    # the normalized query and window copies live in the workspace
    assert L.csa_forward_workspace_size(C.byref(d)) >= L.csa_forward_workspace_size(C.byref(plain)) + 16 * 128 * 512 * 2
    d.norm_eps = float("inf")
    assert L.csa_forward_workspace_size(C.byref(d)) == 0
    d.norm_eps = 1e-6
    d.reserved = 1
    assert L.csa_forward_workspace_size(C.byref(d)) == 0
    d.reserved = 0
    io = csa_forward_io()
    assert L.csa_forward(C.byref(d), C.byref(io), None, 0, None) != 0


def _decode_desc(**over):
    from compressed_sparse_attention_07_amd import decode_desc
    kw = dict(mode=0, B=16, slots=16, pages=1100, max_pages=64, page_tokens=2048, D=512, H=128, HI=64, DI=128,
              ratio=4, topk=1024, n_win=128, rope_dims=64, rope_base=10000.0, softmax_scale=0.044, stream_dtype=1)
    kw.update(over)
    return decode_desc(**kw)


def test_decode_step_rejects_bad_descriptors(L):
    """Page size rules (a power of two, a multiple of the ratio; CSA pages of at least
    512 entries so an indexer key range stays in one page), shape limits and the struct
    size: rejected by the size query (0) and the call."""
    from compressed_sparse_attention_07_amd._lib import csa_decode_io
    assert L.csa_decode_step_workspace_size(C.byref(_decode_desc())) > 0
    assert L.csa_decode_step_workspace_size(C.byref(_decode_desc(mode=1, ratio=128, page_tokens=4096))) > 0
    bad = [dict(page_tokens=3072), dict(page_tokens=1024), dict(page_tokens=2), dict(DI=1024),
           dict(B=17), dict(max_pages=0), dict(ratio=0), dict(topk=0), dict(n_win=0), dict(flags=8),
           dict(reserved=1), dict(D=2048)]
    io = csa_decode_io()
    for over in bad:
        d = _decode_desc(**over)
        assert L.csa_decode_step_workspace_size(C.byref(d)) == 0, over
        assert L.csa_decode_step(C.byref(d), C.byref(io), None, 0, None) != 0, over
    d = _decode_desc()
    d.struct_size = 8
    assert L.csa_decode_step(C.byref(d), C.byref(io), None, 0, None) == 2
    # a valid descriptor with empty io: a missing pointer is reported, nothing launched
    assert L.csa_decode_step(C.byref(_decode_desc()), C.byref(io), None, 0, None) == 1
    # no sequences: nothing to do
    assert L.csa_decode_step(C.byref(_decode_desc(B=0)), C.byref(io), None, 0, None) == 0


def test_decode_workspace_grows_with_norms_and_scales_with_batch(L):
    from compressed_sparse_attention_07_amd import CSA_FLAG_QKV_NORM
    a = L.csa_decode_step_workspace_size(C.byref(_decode_desc(B=1)))
    b = L.csa_decode_step_workspace_size(C.byref(_decode_desc(B=16)))
    n = L.csa_decode_step_workspace_size(C.byref(_decode_desc(B=16, flags=CSA_FLAG_QKV_NORM, norm_eps=1e-6)))
    assert 0 < a < b < n
    # HCA uses every visible entry: the index list spans the whole block table
    h = L.csa_decode_step_workspace_size(C.byref(_decode_desc(mode=1, ratio=128, page_tokens=4096, max_pages=256)))
    assert h >= 16 * 256 * 32 * 4


def test_topk_and_index_reject_bad_arguments(L):
    p = 0x100000
    assert L.csa_topk(None, 1, 10, 4, p, None, None, 0, None) == 1
    assert L.csa_topk(p, 1, 10, 0, p, None, None, 0, None) == 2
    assert L.csa_topk(p, 1, 10, 5000, p, None, None, 0, None) == 2
    q, k = _buf(1), _buf(0)
    st = L.csa_index_scores(C.byref(q), p, C.byref(k), p, 1, 1, 4, 32, 8, 8, 4, p, None)
    assert st == 3  # dtype mismatch
    k = _buf(1)
    st = L.csa_index_scores(C.byref(q), p, C.byref(k), p, 1, 1, 4, 30, 8, 8, 4, p, None)
    assert st == 2  # DI not a multiple of 8
    st = L.csa_index_scores(C.byref(q), p, C.byref(k), p, 1, 1, 4, 32, 8, 4, 4, p, None)
    assert st == 2  # kI_rows < N


def test_attention_rejects_bad_arguments(L):
    p = 0x100000
    q, kv, win, out = _buf(1), _buf(1), _buf(1), _buf(1)
    args = lambda **o: dict(dict(K=4, n_win=8, H=16, D=128, N=10, kv_rows=10, Tw=16, out=out), **o)
    def call(**o):
        a = args(**o)
        return L.csa_sparse_mqa(C.byref(q), p, C.byref(kv), a["kv_rows"], p, a["K"], C.byref(win), p, a["Tw"], p,
                                1.0, 64, 10000.0, 0, 1, 1, a["H"], a["D"], a["N"], a["n_win"], C.byref(a["out"]),
                                None, 0, None)
    assert call(n_win=0) == 2
    assert call(kv_rows=5) == 2
    assert call(D=1030) == 2
    assert call(out=_buf(0)) == 3          # out dtype differs from q
    fp8 = _buf(2)                           # FP8MIX without a scale pointer
    assert L.csa_sparse_mqa(C.byref(q), p, C.byref(fp8), 10, p, 4, C.byref(win), p, 16, p, 1.0, 64, 10000.0, 0, 1,
                            1, 16, 128, 10, 8, C.byref(out), None, 0, None) == 1


def test_fp8_queries_are_fenced(L):
    # FP8MIX queries run only on the fp8-product attention kernel: an FP8MIX cache,
    # D = 512 with 64 RoPE dims, 64 / 128 / 256 heads, a BF16 output (every other
    # combination is rejected before any launch)
    p = 0x100000
    def fp8buf():
        b = _buf(2)
        b.rope, b.scale = p, p
        return b
    q8, kv8, win8 = fp8buf(), fp8buf(), fp8buf()
    def call(q=q8, kv=kv8, win=win8, out=None, H=128, D=512, R=64):
        out = out if out is not None else _buf(1)
        return L.csa_sparse_mqa(C.byref(q), p, C.byref(kv), 10, p, 4, C.byref(win), p, 16, p, 1.0, R, 10000.0, 0, 1,
                                1, H, D, 10, 8, C.byref(out), None, 0, None)
    assert call(kv=_buf(1), win=_buf(1)) == 6   # bf16 cache
    assert call(D=256) == 6
    assert call(R=32) == 6
    assert call(H=96) == 6
    assert call(out=_buf(0)) == 3              # F32 output
    q_norope = fp8buf()
    q_norope.rope = None
    assert call(q=q_norope) == 1
    import torch
    if not torch.cuda.is_available():
        assert call() == 5                      # valid: fails only for want of a GPU


def test_forward_rejects_bad_descriptor(L):
    from compressed_sparse_attention_07_amd._lib import csa_forward_io, csa_layer_desc
    d = csa_layer_desc()
    d.struct_size = 12
    io = csa_forward_io()
    assert L.csa_forward(C.byref(d), C.byref(io), None, 0, None) == 2
    assert L.csa_forward_workspace_size(C.byref(d)) == 0


def test_valid_call_without_gpu_reports_device_error(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert L.csa_device_check() == 5
    p = 0x100000
    out = _buf()
    st = L.csa_compress(p, p, p, p, 1, None, None, None, None, 1, 8, 16, 4, 1, 0, 0, 10000.0, 0, C.byref(out), 2, None)
    assert st == 5 and L.csa_last_error()


def test_workspace_sizes_with_no_query_tokens(L):
    """Sizes are host arithmetic: zero query tokens (a compress-only forward) need no
    attention workspace and must not divide by zero."""
    from compressed_sparse_attention_07_amd import layer_desc
    assert L.csa_sparse_mqa_workspace_size(16, 0, 128, 512, 1024, 128) == 0
    assert L.csa_sparse_mqa_workspace_size(0, 1, 128, 512, 1024, 128) == 0
    assert L.hca_dense_attn_workspace_size(1, 0, 128, 512, 8192, 128) == 0
    assert L.csa_topk_workspace_size(0, 32768, 1024) == 0
    d = layer_desc(mode=0, B=16, T=4, t0=131068, Tq=0, cache_rows=32768, Tw=128, D=512, H=128, HI=64, DI=128, ratio=4,
                   topk=1024, n_win=128, rope_dims=64, rope_base=10000.0, softmax_scale=0.044, stream_dtype=1)
    assert L.csa_forward_workspace_size(C.byref(d)) >= 0
    d.Tq = 1
    assert L.csa_forward_workspace_size(C.byref(d)) > 0


@pytest.mark.parametrize("H,D", [(80, 512), (72, 512), (112, 512), (144, 128), (176, 128), (200, 128),
                                 (48, 256), (240, 512), (17, 64)])
def test_head_counts_without_an_mfma_head_group(L, H, D):
    """Head counts the MFMA kernels cannot split into instantiated head groups take the
    SIMT kernel: every size query answers (0 bytes: that kernel needs no workspace)
    and a forward call returns a status instead of failing inside the planner."""
    from compressed_sparse_attention_07_amd import layer_desc
    from compressed_sparse_attention_07_amd._lib import csa_forward_io
    assert L.csa_sparse_mqa_workspace_size(16, 1, H, D, 1024, 128) >= 0
    assert L.hca_dense_attn_workspace_size(32, 1, H, D, 8192, 128) >= 0
    for mode in (0, 1):
        d = layer_desc(mode=mode, B=16, T=0, t0=4096, Tq=1, cache_rows=1024 if mode == 0 else 32, Tw=128, D=D, H=H,
                       HI=64, DI=128, ratio=4 if mode == 0 else 128, topk=512, n_win=128, rope_dims=64 if D >= 64
                       else 0, rope_base=10000.0, softmax_scale=1.0, stream_dtype=1)
        assert L.csa_forward_workspace_size(C.byref(d)) >= 0
        io = csa_forward_io()
        assert L.csa_forward(C.byref(d), C.byref(io), None, 0, None) != 0
