"""csa_sparse_mqa_noalloc (the allocation-free variant of csa_sparse_mqa) through the C
ABI: two calls in a row, the second with a smaller input, each compared with
csa_sparse_mqa on the same inputs.  Both run the same kernels, so the outputs must be
bitwise equal (stricter than the attention tolerance).  Also: a request above the
scratch limit is rejected on the host."""

import sys

import pytest
import torch

from helpers import ensure_built
from synth import Gen, qstd

pytestmark = pytest.mark.gpu

import compressed_sparse_attention_07_amd as csa  # noqa: E402

DEV = "cuda"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(seed, B, H, D, N, K, W, kvf):
    g = Gen(seed, DEV)
    q = g.normal((B, 1, H, D), qstd(D), dtype=torch.bfloat16)
    pos = torch.full((B, 1), 4 * N, dtype=torch.int64, device=DEV)
    kv32 = g.normal((B, N, D))
    win32 = g.normal((B, W, D))
    if kvf == "fp8mix":
        kv = csa.Buf.empty((B, N, D), csa.CSA_FP8MIX, rope_dims=64)
        win = csa.Buf.empty((B, W, D), csa.CSA_FP8MIX, rope_dims=64)
        csa.csa_quantize(kv32, kv, rope_dims=64)
        csa.csa_quantize(win32, win, rope_dims=64)
    else:
        kv, win = kv32.to(torch.bfloat16), win32.to(torch.bfloat16)
    r = torch.rand((B, 1, N), generator=g.g, device=DEV)
    idx = torch.sort(torch.argsort(r, dim=-1)[..., :K].to(torch.int32), dim=-1).values.contiguous()
    wp0 = torch.full((B,), 4 * N - W + 1, dtype=torch.int64, device=DEV)
    sink = g.normal((H,))
    return q, pos, kv, idx, win, wp0, sink


def test_noalloc_matches_workspace_entry_point_twice():
    ensure_built()
    assert csa.lib().csa_device_check() == 0, csa.lib().csa_last_error()
    say(f"scratch limit {csa.lib().csa_sparse_mqa_noalloc_limit()} bytes")
    # the 128K decode shape, then a smaller one (fewer sequences, shorter selection,
    # FP8MIX cache), so the second call reuses the array the first one filled
    for seed, B, H, D, N, K, W, kvf in ((5, 16, 128, 512, 32768, 1024, 128, "bf16"),
                                        (6, 3, 64, 512, 4096, 200, 128, "fp8mix")):
        say(f"noalloc vs workspace: B={B} H={H} N={N} K={K} {kvf}")
        q, pos, kv, idx, win, wp0, sink = _case(seed, B, H, D, N, K, W, kvf)
        assert csa.lib().csa_sparse_mqa_workspace_size(B, 1, H, D, K, W) <= csa.lib().csa_sparse_mqa_noalloc_limit()
        o_ws = torch.empty_like(q)
        o_na = torch.full_like(q, float("nan"))
        kw = dict(N=N, n_win=W, softmax_scale=1.0, rope_dims=64)
        csa.csa_sparse_mqa(q, pos, kv, idx, win, wp0, sink, o_ws, **kw)
        csa.csa_sparse_mqa_noalloc(q, pos, kv, idx, win, wp0, sink, o_na, **kw)
        torch.cuda.synchronize()
        assert torch.equal(o_ws.view(torch.int16), o_na.view(torch.int16)), "outputs differ"


def test_noalloc_rejects_requests_above_the_limit():
    ensure_built()
    # 64 sequences x 4 query tokens x 128 heads x 12 splits of 1 KiB partials > 32 MiB
    B, Tq, H, D, N, K, W = 64, 4, 128, 512, 64, 1024, 128
    need = csa.lib().csa_sparse_mqa_workspace_size(B, Tq, H, D, K, W)
    assert need > csa.lib().csa_sparse_mqa_noalloc_limit()
    q = torch.zeros((B, Tq, H, D), dtype=torch.bfloat16, device=DEV)
    pos = torch.full((B, Tq), 4 * N, dtype=torch.int64, device=DEV)
    kv = torch.zeros((B, N, D), dtype=torch.bfloat16, device=DEV)
    idx = torch.zeros((B, Tq, K), dtype=torch.int32, device=DEV)
    win = torch.zeros((B, W, D), dtype=torch.bfloat16, device=DEV)
    wp0 = torch.full((B,), 4 * N - W + 1, dtype=torch.int64, device=DEV)
    sink = torch.zeros((H,), device=DEV)
    out = torch.empty_like(q)
    with pytest.raises(csa.CSAError) as e:
        csa.csa_sparse_mqa_noalloc(q, pos, kv, idx, win, wp0, sink, out, N=N, n_win=W, softmax_scale=1.0, rope_dims=64)
    assert e.value.status == 6
