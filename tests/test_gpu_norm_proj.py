"""GPU parity of the steps either side of core attention: RMSNorm (standalone and
fused into the compressor before RoPE) and the grouped output projection, against
the oracle on the same seeded inputs."""

import sys

import numpy as np
import pytest
import torch

from helpers import assert_close, ensure_built, f64
from oracle import csa_oracle as O
from synth import Gen

pytestmark = pytest.mark.gpu

import compressed_sparse_attention_07_amd as csa  # noqa: E402

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype,rows,D", [("f32", 37, 128), ("bf16", 37, 512), ("bf16", 1, 2048), ("f32", 300, 8),
                                          ("bf16", 0, 512)])
def test_rmsnorm(dtype, rows, D):
    say(f"rmsnorm {dtype} rows={rows} D={D}")
    g = Gen(31 + rows + D, DEV)
    td = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    x = g.normal((max(rows, 1), D), 3.0, dtype=td)[:rows]
    w = g.uniform((D,), 0.5, 1.5)
    y = torch.empty_like(x)
    csa.csa_rmsnorm(x, w, y, eps=1e-6)
    torch.cuda.synchronize()
    if rows == 0:
        return
    want = O.store(O.rmsnorm(f64(x), f64(w), 1e-6), dtype)
    assert_close(f64(y), want, dtype, "rmsnorm")


def test_rmsnorm_in_place_and_zero_rows():
    # y may alias x; an all-zero row stays zero (eps keeps the scale finite)
    g = Gen(77, DEV)
    x = g.normal((8, 256), dtype=torch.bfloat16)
    x[3] = 0
    ref = O.store(O.rmsnorm(f64(x), np.ones(256), 1e-6), "bf16")
    w = torch.ones(256, dtype=torch.float32, device=DEV)
    csa.csa_rmsnorm(x, w, x, eps=1e-6)
    torch.cuda.synchronize()
    assert_close(f64(x), ref, "bf16", "in-place rmsnorm")
    assert torch.all(x[3] == 0)


COMPRESS_NORM_CASES = [
    # (overlap, ratio, D, R, dtype, B, T)
    (True, 4, 512, 64, "bf16", 2, 64),     # CSA at the pages' width: small path
    (True, 4, 128, 64, "f32", 1, 96),
    (False, 128, 512, 64, "bf16", 1, 512),  # HCA: row-group path
    (True, 6, 64, 16, "f32", 1, 48),        # general path (online softmax)
]


@pytest.mark.parametrize("overlap,ratio,D,R,dtype,B,T", COMPRESS_NORM_CASES)
def test_compress_with_norm(overlap, ratio, D, R, dtype, B, T):
    say(f"compress+norm overlap={overlap} ratio={ratio} D={D} {dtype}")
    g = Gen(500 + ratio + D, DEV)
    td = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    st = [g.normal((B, T, D), dtype=td) for _ in range(4)]
    ba, bb = g.normal((ratio, D), 0.5), g.normal((ratio, D), 0.5)
    w = g.uniform((D,), 0.5, 1.5)
    N = T // ratio
    out = csa.Buf.empty((B, N, D), csa.CSA_F32 if dtype == "f32" else csa.CSA_BF16)
    cb, zb = (st[1], st[3]) if overlap else (None, None)
    csa.csa_compress_norm(st[0], cb, st[2], zb, out, ratio=ratio, overlap=overlap, norm_weight=w, norm_eps=1e-6,
                          bias_a=ba, bias_b=bb if overlap else None, rope_dims=R, rope_base=10000.0, pos_offset=3)
    torch.cuda.synchronize()
    for b in range(B):
        want = O.compress(f64(st[0][b]), f64(st[1][b]) if overlap else None, f64(st[2][b]),
                          f64(st[3][b]) if overlap else None, ratio=ratio, overlap=overlap, bias_a=f64(ba),
                          bias_b=f64(bb) if overlap else None, rope_dims=R, rope_base=10000.0, pos_offset=3,
                          norm_weight=f64(w), norm_eps=1e-6)
        assert_close(f64(out.data[b]), O.store(want, dtype), dtype, f"normalized entries of sequence {b}")


def _proj_case(seed, T, n_h, c, g_, d_g, d):
    g = Gen(seed, DEV)
    o = g.normal((T, n_h, c), dtype=torch.bfloat16)
    k1 = (n_h // g_) * c
    wg = g.normal((g_, d_g, k1), k1 ** -0.5, dtype=torch.bfloat16)
    wo = g.normal((d, g_ * d_g), (g_ * d_g) ** -0.5, dtype=torch.bfloat16)
    return o, wg, wo


# With an fp32 output the two sides differ only where the fp32 and fp64 intermediate
# sums round to neighbouring bf16 values (mid is stored in bf16 on both sides): a
# fraction ~1e-3 of the intermediates, each moving one term of the second product by
# 2^-8 relative.  Terms are independent with rms(out) ~ sqrt(K2) * rms(term), so the
# resulting error stays below 1e-3 of rms(out); the fp32 accumulation itself adds
# ~1e-6.  bf16 outputs take the usual bf16 tolerance.
PROJ_F32_TOL = dict(rtol=1e-3, atol_rms=1e-3)


def _check_proj(got, o, wg, wo, rows, dtype, what):
    want = O.grouped_out_proj(f64(o[rows]), f64(wg), f64(wo), dtype="bf16")
    got = f64(got[rows])
    if dtype == "bf16":
        assert_close(got, O.store(want, "bf16"), "bf16", what)
        return
    rms = np.sqrt(np.mean(want ** 2))
    err = np.abs(got - want)
    bad = err > PROJ_F32_TOL["atol_rms"] * rms + PROJ_F32_TOL["rtol"] * np.abs(want)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside; worst {err.max()} (rms {rms})"


@pytest.mark.parametrize("T,n_h,c,g_,d_g,d,dtype", [
    (5, 8, 64, 4, 96, 200, "f32"),       # ragged rows and columns, contraction split
    (70, 8, 64, 2, 64, 130, "bf16"),     # 64 x 64 tiles with a ragged edge
    (33, 4, 128, 4, 32, 96, "f32"),      # one row past the few-rows tiles
    (1, 16, 32, 16, 32, 64, "bf16"),     # single token, one head per group
    (300, 8, 64, 2, 96, 300, "f32"),     # LDS-tiled blocks: ragged rows and columns
    (256, 4, 128, 4, 256, 512, "bf16"),  # LDS-tiled blocks, exact tiles
    (0, 8, 64, 4, 96, 200, "f32"),       # no rows
])
def test_grouped_out_proj_small(T, n_h, c, g_, d_g, d, dtype):
    say(f"grouped projection T={T} n_h={n_h} c={c} g={g_} d_g={d_g} d={d} {dtype}")
    o, wg, wo = _proj_case(900 + T, T, n_h, c, g_, d_g, d)
    out = torch.empty((T, d), dtype=torch.float32 if dtype == "f32" else torch.bfloat16, device=DEV)
    csa.csa_grouped_out_proj(o, wg, wo, out)
    torch.cuda.synchronize()
    if T:
        _check_proj(out, o, wg, wo, np.arange(T), dtype, "grouped projection")


@pytest.mark.parametrize("T", [16, 512])
def test_grouped_out_proj_pro_shape(T):
    # n_h = 128 heads of c = 512, g = 16 groups of d_g = 1024, d = 7168 (the pages'
    # large model); decode (T = 16: every row checked) and a prefill chunk (sampled rows)
    say(f"grouped projection at the large-model shape, T={T}")
    n_h, c, g_, d_g, d = 128, 512, 16, 1024, 7168
    o, wg, wo = _proj_case(4242 + T, T, n_h, c, g_, d_g, d)
    out = torch.empty((T, d), dtype=torch.float32, device=DEV)
    csa.csa_grouped_out_proj(o, wg, wo, out)
    torch.cuda.synchronize()
    rows = np.arange(T) if T <= 16 else np.array([0, 1, 63, 64, 200, 255, 256, 400, T - 2, T - 1])
    _check_proj(out, o, wg, wo, rows, "f32", "grouped projection (large model)")
