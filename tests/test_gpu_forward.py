"""End-to-end csa_forward parity (compress -> indexer -> top-k -> sparse MQA, and
the HCA chain) against the oracle's whole-layer functions.

The oracle runs its own pipeline from the same inputs.  Top-k sets must agree
except for entries whose oracle score lies within the near-tie band of the k-th
score: 1e-4 relative in fp32; in bf16 the band also covers the largest score
change one bf16 rounding step of a compressed key can cause (2^-8 relative per key
element, summed with the head weights).  Outputs are compared on every query
whose selected set is identical.
"""

import sys

import numpy as np
import pytest
import torch

from helpers import assert_close, ensure_built, f64, topk_sets_agree
from oracle import csa_oracle as O
from synth import CONFIGS, Gen, qstd

pytestmark = pytest.mark.gpu

import compressed_sparse_attention_07_amd as csa  # noqa: E402

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _csa_case(g, B, T, D, DI, H, HI, Tq, dtype):
    td = {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    streams = [g.normal((B, T, D), dtype=td) for _ in range(4)]
    istreams = [g.normal((B, T, DI), dtype=td) for _ in range(4)]
    q = g.normal((B, Tq, H, D), qstd(D), dtype=td)
    qI = g.normal((B, Tq, HI, DI), qstd(DI), dtype=td)
    wI = g.uniform((B, Tq, HI))
    win = g.normal((B, T, D), dtype=td)
    sink = g.normal((H,))
    return streams, istreams, q, qI, wI, win, sink


def _run_forward(dtype, B, T, D, DI, H, HI, Tq, k, ratio, n_win, R, scale, seed):
    g = Gen(seed, DEV)
    streams, istreams, q, qI, wI, win, sink = _csa_case(g, B, T, D, DI, H, HI, Tq, dtype)
    N = T // ratio
    dt = csa.CSA_F32 if dtype == "f32" else csa.CSA_BF16
    kv = csa.Buf.empty((B, N, D), dt)
    ik = csa.Buf.empty((B, N, DI), dt)
    pos = torch.arange(T - Tq, T, dtype=torch.int64, device=DEV).expand(B, Tq).contiguous()
    win_pos0 = torch.zeros((B,), dtype=torch.int64, device=DEV)
    out = torch.empty_like(q)
    scores = torch.empty((B, Tq, N), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device=DEV)
    desc = csa.layer_desc(mode=csa.CSA_MODE_CSA, B=B, T=T, t0=0, Tq=Tq, cache_rows=N, Tw=T, D=D, H=H, HI=HI, DI=DI,
                          ratio=ratio, topk=k, n_win=n_win, rope_dims=R, rope_base=10000.0, softmax_scale=scale,
                          pos_offset=0, stream_dtype=dt)
    io = dict(ca=streams[0], cb=streams[1], za=streams[2], zb=streams[3], ica=istreams[0], icb=istreams[1],
              iza=istreams[2], izb=istreams[3], kv_cache=kv, ik_cache=ik, q=q, q_pos=pos, qI=qI, wI=wI, win=win,
              win_pos0=win_pos0, sink=sink, out=out, scores_out=scores, idx_out=idx)
    csa.csa_forward(desc, io)
    torch.cuda.synchronize()
    return dict(streams=streams, istreams=istreams, q=q, qI=qI, wI=wI, win=win, sink=sink, pos=pos, kv=kv, ik=ik,
                out=out, scores=scores, idx=idx)


def _check_layer(r, b, dtype, k, ratio, n_win, R, scale, band_fn=None):
    want = O.csa_layer([f64(s[b]) for s in r["streams"]], [f64(s[b]) for s in r["istreams"]], f64(r["q"][b]),
                       r["pos"][b].cpu().numpy(), f64(r["qI"][b]), f64(r["wI"][b]), f64(r["win"][b]), 0,
                       f64(r["sink"]), ratio=ratio, k=k, n_win=n_win, scale=scale, rope_dims=R, rope_base=10000.0,
                       dtype=dtype)
    kind = "f32" if dtype == "f32" else "bf16"
    assert_close(f64(r["kv"].data[b]), want["kv"], kind, "compressed KV")
    assert_close(f64(r["ik"].data[b]), want["ik"], kind, "compressed indexer keys")
    gs = r["scores"][b].cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(gs), np.isneginf(want["scores"]))
    fin = np.isfinite(want["scores"])
    if dtype == "f32":
        assert_close(gs[fin], want["scores"][fin], "f32", "scores")
    gi = r["idx"][b].cpu().numpy()
    exact_rows = []
    for t in range(gi.shape[0]):
        cnt = int((gi[t] >= 0).sum())
        band_abs = band_fn(b, t) if band_fn else None
        ok, exact = topk_sets_agree(gi[t], cnt, want["scores"][t], k, band_abs=band_abs)
        assert ok, f"top-k set of query {t} differs beyond the near-tie band"
        if exact:
            exact_rows.append(t)
    assert len(exact_rows) >= 0.9 * gi.shape[0], len(exact_rows)
    rows = np.array(exact_rows)
    assert_close(f64(r["out"][b])[rows], want["out"][rows], kind, "output")


def test_forward_config0_fp32_full():
    c = CONFIGS[0]
    say("forward config 0 (fp32, T=1024, every query)")
    r = _run_forward("f32", c.B, c.ctx, c.D, c.DI, c.H, c.HI, c.Tq, c.k, c.m, c.n_win, c.R, c.softmax_scale, c.seed)
    _check_layer(r, 0, "f32", c.k, c.m, c.n_win, c.R, c.softmax_scale)


def test_forward_bf16_mfma_paths():
    say("forward bf16 small (MFMA indexer + attention)")
    B, T, D, DI, H, HI, Tq, k, ratio, n_win, R = 2, 512, 128, 32, 16, 16, 24, 16, 4, 32, 64
    r = _run_forward("bf16", B, T, D, DI, H, HI, Tq, k, ratio, n_win, R, 1.0, 1234)

    def band(b, t):
        # one bf16 step of every key element, weighted by |q| and w, bounds the score change
        qI, wI = f64(r["qI"][b, t]), f64(r["wI"][b, t])
        keys = np.abs(f64(r["ik"].data[b]))
        return 2.0 ** -8 * float((wI[:, None] * (np.abs(qI) @ keys.T)).sum(0).max())

    for b in range(B):
        _check_layer(r, b, "bf16", k, ratio, n_win, R, 1.0, band_fn=band)


def test_forward_chunked_compression_matches_whole():
    # two csa_forward calls (t0 = 0, then t0 = 128 with the previous block) build the
    # same caches as one compression of the whole sequence
    say("forward chunked prefill")
    g = Gen(99, DEV)
    B, T, D, DI, H, HI, ratio = 1, 256, 128, 32, 16, 16, 4
    streams, istreams, q, qI, wI, win, sink = _csa_case(g, B, T, D, DI, H, HI, 4, "f32")
    N = T // ratio
    kv = csa.Buf.empty((B, N, D), csa.CSA_F32)
    ik = csa.Buf.empty((B, N, DI), csa.CSA_F32)
    win_pos0 = torch.zeros((B,), dtype=torch.int64, device=DEV)
    half = T // 2
    for t0 in (0, half):
        sl = slice(t0, t0 + half)
        pos = torch.arange(t0 + half - 4, t0 + half, dtype=torch.int64, device=DEV).expand(B, 4).contiguous()
        desc = csa.layer_desc(mode=csa.CSA_MODE_CSA, B=B, T=half, t0=t0, Tq=4, cache_rows=N, Tw=T, D=D, H=H, HI=HI,
                              DI=DI, ratio=ratio, topk=8, n_win=16, rope_dims=64, rope_base=10000.0,
                              softmax_scale=1.0, stream_dtype=csa.CSA_F32)
        io = dict(ca=streams[0][:, sl].contiguous(), cb=streams[1][:, sl].contiguous(),
                  za=streams[2][:, sl].contiguous(), zb=streams[3][:, sl].contiguous(),
                  ica=istreams[0][:, sl].contiguous(), icb=istreams[1][:, sl].contiguous(),
                  iza=istreams[2][:, sl].contiguous(), izb=istreams[3][:, sl].contiguous(),
                  kv_cache=kv, ik_cache=ik, q=q, q_pos=pos, qI=qI, wI=wI, win=win, win_pos0=win_pos0, sink=sink,
                  out=torch.empty_like(q))
        if t0 > 0:
            io.update(prev_cb=streams[1][:, t0 - ratio:t0].contiguous(), prev_zb=streams[3][:, t0 - ratio:t0].contiguous(),
                      iprev_cb=istreams[1][:, t0 - ratio:t0].contiguous(),
                      iprev_zb=istreams[3][:, t0 - ratio:t0].contiguous())
        csa.csa_forward(desc, io)
    torch.cuda.synchronize()
    whole = O.compress(*[f64(s[0]) for s in streams], ratio=ratio, overlap=True, rope_dims=64, rope_base=10000.0)
    assert_close(f64(kv.data[0]), whole, "f32", "chunked KV cache")
    iwhole = O.compress(*[f64(s[0]) for s in istreams], ratio=ratio, overlap=True)
    assert_close(f64(ik.data[0]), iwhole, "f32", "chunked indexer cache")


def test_forward_hca():
    say("forward HCA")
    g = Gen(7003, DEV)
    B, T, D, H, Tq, ratio, n_win = 1, 2048, 512, 64, 4, 128, 128
    C_, Z = g.normal((B, T, D), dtype=torch.bfloat16), g.normal((B, T, D), dtype=torch.bfloat16)
    q = g.normal((B, Tq, H, D), qstd(D), dtype=torch.bfloat16)
    win = g.normal((B, T, D), dtype=torch.bfloat16)
    sink = g.normal((H,))
    N = T // ratio
    kv = csa.Buf.empty((B, N, D), csa.CSA_BF16)
    pos = torch.tensor([[127, 128, 1500, 2047]], dtype=torch.int64, device=DEV)
    win_pos0 = torch.zeros((B,), dtype=torch.int64, device=DEV)
    out = torch.empty_like(q)
    desc = csa.layer_desc(mode=csa.CSA_MODE_HCA, B=B, T=T, t0=0, Tq=Tq, cache_rows=N, Tw=T, D=D, H=H, ratio=ratio,
                          n_win=n_win, rope_dims=64, rope_base=10000.0, softmax_scale=1.0, stream_dtype=csa.CSA_BF16)
    csa.csa_forward(desc, dict(ca=C_, za=Z, kv_cache=kv, q=q, q_pos=pos, win=win, win_pos0=win_pos0, sink=sink,
                               out=out))
    torch.cuda.synchronize()
    want = O.hca_layer((f64(C_[0]), f64(Z[0])), f64(q[0]), pos[0].cpu().numpy(), f64(win[0]), 0, f64(sink),
                       ratio=ratio, n_win=n_win, scale=1.0, rope_dims=64, rope_base=10000.0, dtype="bf16")
    assert_close(f64(kv.data[0]), want["kv"], "bf16", "HCA cache")
    assert_close(f64(out[0]), want["out"], "bf16", "HCA output")
