"""End-to-end csa_forward parity (compress -> indexer -> top-k -> sparse MQA, and
the HCA chain) against the oracle's whole-layer functions.

The oracle runs its own pipeline from the same inputs.  Top-k sets must agree
except for entries whose oracle score lies within 1e-4 (relative) of the k-th
score.  In fp32 the oracle scores its own compressed keys.  In bf16 the stored keys
of the two sides may differ by one bf16 rounding step (the compressors accumulate
in fp32 and fp64), which moves scores by up to ~2^-8 relative, far beyond the 1e-4
band; there the oracle scores the keys the GPU stored (themselves checked against
the oracle's compression within the bf16 tolerance), as each stage's oracle input
is the tensor that GPU stage consumed.  Every query's output is checked: against
the oracle layer where the selected sets are identical, and against the oracle's
attention over the GPU's own selection where a near tie made them differ.
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


def _run_forward(dtype, B, T, D, DI, H, HI, Tq, k, ratio, n_win, R, scale, seed, norm=False):
    g = Gen(seed, DEV)
    streams, istreams, q, qI, wI, win, sink = _csa_case(g, B, T, D, DI, H, HI, Tq, dtype)
    # RMSNorm weights of the query heads and the KV (near 1, as trained norms are)
    q_norm = g.uniform((D,), 0.5, 1.5) if norm else None
    kv_norm = g.uniform((D,), 0.5, 1.5) if norm else None
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
                          pos_offset=0, stream_dtype=dt, flags=csa.CSA_FLAG_QKV_NORM if norm else 0,
                          norm_eps=1e-6)
    io = dict(ca=streams[0], cb=streams[1], za=streams[2], zb=streams[3], ica=istreams[0], icb=istreams[1],
              iza=istreams[2], izb=istreams[3], kv_cache=kv, ik_cache=ik, q=q, q_pos=pos, qI=qI, wI=wI, win=win,
              win_pos0=win_pos0, sink=sink, out=out, scores_out=scores, idx_out=idx, q_norm=q_norm, kv_norm=kv_norm)
    csa.csa_forward(desc, io)
    torch.cuda.synchronize()
    return dict(streams=streams, istreams=istreams, q=q, qI=qI, wI=wI, win=win, sink=sink, pos=pos, kv=kv, ik=ik,
                out=out, scores=scores, idx=idx, q_norm=None if q_norm is None else f64(q_norm),
                kv_norm=None if kv_norm is None else f64(kv_norm))


def _check_layer(r, b, dtype, k, ratio, n_win, R, scale):
    norms = dict(q_norm=r.get("q_norm"), kv_norm=r.get("kv_norm"), norm_eps=1e-6)
    want = O.csa_layer([f64(s[b]) for s in r["streams"]], [f64(s[b]) for s in r["istreams"]], f64(r["q"][b]),
                       r["pos"][b].cpu().numpy(), f64(r["qI"][b]), f64(r["wI"][b]), f64(r["win"][b]), 0,
                       f64(r["sink"]), ratio=ratio, k=k, n_win=n_win, scale=scale, rope_dims=R, rope_base=10000.0,
                       dtype=dtype, **norms)
    kind = "f32" if dtype == "f32" else "bf16"
    assert_close(f64(r["kv"].data[b]), want["kv"], kind, "compressed KV")
    assert_close(f64(r["ik"].data[b]), want["ik"], kind, "compressed indexer keys")
    pos = r["pos"][b].cpu().numpy()
    if dtype == "f32":
        ref_scores = want["scores"]
    else:
        ref_scores = O.index_scores(f64(r["qI"][b]), f64(r["wI"][b]), f64(r["ik"].data[b]), pos, ratio)
    gs = r["scores"][b].cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isneginf(gs), np.isneginf(ref_scores))
    fin = np.isfinite(ref_scores)
    assert_close(gs[fin], ref_scores[fin], "f32", "scores")
    gi = r["idx"][b].cpu().numpy()
    got_out = f64(r["out"][b])
    n_exact = 0
    for t in range(gi.shape[0]):
        cnt = int((gi[t] >= 0).sum())
        ok, exact = topk_sets_agree(gi[t], cnt, ref_scores[t], k)
        assert ok, f"top-k set of query {t} differs beyond the near-tie band"
        n_exact += exact
        ref_idx = want["idx"][t] if dtype == "f32" else O.topk(ref_scores[t:t + 1], k)[0][0]
        if np.array_equal(gi[t], ref_idx) and dtype == "f32":
            wt = want["out"][t]
        else:
            # the oracle's attention over the GPU's own selection (and the oracle's cache)
            wt = O.store(O.mqa(f64(r["q"][b, t:t + 1]), pos[t:t + 1], want["kv"], gi[t:t + 1], f64(r["win"][b]), 0,
                               n_win, f64(r["sink"]), scale=scale, rope_dims=R, rope_base=10000.0, **norms)[0], dtype)
        assert_close(got_out[t], wt, kind, f"output of query {t}")
    say(f"  sequence {b}: {n_exact} of {gi.shape[0]} selections identical, every output checked")


def test_forward_config0_fp32_full():
    c = CONFIGS[0]
    say("forward config 0 (fp32, T=1024, every query)")
    r = _run_forward("f32", c.B, c.ctx, c.D, c.DI, c.H, c.HI, c.Tq, c.k, c.m, c.n_win, c.R, c.softmax_scale, c.seed)
    _check_layer(r, 0, "f32", c.k, c.m, c.n_win, c.R, c.softmax_scale)


def test_forward_bf16_mfma_paths():
    say("forward bf16 small (MFMA indexer + attention)")
    B, T, D, DI, H, HI, Tq, k, ratio, n_win, R = 2, 512, 128, 32, 16, 16, 24, 16, 4, 32, 64
    r = _run_forward("bf16", B, T, D, DI, H, HI, Tq, k, ratio, n_win, R, 1.0, 1234)
    for b in range(B):
        _check_layer(r, b, "bf16", k, ratio, n_win, R, 1.0)


def test_forward_bf16_decode_fused_selection():
    # few queries per sequence: the indexer selects while it scores (2048-entry slices,
    # so several slices and a partial last one here)
    say("forward bf16 decode shape (fused indexer + top-k)")
    B, T, D, DI, H, HI, Tq, k, ratio, n_win, R = 3, 20480, 128, 64, 16, 16, 2, 64, 4, 64, 64
    r = _run_forward("bf16", B, T, D, DI, H, HI, Tq, k, ratio, n_win, R, 1.0, 4321)
    for b in range(B):
        _check_layer(r, b, "bf16", k, ratio, n_win, R, 1.0)


def test_forward_qkv_norm_fp32():
    # query heads, compressed entries and window rows RMS-normalized before attention
    say("forward fp32 with Q/KV RMSNorm")
    B, T, D, DI, H, HI, Tq, k, ratio, n_win, R = 1, 512, 128, 32, 8, 8, 40, 16, 4, 32, 64
    r = _run_forward("f32", B, T, D, DI, H, HI, Tq, k, ratio, n_win, R, D ** -0.5, 2024, norm=True)
    _check_layer(r, 0, "f32", k, ratio, n_win, R, D ** -0.5)


def test_forward_qkv_norm_bf16_decode():
    # the headline layer shape (512-dim heads, 64 RoPE dims) at decode: the wave-pair
    # attention kernel reads the normalized query and window copies
    say("forward bf16 decode with Q/KV RMSNorm")
    B, T, D, DI, H, HI, Tq, k, ratio, n_win, R = 2, 8192, 512, 128, 64, 64, 1, 256, 4, 128, 64
    r = _run_forward("bf16", B, T, D, DI, H, HI, Tq, k, ratio, n_win, R, D ** -0.5, 2025, norm=True)
    for b in range(B):
        _check_layer(r, b, "bf16", k, ratio, n_win, R, D ** -0.5)


def test_forward_qkv_norm_multilevel_topk():
    # more than 64 selection rows over 5120 entries: the selection runs in two levels and
    # the normalization job rides on the last one
    say("forward bf16 with Q/KV RMSNorm, two-level top-k")
    B, T, D, DI, H, HI, Tq, k, ratio, n_win, R = 1, 20480, 128, 64, 16, 16, 70, 64, 4, 128, 64
    r = _run_forward("bf16", B, T, D, DI, H, HI, Tq, k, ratio, n_win, R, D ** -0.5, 2026, norm=True)
    _check_layer(r, 0, "bf16", k, ratio, n_win, R, D ** -0.5)


def test_forward_with_no_queries_only_compresses():
    # Tq = 0 (a compression-only step, bf16 decode shape): the caches are written and
    # no selection or attention launch runs
    say("forward with Tq = 0")
    g = Gen(98, DEV)
    B, T, D, DI, H, HI, ratio = 2, 64, 128, 64, 16, 16, 4
    # the query buffers exist (one token each) but the descriptor asks for none
    streams, istreams, q, qI, wI, win, sink = _csa_case(g, B, T, D, DI, H, HI, 1, "bf16")
    N = T // ratio
    kv = csa.Buf.empty((B, N, D), csa.CSA_BF16)
    ik = csa.Buf.empty((B, N, DI), csa.CSA_BF16)
    desc = csa.layer_desc(mode=csa.CSA_MODE_CSA, B=B, T=T, t0=0, Tq=0, cache_rows=N, Tw=T, D=D, H=H, HI=HI, DI=DI,
                          ratio=ratio, topk=8, n_win=16, rope_dims=64, rope_base=10000.0, softmax_scale=1.0,
                          stream_dtype=csa.CSA_BF16)
    io = dict(ca=streams[0], cb=streams[1], za=streams[2], zb=streams[3], ica=istreams[0], icb=istreams[1],
              iza=istreams[2], izb=istreams[3], kv_cache=kv, ik_cache=ik, q=q, q_pos=torch.zeros((B, 1), dtype=torch.int64,
              device=DEV), qI=qI, wI=wI, win=win, win_pos0=torch.zeros((B,), dtype=torch.int64, device=DEV), sink=sink,
              out=torch.empty_like(q))
    csa.csa_forward(desc, io)
    torch.cuda.synchronize()
    for b in range(B):
        want = O.compress(*[f64(x[b]) for x in streams], ratio=ratio, overlap=True, rope_dims=64, rope_base=10000.0)
        assert_close(f64(kv.data[b]), want, "bf16", "KV cache")
        iwant = O.compress(*[f64(x[b]) for x in istreams], ratio=ratio, overlap=True)
        assert_close(f64(ik.data[b]), iwant, "bf16", "indexer cache")


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


def test_forward_hca_qkv_norm():
    say("forward HCA with Q/KV RMSNorm")
    g = Gen(7004, DEV)
    B, T, D, H, Tq, ratio, n_win = 2, 1024, 512, 16, 3, 128, 128
    C_, Z = g.normal((B, T, D), dtype=torch.bfloat16), g.normal((B, T, D), dtype=torch.bfloat16)
    q = g.normal((B, Tq, H, D), qstd(D), dtype=torch.bfloat16)
    win = g.normal((B, T, D), dtype=torch.bfloat16)
    sink = g.normal((H,))
    q_norm, kv_norm = g.uniform((D,), 0.5, 1.5), g.uniform((D,), 0.5, 1.5)
    N = T // ratio
    kv = csa.Buf.empty((B, N, D), csa.CSA_BF16)
    # queries of the two sequences at different positions (each sequence's own window span)
    pos = torch.tensor([[5, 640, 1023], [127, 128, 900]], dtype=torch.int64, device=DEV)
    win_pos0 = torch.zeros((B,), dtype=torch.int64, device=DEV)
    out = torch.empty_like(q)
    scale = D ** -0.5
    desc = csa.layer_desc(mode=csa.CSA_MODE_HCA, B=B, T=T, t0=0, Tq=Tq, cache_rows=N, Tw=T, D=D, H=H, ratio=ratio,
                          n_win=n_win, rope_dims=64, rope_base=10000.0, softmax_scale=scale, stream_dtype=csa.CSA_BF16,
                          flags=csa.CSA_FLAG_QKV_NORM, norm_eps=1e-6)
    csa.csa_forward(desc, dict(ca=C_, za=Z, kv_cache=kv, q=q, q_pos=pos, win=win, win_pos0=win_pos0, sink=sink,
                               out=out, q_norm=q_norm, kv_norm=kv_norm))
    torch.cuda.synchronize()
    for b in range(B):
        want = O.hca_layer((f64(C_[b]), f64(Z[b])), f64(q[b]), pos[b].cpu().numpy(), f64(win[b]), 0, f64(sink),
                           ratio=ratio, n_win=n_win, scale=scale, rope_dims=64, rope_base=10000.0, dtype="bf16",
                           q_norm=f64(q_norm), kv_norm=f64(kv_norm), norm_eps=1e-6)
        assert_close(f64(kv.data[b]), want["kv"], "bf16", f"HCA normalized cache of sequence {b}")
        assert_close(f64(out[b]), want["out"], "bf16", f"HCA output with norms, sequence {b}")
