"""Parity at the workloads' full sizes, in the launch configuration bench.py times.

Each test builds one workload with bench.build_workload (same shapes, caches, seeds
and csa_forward descriptors as the benchmark), runs one step, and checks sampled
outputs against the oracle one by one:

- compressed entries of the step's chunk (oracle over the chunk's own streams) and
  of the cache build (streams regenerated from the same seeded generator);
- whole index-score rows of sampled queries (oracle over the GPU-stored keys);
- the top-k set of those rows (near-tie rule: differences only where the oracle
  score is within 1e-4 relative of the k-th score);
- attention outputs of the sampled queries (oracle over the GPU-stored cache, the
  GPU's own selection, the window and the sink).

Tolerances: bf16 2e-2 abs/rel; FP8-mixed cache / MXFP4 indexer 5e-2 on dequantized
inputs; index scores 1e-4 relative (fp32 accumulation of exact products).
"""

import sys

import numpy as np
import pytest
import torch

from helpers import assert_close, ensure_built, f64, topk_sets_agree
from oracle import csa_oracle as O
from oracle import quant as Q

pytestmark = pytest.mark.gpu

import bench  # noqa: E402
import compressed_sparse_attention_07_amd as csa  # noqa: E402
from synth import Gen  # noqa: E402

DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _lib():
    ensure_built()
    yield
    torch.cuda.empty_cache()


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def deq(x, b):
    """fp64 values of sequence b of a tensor or storage buffer."""
    if isinstance(x, torch.Tensor):
        return f64(x[b])
    if x.dtype == csa.CSA_FP8MIX:
        return Q.fp8mix_dequantize(x.data[b].cpu().numpy(), x.rope[b].view(torch.int16).cpu().numpy().view(np.uint16),
                                   x.scale[b].cpu().numpy())
    if x.dtype == csa.CSA_MXFP4:
        return Q.mxfp4_dequantize(x.data[b].cpu().numpy(), x.scale[b].cpu().numpy())
    return f64(x.data[b])


def _run_step(wl, scores=True):
    io = dict(wl.ios[0])
    M = wl.meta
    if M["mode"] == "csa" and scores:
        io["scores_out"] = torch.empty((M["B"], M["Tq"], M["N"]), dtype=torch.float32, device=DEV)
        io["idx_out"] = torch.empty((M["B"], M["Tq"], M["k"]), dtype=torch.int32, device=DEV)
    desc = wl.desc_full if wl.desc_full is not None else wl.desc_attend
    csa.csa_forward(desc, io, ws=wl.ws)
    torch.cuda.synchronize()
    return io


def _check_chunk_compress(wl, io, b):
    """Entries written by the step's chunk compression vs the oracle over its streams."""
    M, cfg = wl.meta, wl.cfg
    T, m, R = M["T_step"], M["m"], M["R"]
    if not T:
        return
    t0 = M["ctx"] - T
    hca = M["mode"] == "hca"
    if hca:
        want = O.compress(f64(io["ca"][b]), None, f64(io["za"][b]), None, ratio=m, overlap=False, t0=t0,
                          rope_dims=R, rope_base=cfg.rope_base)
    else:
        want = O.compress(f64(io["ca"][b]), f64(io["cb"][b]), f64(io["za"][b]), f64(io["zb"][b]), ratio=m,
                          overlap=True, t0=t0, prev_cb=f64(io["prev_cb"][b]), prev_zb=f64(io["prev_zb"][b]),
                          rope_dims=R, rope_base=cfg.rope_base)
        wi = O.compress(f64(io["ica"][b]), f64(io["icb"][b]), f64(io["iza"][b]), f64(io["izb"][b]), ratio=m,
                        overlap=True, t0=t0, prev_cb=f64(io["iprev_cb"][b]), prev_zb=f64(io["iprev_zb"][b]))
        got_i = f64(io["ik_cache"].data[b, t0 // m:(t0 + T) // m])
        assert_close(got_i, wi, "bf16", "chunk indexer keys")
    got = f64(io["kv_cache"].data[b, t0 // m:(t0 + T) // m])
    assert_close(got, want, "bf16", "chunk KV entries")


def _check_bulk_compress(wl, samples=48):
    """Sampled entries of sequence 0's cache build (streams regenerated: each sequence's
    generator draws its whole KV streams, then its whole indexer streams)."""
    M, cfg = wl.meta, wl.cfg
    m, D, R, DI = M["m"], M["D"], M["R"], M["DI"]
    hca = M["mode"] == "hca"
    tokens = (M["ctx"] - M["T_step"]) if M["T_step"] else M["ctx"]
    T = tokens
    g = Gen(cfg.seed * 1000, DEV)
    n_st = 2 if hca else 4
    s = [g.normal((T, D), dtype=torch.bfloat16) for _ in range(n_st)]
    rng = np.random.default_rng(5)
    ents = sorted(set([0, 1, T // m - 1] + list(rng.integers(0, T // m, samples))))
    for i in ents:
        lo, hi = max(0, m * (i - 1)), m * (i + 1)
        blk = [f64(x[lo:hi]) for x in s]
        if hca:
            want = O.compress(blk[0][m:] if i > 0 else blk[0][:m], None, blk[1][m:] if i > 0 else blk[1][:m], None,
                              ratio=m, overlap=False, t0=m * i, rope_dims=R, rope_base=cfg.rope_base)
        elif i == 0:
            want = O.compress(blk[0], blk[1], blk[2], blk[3], ratio=m, overlap=True, t0=0, rope_dims=R,
                              rope_base=cfg.rope_base)
        else:
            want = O.compress(blk[0][m:], blk[1][m:], blk[2][m:], blk[3][m:], ratio=m, overlap=True, t0=m * i,
                              prev_cb=blk[1][:m], prev_zb=blk[3][:m], rope_dims=R, rope_base=cfg.rope_base)
        got = f64(wl.ios[0]["kv_cache"].data[0, i:i + 1])
        assert_close(got, want[:1], "bf16", f"bulk KV entry {i}")
    if not hca:
        del s
        si = [g.normal((T, DI), dtype=torch.bfloat16) for _ in range(4)]
        for i in ents[1:8]:
            blk = [f64(x[m * (i - 1):m * (i + 1)]) for x in si]
            want = O.compress(blk[0][m:], blk[1][m:], blk[2][m:], blk[3][m:], ratio=m, overlap=True, t0=m * i,
                              prev_cb=blk[1][:m], prev_zb=blk[3][:m])
            got = f64(wl.ios[0]["ik_cache"].data[0, i:i + 1])
            assert_close(got, want[:1], "bf16", f"bulk indexer key {i}")


def _check_queries(wl, io, units):
    """Index scores, top-k and attention output of sampled (sequence, query) units."""
    M, cfg = wl.meta, wl.cfg
    m, R, W, k = M["m"], M["R"], M["W"], M["k"]
    hca = M["mode"] == "hca"
    kind = "fp8" if M["kv_format"] == "fp8mix" else "bf16"
    by_seq = {}
    for b, t in units:
        by_seq.setdefault(b, []).append(t)
    for b, ts in by_seq.items():
        kv = deq(io["kv_cache"], b)
        win = deq(io["win"], b)
        wp0 = int(io["win_pos0"][b])
        sink = f64(io["sink"])
        pos = io["q_pos"][b].cpu().numpy()
        if not hca:
            ik = deq(io["ik_cache"], b)
            qI = deq(io["qI"], b)
        for t in ts:
            say(f"  unit b={b} t={t} pos={pos[t]}")
            q = deq(io["q"], b)[t:t + 1]
            p = pos[t:t + 1]
            if hca:
                want = O.hca_dense(q, p, kv, win, wp0, W, sink, ratio=m, scale=cfg.softmax_scale, rope_dims=R,
                                   rope_base=cfg.rope_base)
            else:
                sc = O.index_scores(qI[t:t + 1], f64(io["wI"][b, t:t + 1]), ik, p, m)
                got_sc = io["scores_out"][b, t].cpu().numpy().astype(np.float64)
                fin = np.isfinite(sc[0])
                assert np.array_equal(np.isneginf(got_sc), np.isneginf(sc[0])), "score mask differs"
                assert_close(got_sc[fin], sc[0][fin], "f32", f"scores b={b} t={t}")
                gidx = io["idx_out"][b, t].cpu().numpy()
                ok, _ = topk_sets_agree(gidx, int((gidx >= 0).sum()), sc[0], k)
                assert ok, f"top-k set differs beyond the near-tie band (b={b} t={t})"
                want = O.mqa(q, p, kv, gidx[None], win, wp0, W, sink, scale=cfg.softmax_scale, rope_dims=R,
                             rope_base=cfg.rope_base)
            assert_close(f64(io["out"][b, t:t + 1]), want, kind, f"output b={b} t={t}")
        del kv, win


@pytest.mark.timeout(900)
def test_csa_decode_128k_b16():
    say("full size: CSA decode, B=16, 128K context")
    wl = bench.build_workload("1", layers=1)
    io = _run_step(wl)
    _check_chunk_compress(wl, io, 0)
    _check_chunk_compress(wl, io, 15)
    _check_bulk_compress(wl)
    _check_queries(wl, io, [(0, 0), (7, 0), (15, 0)])


@pytest.mark.timeout(900)
def test_csa_prefill_1m_t2048():
    say("full size: CSA chunked prefill, 1M context, 2048 queries")
    wl = bench.build_workload("2", layers=1)
    io = _run_step(wl)
    _check_chunk_compress(wl, io, 0)
    _check_bulk_compress(wl)
    _check_queries(wl, io, [(0, 0), (0, 1023), (0, 2047)])


@pytest.mark.timeout(900)
def test_hca_decode_1m_b32():
    say("full size: HCA decode, B=32, 1M context")
    wl = bench.build_workload("3d", layers=1)
    io = _run_step(wl)
    _check_bulk_compress(wl)
    _check_queries(wl, io, [(0, 0), (13, 0), (31, 0)])


@pytest.mark.timeout(900)
def test_hca_prefill_1m_t2048():
    say("full size: HCA prefill, 1M context, 2048 queries")
    wl = bench.build_workload("3p", layers=1)
    io = _run_step(wl)
    _check_chunk_compress(wl, io, 0)
    _check_queries(wl, io, [(0, 0), (0, 777), (0, 2047)])


@pytest.mark.timeout(900)
def test_mixed_precision_decode_1m_b8():
    say("full size: CSA decode, B=8, 1M context, FP8-mixed KV, MXFP4 indexer")
    wl = bench.build_workload("4", layers=1)
    io = _run_step(wl)
    _check_queries(wl, io, [(0, 0), (3, 0), (7, 0)])
    # the same step with FP8MIX queries: the QK products of the codes on fp8 MFMA
    say("  ... with FP8MIX queries")
    q = io["q"]
    D, R = q.shape[-1], wl.meta["R"]
    q8 = csa.Buf.empty(tuple(q.shape), csa.CSA_FP8MIX, rope_dims=R)
    csa.csa_quantize(q.float().reshape(-1, D).contiguous(),
                     csa.Buf(q8.dtype, q8.data.view(-1, D - R), q8.rope.view(-1, R), q8.scale.view(-1)), rope_dims=R)
    io8 = dict(io, q=q8, out=torch.empty_like(io["out"]))
    desc = wl.desc_full if wl.desc_full is not None else wl.desc_attend
    csa.csa_forward(desc, io8, ws=wl.ws)
    torch.cuda.synchronize()
    _check_queries(wl, io8, [(1, 0), (6, 0)])
