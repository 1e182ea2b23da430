"""Pins of oracle/csa_oracle.py against closed forms, invariants and brute force.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, the wrong softmax axis, a wrong RoPE
position) fails at least one of them.
"""

import math

import numpy as np
import pytest
import scipy.special

from oracle import csa_oracle as O

RB = 10000.0


def rng(seed=0):
    return np.random.default_rng(seed)


# ------------------------------------------------------------------------- RoPE


def test_rope_identity_norm_composition():
    r = rng(1)
    x = r.standard_normal((5, 32))
    assert np.array_equal(O.rope(x, 0, 16, RB), x)
    y = O.rope(x, 123456.0, 16, RB)
    assert np.allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    assert np.array_equal(y[:, :16], x[:, :16])            # non-RoPE dims untouched
    assert np.allclose(O.rope(O.rope(x, 700, 16, RB), 45, 16, RB), O.rope(x, 745, 16, RB), atol=1e-12)
    assert np.allclose(O.rope(y, -123456.0, 16, RB), x, atol=1e-10)


def test_rope_relative_dot_product():
    r = rng(2)
    q, k = r.standard_normal(64), r.standard_normal(64)
    d1 = O.rope(q, 1000, 64, RB) @ O.rope(k, 990, 64, RB)
    d2 = O.rope(q, 20, 64, RB) @ O.rope(k, 10, 64, RB)
    assert abs(d1 - d2) < 1e-10


def test_rope_closed_form_pairs():
    # unit vector in pair 0 (frequency 1) and in the last pair (frequency base^(-62/64))
    D, R, p = 80, 64, 777
    x = np.zeros(D)
    x[D - R] = 1.0
    y = O.rope(x, p, R, RB)
    assert np.allclose(y[D - R:D - R + 2], [math.cos(p), math.sin(p)], atol=1e-12)
    x = np.zeros(D)
    x[D - 1] = 1.0                       # odd element of the last pair
    y = O.rope(x, p, R, RB)
    th = 10.0 ** -3.875                  # 10000^(-62/64)
    assert np.allclose(y[D - 2:], [-math.sin(p * th), math.cos(p * th)], atol=1e-12)


# --------------------------------------------------------------------- compress


def _streams(T, D, seed=0):
    r = rng(seed)
    return [r.standard_normal((T, D)) for _ in range(4)]


def test_compress_constant_reproduces_constant():
    T, D = 32, 8
    _, _, Za, Zb = _streams(T, D)
    C = np.full((T, D), 2.5)
    e = O.compress(C, C, Za, Zb, ratio=4, overlap=True)
    assert np.allclose(e, 2.5, rtol=1e-14)
    e = O.compress(C, None, Za, None, ratio=8, overlap=False)
    assert np.allclose(e, 2.5, rtol=1e-14)


def test_compress_zero_logits_is_mean():
    T, D, m = 24, 6, 4
    Ca, Cb, _, _ = _streams(T, D, 3)
    Z = np.zeros((T, D))
    e = O.compress(Ca, Cb, Z, Z, ratio=m, overlap=True)
    # entry 0: no previous block -> mean of its own m a-rows
    assert np.allclose(e[0], Ca[0:m].mean(0))
    for i in range(1, T // m):
        want = (Ca[m * i:m * i + m].sum(0) + Cb[m * (i - 1):m * i].sum(0)) / (2 * m)
        assert np.allclose(e[i], want, rtol=1e-13)


def test_compress_dominant_logit_selects_row():
    # one large logit per (entry, channel) picks exactly that row: pins which rows feed
    # the a- and b-branches and that the softmax runs per channel over positions
    T, D, m = 32, 5, 4
    Ca, Cb, Za, Zb = _streams(T, D, 4)
    Za, Zb = Za * 0.01, Zb * 0.01
    r = rng(7)
    want = np.zeros((T // m, D))
    for i in range(T // m):
        for d in range(D):
            use_b = i >= 1 and r.random() < 0.5
            j = int(r.integers(m))
            if use_b:
                Zb[m * (i - 1) + j, d] = 60.0
                want[i, d] = Cb[m * (i - 1) + j, d]
            else:
                Za[m * i + j, d] = 60.0
                want[i, d] = Ca[m * i + j, d]
    e = O.compress(Ca, Cb, Za, Zb, ratio=m, overlap=True)
    assert np.allclose(e, want, atol=1e-20 + 1e-20 * 0 + 1e-22, rtol=1e-12)


def test_compress_bias_indexes_in_block_position():
    T, D, m = 16, 3, 4
    Ca, Cb, Za, Zb = _streams(T, D, 5)
    ba = np.zeros((m, D))
    bb = np.zeros((m, D))
    ba[2, 1] = 80.0                       # channel 1 follows in-block a-row 2
    bb[3, 0] = 80.0                       # channel 0 follows in-block b-row 3 (i >= 1)
    e = O.compress(Ca, Cb, Za, Zb, ratio=m, overlap=True, bias_a=ba, bias_b=bb)
    for i in range(T // m):
        assert np.isclose(e[i, 1], Ca[m * i + 2, 1], rtol=1e-12)
        if i >= 1:
            assert np.isclose(e[i, 0], Cb[m * (i - 1) + 3, 0], rtol=1e-12)


def test_compress_logit_shift_invariance_and_minus_inf_branch():
    T, D, m = 16, 4, 4
    Ca, Cb, Za, Zb = _streams(T, D, 6)
    e1 = O.compress(Ca, Cb, Za, Zb, ratio=m, overlap=True)
    e2 = O.compress(Ca, Cb, Za + 3.0, Zb + 3.0, ratio=m, overlap=True)
    assert np.allclose(e1, e2, rtol=1e-12)
    # a b-branch at -inf reduces CSA to non-overlapping compression with ratio m
    e3 = O.compress(Ca, Cb, Za, np.full_like(Zb, -np.inf), ratio=m, overlap=True)
    e4 = O.compress(Ca, None, Za, None, ratio=m, overlap=False)
    assert np.allclose(e3, e4, rtol=1e-13)


def test_compress_chunked_equals_whole():
    T, D, m = 48, 8, 4
    Ca, Cb, Za, Zb = _streams(T, D, 8)
    whole = O.compress(Ca, Cb, Za, Zb, ratio=m, overlap=True, rope_dims=4, rope_base=RB)
    t0 = 20
    part = O.compress(Ca[t0:], Cb[t0:], Za[t0:], Zb[t0:], ratio=m, overlap=True, t0=t0,
                      prev_cb=Cb[t0 - m:t0], prev_zb=Zb[t0 - m:t0], rope_dims=4, rope_base=RB)
    assert np.allclose(part, whole[t0 // m:], rtol=1e-13)


def test_compress_rope_position_is_ratio_times_index():
    T, D, m, R = 32, 8, 4, 4
    _, _, Za, Zb = _streams(T, D, 9)
    C = np.zeros((T, D))
    C[:, D - R] = 1.0                     # constant vector (1, 0) in RoPE pair 0
    off = 1000
    e = O.compress(C, C, Za, Zb, ratio=m, overlap=True, rope_dims=R, rope_base=RB, pos_offset=off)
    for i in range(T // m):
        p = off + m * i
        assert np.allclose(e[i, D - R:D - R + 2], [math.cos(p), math.sin(p)], atol=1e-12)
    # HCA: position ratio * i as well
    e = O.compress(C, None, Za, None, ratio=8, overlap=False, rope_dims=R, rope_base=RB)
    for i in range(T // 8):
        assert np.allclose(e[i, D - R:D - R + 2], [math.cos(8 * i), math.sin(8 * i)], atol=1e-12)


def test_compress_brute_force_scalar_loops():
    # tiny case, evaluated with scalar math.exp loops over an explicit position list
    T, D, m = 12, 2, 3
    Ca, Cb, Za, Zb = _streams(T, D, 10)
    e = O.compress(Ca, Cb, Za, Zb, ratio=m, overlap=True)
    for i in range(T // m):
        for d in range(D):
            pairs = [(Za[r, d], Ca[r, d]) for r in range(m * i, m * i + m)]
            if i > 0:
                pairs += [(Zb[r, d], Cb[r, d]) for r in range(m * i - m, m * i)]
            num = sum(math.exp(z) * c for z, c in pairs)
            den = sum(math.exp(z) for z, _ in pairs)
            assert math.isclose(e[i, d], num / den, rel_tol=1e-12)


# ------------------------------------------------------------------ index scores


def test_scores_brute_force_and_mask():
    r = rng(12)
    Tq, HI, DI, N, m = 6, 3, 4, 9, 4
    q = r.standard_normal((Tq, HI, DI))
    w = r.uniform(0, 1, (Tq, HI))
    K = r.standard_normal((N, DI))
    pos = np.array([0, 3, 4, 7, 17, 40])
    s = O.index_scores(q, w, K, pos, m)
    for t in range(Tq):
        vis = min(N, pos[t] // m)
        assert np.all(np.isneginf(s[t, vis:]))
        for j in range(vis):
            tot = 0.0
            for h in range(HI):
                dot = sum(q[t, h, d] * K[j, d] for d in range(DI))
                tot += w[t, h] * (dot if dot > 0 else 0.0)
            assert math.isclose(s[t, j], tot, rel_tol=1e-12, abs_tol=1e-14)


def test_scores_single_head_is_relu_dot():
    r = rng(13)
    q = r.standard_normal((1, 1, 8))
    K = r.standard_normal((5, 8))
    s = O.index_scores(q, np.ones((1, 1)), K, np.array([100]), 4)
    assert np.allclose(s[0], np.maximum(K @ q[0, 0], 0.0))


def test_scores_positive_scaling_keeps_ranking():
    r = rng(14)
    q = r.standard_normal((2, 4, 8))
    w = r.uniform(0, 1, (2, 4))
    K = r.standard_normal((30, 8))
    pos = np.array([200, 200])
    a = O.index_scores(q, w, K, pos, 4)
    b = O.index_scores(3.0 * q, 0.5 * w, K, pos, 4)
    assert np.array_equal(np.argsort(-a, axis=1, kind="stable"), np.argsort(-b, axis=1, kind="stable"))


# ------------------------------------------------------------------------- top-k


def _valid_topk(row, sel, k):
    vis = [j for j in range(len(row)) if np.isfinite(row[j])]
    S = set(int(x) for x in sel if x >= 0)
    if len(S) != min(k, len(vis)):
        return False
    for s in S:
        for u in vis:
            if u in S:
                continue
            if not (row[s] > row[u] or (row[s] == row[u] and s < u)):
                return False
    return True


def test_topk_definition_property_and_format():
    r = rng(15)
    R, N, k = 12, 40, 7
    sc = np.round(r.standard_normal((R, N)), 1)           # many exact ties
    sc[3, 5:] = -np.inf
    sc[4, :] = -np.inf
    sc[5, ::3] = np.nan
    idx, cnt = O.topk(sc, k)
    for i in range(R):
        assert _valid_topk(sc[i], idx[i], k)
        c = cnt[i]
        assert np.all(idx[i, c:] == -1)
        assert np.all(np.diff(idx[i, :c]) > 0)            # ascending
    assert cnt[3] == 5 and cnt[4] == 0


def test_topk_constant_row_takes_lowest_indices():
    idx, cnt = O.topk(np.ones((1, 10)), 4)
    assert list(idx[0]) == [0, 1, 2, 3] and cnt[0] == 4


def test_topk_k_ge_visible_takes_all():
    sc = np.array([[3.0, -np.inf, 1.0, 2.0]])
    idx, cnt = O.topk(sc, 6)
    assert list(idx[0]) == [0, 2, 3, -1, -1, -1] and cnt[0] == 3


# --------------------------------------------------------------------------- MQA


def _mqa_inputs(seed, Tq=3, H=4, D=16, N=10, K=5, Tw=40):
    r = rng(seed)
    q = r.standard_normal((Tq, H, D))
    kv = r.standard_normal((N, D))
    win = r.standard_normal((Tw, D))
    pos = np.array([60, 70, 79])[:Tq]
    sel = np.stack([r.choice(N, K, replace=False) for _ in range(Tq)])
    sink = r.standard_normal(H)
    return q, pos, kv, sel, win, sink


def test_mqa_sink_minus_inf_weights_sum_to_one():
    q, pos, kv, sel, win, _ = _mqa_inputs(20)
    ones_kv = np.ones_like(kv)
    ones_win = np.ones_like(win)
    out = O.mqa(q, pos, ones_kv, sel, ones_win, 40, 8, np.full(4, -np.inf), scale=0.3,
                rope_dims=0, rope_base=RB)
    assert np.allclose(out, 1.0, rtol=1e-13)


def test_mqa_sink_plus_inf_gives_zero():
    q, pos, kv, sel, win, _ = _mqa_inputs(21)
    out = O.mqa(q, pos, kv, sel, win, 40, 8, np.full(4, np.inf), scale=0.3, rope_dims=8, rope_base=RB)
    assert np.all(out == 0.0)


def test_mqa_single_key_closed_form():
    # window of one position and no selected entry: one key, the query's own raw row
    q, pos, kv, _, win, sink = _mqa_inputs(22)
    sel = np.full((3, 2), -1)
    out = O.mqa(q, pos, kv, sel, win, 40, 1, sink, scale=0.25, rope_dims=8, rope_base=RB)
    for t in range(3):
        raw = win[pos[t] - 40]
        for h in range(4):
            z = 0.25 * (q[t, h] @ raw)      # rotation preserves the dot product at equal positions
            g = 1.0 / (1.0 + math.exp(sink[h] - z))
            assert np.allclose(out[t, h], g * raw, rtol=1e-11, atol=1e-13)


def test_mqa_sink_is_extra_zero_value_column_library_softmax():
    q, pos, kv, sel, win, sink = _mqa_inputs(23)
    scale = 0.2
    out = O.mqa(q, pos, kv, sel, win, 40, 6, sink, scale=scale, rope_dims=0, rope_base=RB)
    for t in range(3):
        keys = np.concatenate([kv[sel[t]], win[pos[t] - 5 - 40:pos[t] + 1 - 40]])
        z = scale * q[t] @ keys.T
        full = np.concatenate([z, sink[:, None]], axis=1)
        p = scipy.special.softmax(full, axis=1)
        vals = np.concatenate([keys, np.zeros((1, keys.shape[1]))])
        assert np.allclose(out[t], p @ vals, rtol=1e-11, atol=1e-14)


def test_mqa_output_is_inverse_rotated():
    # with all keys equal to one roped vector, the output is that key rotated back by -t
    q, pos, kv, sel, win, _ = _mqa_inputs(24)
    D, R = 16, 8
    v = rng(0).standard_normal(D)
    t = pos[0]
    keyvec = O.rope(v, 5000, R, RB)
    kv2 = np.tile(keyvec, (kv.shape[0], 1))
    sel2 = sel[:1]
    # window keys roped at their own positions would differ: use a 1-row window whose
    # raw row is chosen so that RoPE(raw, t) == keyvec
    win2 = np.tile(O.rope(keyvec, -t, R, RB), (win.shape[0], 1))
    out = O.mqa(q[:1], pos[:1], kv2, sel2, win2, 40, 1, np.full(4, -np.inf), scale=0.3,
                rope_dims=R, rope_base=RB)
    assert np.allclose(out[0], np.tile(O.rope(keyvec, -t, R, RB), (4, 1)), atol=1e-12)


def test_hca_dense_equals_mqa_over_all_visible():
    q, pos, kv, _, win, sink = _mqa_inputs(25, N=30)
    ratio = 4
    out = O.hca_dense(q, pos, kv, win, 40, 8, sink, ratio=ratio, scale=0.3, rope_dims=8, rope_base=RB)
    for t in range(3):
        v = min(30, pos[t] // ratio)
        sel = np.arange(v)[None, :]
        o = O.mqa(q[t:t + 1], pos[t:t + 1], kv, sel, win, 40, 8, sink, scale=0.3, rope_dims=8,
                  rope_base=RB)
        assert np.allclose(out[t], o[0], rtol=1e-13)


# ------------------------------------------------------------------ whole layer


def _layer_inputs(seed, T=64, D=16, DI=8, H=4, HI=2, Tq=8):
    r = rng(seed)
    streams = [r.standard_normal((T, D)) for _ in range(4)]
    istreams = [r.standard_normal((T, DI)) for _ in range(4)]
    q = r.standard_normal((Tq, H, D)) / math.sqrt(D)
    qI = r.standard_normal((Tq, HI, DI)) / math.sqrt(DI)
    wI = r.uniform(0, 1, (Tq, HI))
    win = r.standard_normal((T, D))
    sink = r.standard_normal(H)
    pos = np.arange(T - Tq, T)
    return streams, istreams, q, pos, qI, wI, win, sink


def test_layer_shift_invariance():
    ins = _layer_inputs(30)
    kw = dict(ratio=4, k=5, n_win=8, scale=1.0, rope_dims=8, rope_base=RB)
    a = O.csa_layer(*ins[:7], 0, ins[7], pos_offset=0, dtype="f32", **kw)
    b = O.csa_layer(*ins[:7], 0, ins[7], pos_offset=12345, dtype="f32", **kw)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.allclose(a["out"], b["out"], rtol=1e-5, atol=1e-7)


def test_layer_topk_ge_visible_equals_dense():
    streams, istreams, q, pos, qI, wI, win, sink = _layer_inputs(31)
    kw = dict(n_win=8, scale=1.0, rope_dims=8, rope_base=RB)
    a = O.csa_layer(streams, istreams, q, pos, qI, wI, win, 0, sink, ratio=4, k=64, dtype="f32", **kw)
    d = O.hca_dense(q, pos, a["kv"], win, 0, 8, sink, ratio=4, scale=1.0, rope_dims=8, rope_base=RB)
    assert np.allclose(a["out"], O.store(d, "f32"), rtol=1e-6)


def test_visible_set_sizes_printed_on_the_pages():
    # [NOTES] visible-set model: at n = 2^20, CSA chooses from 262,144 compressed
    # candidates (m = 4) and HCA attends to 8,192 entries (m' = 128)
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "visible_set.json")))
    n = g["n_tokens"]
    assert O.visible_count(n, g["m"], 10 ** 9) == g["csa_candidates"]
    assert O.visible_count(n, g["m_prime"], 10 ** 9) == g["hca_entries"]
    assert min(g["topk"], O.visible_count(n, g["m"], 10 ** 9)) + g["n_win"] == g["csa_visible"]


# ------------------------------------------------------------------ HCA layer pins


def _hca_inputs(seed, T=48, D=12, H=3, Tq=5):
    r = rng(seed)
    C_ = r.standard_normal((T, D))
    Z = r.standard_normal((T, D))
    q = r.standard_normal((Tq, H, D)) / math.sqrt(D)
    win = r.standard_normal((T, D))
    sink = r.standard_normal(H)
    pos = np.array([3, 17, 30, 41, T - 1])[:Tq]
    return (C_, Z), q, pos, win, sink


def test_hca_layer_shift_invariance():
    # every key and the query carry RoPE at their own position, so a uniform shift of
    # the positions leaves the output unchanged; entries left un-roped would break this
    streams, q, pos, win, sink = _hca_inputs(40)
    kw = dict(ratio=8, n_win=6, scale=0.7, rope_dims=8, rope_base=RB, dtype="f32")
    a = O.hca_layer(streams, q, pos, win, 0, sink, pos_offset=0, **kw)
    b = O.hca_layer(streams, q, pos, win, 0, sink, pos_offset=98765, **kw)
    assert np.allclose(a["out"], b["out"], rtol=1e-5, atol=1e-7)
    c = O.hca_layer(streams, q, pos, win, 0, sink, pos_offset=0, ratio=8, n_win=6, scale=0.7, rope_dims=0,
                    rope_base=RB, dtype="f32")
    assert not np.allclose(a["out"], c["out"], atol=1e-3)   # the RoPE dims do matter here


def test_hca_layer_constant_stream_reproduces_constant():
    # weights sum to 1 in the compressor and in the attention: a constant C and a
    # constant window give that constant at every query and head (no RoPE, no sink term)
    streams, q, pos, win, _ = _hca_inputs(41)
    c = rng(5).standard_normal(12)
    Cc = np.tile(c, (48, 1))
    out = O.hca_layer((Cc, streams[1]), q, pos, np.tile(c, (48, 1)), 0, np.full(3, -np.inf), ratio=8, n_win=6,
                      scale=1.3, rope_dims=0, rope_base=RB, dtype="f32")
    assert np.allclose(out["kv"], np.tile(c, (6, 1)), rtol=1e-6)
    assert np.allclose(out["out"], np.tile(c, (5, 3, 1)), rtol=1e-6)


def test_hca_layer_bf16_storage_points():
    # with bf16 storage, the cached entries and the output are bf16 values (the device
    # stores both), and they differ from the fp32-stored run by at most a few bf16 steps
    streams, q, pos, win, sink = _hca_inputs(42)
    kw = dict(ratio=8, n_win=6, scale=1.0, rope_dims=8, rope_base=RB)
    a = O.hca_layer(streams, q, pos, win, 0, sink, dtype="bf16", **kw)
    b = O.hca_layer(streams, q, pos, win, 0, sink, dtype="f32", **kw)
    for x in (a["kv"], a["out"]):
        bits = np.asarray(x, dtype=np.float32).view(np.uint32)
        assert np.all(bits & 0xFFFF == 0), "values are not bf16-representable"
    assert not np.array_equal(a["kv"], b["kv"])
    assert np.allclose(a["kv"], b["kv"], rtol=2 ** -8, atol=0)
    assert np.allclose(a["out"], b["out"], rtol=2e-2, atol=2e-2)


def _scalar_rope(v, p, R, base):
    v = [float(x) for x in v]
    D = len(v)
    for j in range(R // 2):
        a = p * base ** (-2.0 * j / R)
        x0, x1 = v[D - R + 2 * j], v[D - R + 2 * j + 1]
        v[D - R + 2 * j] = x0 * math.cos(a) - x1 * math.sin(a)
        v[D - R + 2 * j + 1] = x0 * math.sin(a) + x1 * math.cos(a)
    return v


def _scalar_attend(qv, keys, sink, scale):
    z = [scale * sum(a * b for a, b in zip(qv, k)) for k in keys]
    M = max(z + [sink])
    e = [math.exp(x - M) for x in z]
    den = sum(e) + math.exp(sink - M)
    return [sum(e[j] * keys[j][d] for j in range(len(keys))) / den for d in range(len(qv))]


def test_hca_layer_scalar_brute_force():
    # the whole layer written with scalar loops: per-channel softmax over each block's
    # rows, entry i roped at ratio*i, query t sees entries i < t // ratio and the raw
    # tokens t-n_win+1 .. t (roped at their positions), one softmax with the sink,
    # output rotated back by -t
    (C_, Z), q, pos, win, sink = _hca_inputs(43, T=32, D=8, H=2, Tq=4)
    pos = np.array([0, 7, 20, 31])
    ratio, n_win, R, scale = 4, 5, 4, 0.9
    T, D = C_.shape
    ents = []
    for i in range(T // ratio):
        e = []
        for d in range(D):
            lg = [Z[ratio * i + j, d] for j in range(ratio)]
            mx = max(lg)
            w = [math.exp(x - mx) for x in lg]
            e.append(sum(w[j] * C_[ratio * i + j, d] for j in range(ratio)) / sum(w))
        ents.append(_scalar_rope(e, ratio * i, R, RB))
    want = np.zeros(q.shape)
    for t, p in enumerate(pos):
        keys = ents[:p // ratio] + [_scalar_rope(win[r], r, R, RB) for r in range(max(0, p - n_win + 1), p + 1)]
        for h in range(q.shape[1]):
            o = _scalar_attend(_scalar_rope(q[t, h], p, R, RB), keys, sink[h], scale)
            want[t, h] = _scalar_rope(o, -p, R, RB)
    got = O.hca_layer((C_, Z), q, pos, win, 0, sink, ratio=ratio, n_win=n_win, scale=scale, rope_dims=R,
                      rope_base=RB, dtype="f32")
    assert np.allclose(got["kv"], O.store(np.array(ents), "f32"), rtol=1e-6, atol=1e-7)
    assert np.allclose(got["out"], O.store(want, "f32"), rtol=1e-6, atol=1e-7)


def test_csa_layer_scalar_brute_force():
    # the CSA layer with scalar loops: overlapped compression (entry 0 without a
    # previous block), scores over earlier blocks, top-k by sorting (ties to the lower
    # index), attention over the selection and the window with the sink
    streams, istreams, q, pos, qI, wI, win, sink = _layer_inputs(44, T=32, D=8, DI=4, H=2, HI=2, Tq=4)
    pos = np.array([2, 9, 22, 31])
    ratio, k, n_win, R, scale = 4, 3, 5, 4, 0.8
    T = 32

    def comp(Ca, Cb, Za, Zb, rope_R):
        out = []
        for i in range(T // ratio):
            e = []
            for d in range(Ca.shape[1]):
                rows = [(Za[ratio * i + j, d], Ca[ratio * i + j, d]) for j in range(ratio)]
                if i > 0:
                    rows += [(Zb[ratio * (i - 1) + j, d], Cb[ratio * (i - 1) + j, d]) for j in range(ratio)]
                mx = max(z for z, _ in rows)
                w = [math.exp(z - mx) for z, _ in rows]
                e.append(sum(wi * c for wi, (_, c) in zip(w, rows)) / sum(w))
            out.append(_scalar_rope(e, ratio * i, rope_R, RB) if rope_R else e)
        return out
    kv = comp(*streams, R)
    ik = comp(*istreams, 0)
    want = np.zeros(q.shape)
    for t, p in enumerate(pos):
        vis = p // ratio
        sc = [sum(wI[t, h] * max(0.0, sum(a * b for a, b in zip(qI[t, h], ik[s]))) for h in range(2))
              for s in range(vis)]
        chosen = sorted(sorted(range(vis), key=lambda s: (-sc[s], s))[:k])
        keys = [kv[s] for s in chosen] + [_scalar_rope(win[r], r, R, RB) for r in range(max(0, p - n_win + 1), p + 1)]
        for h in range(2):
            o = _scalar_attend(_scalar_rope(q[t, h], p, R, RB), keys, sink[h], scale)
            want[t, h] = _scalar_rope(o, -p, R, RB)
    got = O.csa_layer(streams, istreams, q, pos, qI, wI, win, 0, sink, ratio=ratio, k=k, n_win=n_win, scale=scale,
                      rope_dims=R, rope_base=RB, dtype="f32")
    assert np.allclose(got["out"], O.store(want, "f32"), rtol=1e-6, atol=1e-7)


# ------------------------------------------------------------- RMSNorm pins


def test_rmsnorm_closed_forms_and_brute_force():
    w = rng(60).standard_normal(12)
    for c in (3.5, -0.25):
        # a constant vector normalizes to its sign times the weight (eps = 0)
        assert np.allclose(O.rmsnorm(np.full(12, c), w, 0.0), np.sign(c) * w, rtol=1e-14)
    x = rng(61).standard_normal((4, 12))
    y = O.rmsnorm(x, np.ones(12), 0.0)
    assert np.allclose(np.sqrt(np.mean(y * y, axis=-1)), 1.0, rtol=1e-14)          # unit RMS
    assert np.allclose(O.rmsnorm(7.0 * x, w, 0.0), O.rmsnorm(x, w, 0.0), rtol=1e-13)  # scale invariance
    onehot = np.zeros(12)
    onehot[5] = 2.0
    z = O.rmsnorm(x, onehot, 0.0)
    assert np.all(z[:, np.arange(12) != 5] == 0) and np.all(z[:, 5] != 0)          # per-dim weight
    eps = 1e-3
    for r in range(4):
        ms = sum(float(v) * float(v) for v in x[r]) / 12
        want = [float(x[r, d]) / math.sqrt(ms + eps) * float(w[d]) for d in range(12)]
        assert np.allclose(O.rmsnorm(x[r], w, eps), want, rtol=1e-13)


def test_compress_with_norm_normalizes_before_rope():
    r = rng(62)
    T, D, R, ratio = 32, 16, 8, 4
    v = r.standard_normal(D)
    Cc = np.tile(v, (T, 1))
    Zs = [r.standard_normal((T, D)) for _ in range(2)]
    w = r.uniform(0.5, 1.5, D)
    # constant rows: every entry is v, normalized; no RoPE gives the closed form
    e = O.compress(Cc, Cc, Zs[0], Zs[1], ratio=ratio, overlap=True, rope_dims=0, norm_weight=w, norm_eps=1e-5)
    want = v / math.sqrt(float(np.mean(v * v)) + 1e-5) * w
    assert np.allclose(e, np.tile(want, (T // ratio, 1)), rtol=1e-12)
    # with RoPE and unit weights (eps = 0) every entry has unit RMS: the norm comes
    # first and the rotation keeps pair norms
    C2 = [r.standard_normal((T, D)) for _ in range(2)]
    e2 = O.compress(C2[0], C2[1], Zs[0], Zs[1], ratio=ratio, overlap=True, rope_dims=R, rope_base=RB,
                    norm_weight=np.ones(D), norm_eps=0.0)
    assert np.allclose(np.sqrt(np.mean(e2 * e2, axis=-1)), 1.0, rtol=1e-12)
    # and equals RoPE of the normalized un-roped entries; with uneven weights the order
    # matters (the weights of a rotated pair differ), and the norm comes first
    e3 = O.compress(C2[0], C2[1], Zs[0], Zs[1], ratio=ratio, overlap=True, rope_dims=0)
    pos = ratio * np.arange(T // ratio)
    assert np.allclose(e2, O.rope(O.rmsnorm(e3, np.ones(D), 0.0), pos, R, RB), rtol=1e-12, atol=1e-14)
    e4 = O.compress(C2[0], C2[1], Zs[0], Zs[1], ratio=ratio, overlap=True, rope_dims=R, rope_base=RB,
                    norm_weight=w, norm_eps=1e-5)
    assert np.allclose(e4, O.rope(O.rmsnorm(e3, w, 1e-5), pos, R, RB), rtol=1e-12, atol=1e-14)
    assert not np.allclose(e4, O.rmsnorm(O.rope(e3, pos, R, RB), w, 1e-5), rtol=1e-6)


def test_mqa_norms_make_output_scale_invariant():
    q, pos, kv, sel, win, sink = _mqa_inputs(63)
    D = q.shape[-1]
    qn, kn = rng(64).uniform(0.5, 1.5, D), rng(65).uniform(0.5, 1.5, D)
    kw = dict(scale=0.3, rope_dims=8, rope_base=RB, q_norm=qn, kv_norm=kn, norm_eps=0.0)
    a = O.mqa(q, pos, kv, sel, win, 40, 6, sink, **kw)
    b = O.mqa(5.0 * q, pos, kv, sel, 0.2 * win, 40, 6, sink, **kw)   # scaled queries and raw window rows
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)
    c = O.mqa(5.0 * q, pos, kv, sel, win, 40, 6, sink, scale=0.3, rope_dims=8, rope_base=RB)
    d = O.mqa(q, pos, kv, sel, win, 40, 6, sink, scale=0.3, rope_dims=8, rope_base=RB)
    assert not np.allclose(c, d)   # without the norms the scale does matter


def test_layer_norms_equal_normalized_inputs():
    # the layer with KV norm = the layer without it on pre-normalized window rows and
    # entries (checked through the cache it returns), and q norm = normalized queries
    streams, istreams, q, pos, qI, wI, win, sink = _layer_inputs(66)
    D = q.shape[-1]
    qn, kn = rng(67).uniform(0.5, 1.5, D), rng(68).uniform(0.5, 1.5, D)
    kw = dict(ratio=4, k=5, n_win=8, scale=1.0, rope_dims=8, rope_base=RB, dtype="f32")
    a = O.csa_layer(streams, istreams, q, pos, qI, wI, win, 0, sink, q_norm=qn, kv_norm=kn, norm_eps=1e-6, **kw)
    b = O.csa_layer(streams, istreams, O.rmsnorm(q, qn, 1e-6), pos, qI, wI, O.rmsnorm(win, kn, 1e-6), 0, sink, **kw)
    e = O.compress(*streams, ratio=4, overlap=True, rope_dims=8, rope_base=RB, norm_weight=kn, norm_eps=1e-6)
    assert np.allclose(a["kv"], O.store(e, "f32"))
    assert np.array_equal(a["idx"], b["idx"])
    # b's entries are not normalized: compare the attention over a's entries
    o = O.mqa(O.rmsnorm(q, qn, 1e-6), pos, a["kv"], a["idx"], O.rmsnorm(win, kn, 1e-6), 0, 8, sink, scale=1.0,
              rope_dims=8, rope_base=RB)
    assert np.allclose(a["out"], O.store(o, "f32"), rtol=1e-6, atol=1e-7)


# ------------------------------------------------- grouped output projection pins


def test_grouped_out_proj_identity_groups_and_brute_force():
    r = rng(70)
    T, n_h, c, g = 3, 8, 4, 4
    per = n_h // g
    o = r.standard_normal((T, n_h, c))
    # identity group weights and identity output weights give the flattened outputs
    wg = np.stack([np.eye(per * c) for _ in range(g)])
    assert np.allclose(O.grouped_out_proj(o, wg, np.eye(g * per * c), dtype="f32"),
                       O.store(o.reshape(T, n_h * c), "f32"), rtol=0, atol=0)
    # group j depends on heads j*per .. j*per+per-1 only
    d_g, d = 5, 6
    wg = r.standard_normal((g, d_g, per * c))
    wo = r.standard_normal((d, g * d_g))
    mid_only = O.grouped_out_proj(o, wg, np.eye(g * d_g), dtype="f32")
    o2 = o.copy()
    o2[:, per:2 * per] = 0.0
    mid2 = O.grouped_out_proj(o2, wg, np.eye(g * d_g), dtype="f32")
    assert np.all(mid2[:, d_g:2 * d_g] == 0) and np.array_equal(mid2[:, :d_g], mid_only[:, :d_g])
    # scalar brute force
    got = O.grouped_out_proj(o, wg, wo, dtype="f32")
    for t in range(T):
        mid = []
        for j in range(g):
            flat = [float(o[t, h, k]) for h in range(j * per, (j + 1) * per) for k in range(c)]
            mid += [float(np.float32(sum(wg[j, i, m] * flat[m] for m in range(per * c)))) for i in range(d_g)]
        want = [sum(wo[i, m] * mid[m] for m in range(g * d_g)) for i in range(d)]
        assert np.allclose(got[t], want, rtol=1e-12, atol=1e-12)
    # linear in the outputs
    o3 = r.standard_normal((T, n_h, c))
    lin = O.grouped_out_proj(2.0 * o - 3.0 * o3, wg, wo, dtype="f32")
    assert np.allclose(lin, 2.0 * got - 3.0 * O.grouped_out_proj(o3, wg, wo, dtype="f32"), rtol=1e-5, atol=1e-5)
