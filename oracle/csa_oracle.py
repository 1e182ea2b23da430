"""fp64 CPU oracle of the CSA / HCA attention forward (TEST INFRASTRUCTURE ONLY).

Each function is the plain definition from the pages, written out with NumPy in
float64 and per-sequence loops, with no blocking, fusion or reordering beyond what
the definition states.  Sources (see ``oracle/__init__.py`` for the page list):

* ``compress``      -- [V4-CN] §2.3.1, the two compression equations (CSA, overlap of
  the current block's a-branch with the previous block's b-branch) and §2.3.2
  (HCA, one block, no overlap); [NOTES] "关键设计 1" states the weights are per
  dimension, so the softmax runs across the 2m (or m') positions of each channel.
* ``rope``          -- [V4-CN] §2.3.3: RoPE on the last 64 dims of queries and KV
  entries; output rotated back by the query position.  Pairing and frequencies
  follow the RoFormer form (adjacent pairs, theta_j = base^(-2j/R)).
* ``index_scores``  -- [V4-CN] §2.3.1, lightning indexer score equation, with the
  block-causal visibility of §2.3.3 (a query sees only earlier compressed blocks).
* ``topk``          -- [V4-CN] §2.3.1 (top-k selector) / [NOTES] "关键设计 1"
  (C_t = TopK_k(I_t,:)).
* ``mqa``           -- [V4-CN] §2.3.1 (shared-KV MQA: an entry is both key and
  value), §2.3.3 (sliding-window branch whose raw KV entries join the compressed
  ones in the core attention, attention sink denominator, inverse RoPE).
* ``hca_dense``     -- [V4-CN] §2.3.2 and [NOTES] "关键设计 2": dense attention over
  every visible compressed entry plus the window.
* ``csa_layer`` / ``hca_layer`` -- one layer of one sequence composed from the
  definitions above ([V4-CN] §2.3.1-§2.3.3): compressed entries, each query's
  selected (CSA) or visible (HCA) entries, its window keys, one softmax with the
  sink, the output rotated back.

Readings where the pages are silent or garbled:
softmax axis = positions (per channel); entry 0 has no previous block (b-branch
empty); compressed entry i sits at RoPE position ratio*i; entry i is visible to the
query at t iff i < floor(t/ratio); the window is positions max(0,t-n_win+1)..t,
roped at their own positions, in one softmax with the entries; inverse RoPE uses
-t; the sink logit is not scaled; ties in top-k go to the lower index, output is
ascending and padded with -1; pos_offset shifts every RoPE position (only).

Parity: every function is pinned by tests/test_oracle_*.py (closed forms,
invariants, brute force, library routines); none is "parity unpinned".  The layer
compositions are pinned by shift invariance, constant streams, the bf16 storage
points, the equality of CSA with k >= visible and dense attention, and scalar-loop
brute force of both layers on tiny inputs.
"""

from __future__ import annotations

import numpy as np

from . import quant

# ------------------------------------------------------------------------- RoPE


def rope(x, pos, rope_dims: int, base: float) -> np.ndarray:
    """Rotate the last ``rope_dims`` dims of x[..., D] by position ``pos``.

    Pair j (j = 0..R/2-1) is (x[D-R+2j], x[D-R+2j+1]), rotated by angle
    pos * base^(-2j/R).  ``pos`` broadcasts against x.shape[:-1].  RoPE(x, -p)
    is the inverse of RoPE(x, p).
    """
    x = np.array(x, dtype=np.float64, copy=True)
    if rope_dims == 0:
        return x
    D = x.shape[-1]
    R = rope_dims
    j = np.arange(R // 2, dtype=np.float64)
    theta = base ** (-2.0 * j / R)
    p = np.asarray(pos, dtype=np.float64)[..., None]
    ang = p * theta
    c, s = np.cos(ang), np.sin(ang)
    even = x[..., D - R::2].copy()
    odd = x[..., D - R + 1::2].copy()
    x[..., D - R::2] = even * c - odd * s
    x[..., D - R + 1::2] = even * s + odd * c
    return x


# ---------------------------------------------------------------------- RMSNorm


def rmsnorm(x, weight, eps: float) -> np.ndarray:
    """RMSNorm over the last dim: x / sqrt(mean(x^2) + eps) * weight.

    [V4-CN] §2.3.3 (query and KV normalization): before core attention every query
    head and the single head of the compressed KV entries get an RMSNorm; the pages
    name the learnable weights (trained with AdamW, §2.4) but not eps."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * w


# --------------------------------------------------------------------- compress


def compress(ca, cb, za, zb, *, ratio: int, overlap: bool, t0: int = 0,
             prev_cb=None, prev_zb=None, bias_a=None, bias_b=None,
             rope_dims: int = 0, rope_base: float = 10000.0, pos_offset: int = 0,
             entries=None, norm_weight=None, norm_eps: float = 1e-6) -> np.ndarray:
    """Compressed entries of one sequence.

    ca, za: [T, D] a-branch values / weights of tokens t0..t0+T-1 (for HCA, C and Z).
    cb, zb: [T, D] b-branch (CSA only; ignored when overlap is False).
    prev_cb, prev_zb: [ratio, D] b-branch rows of the block just before t0 (CSA,
      t0 > 0); when t0 == 0 the first entry has no previous block.
    bias_a, bias_b: [ratio, D] learnable additive biases (None = 0).
    entries: local entry indices to compute (default: all T // ratio).

    Entry with absolute index I = t0/ratio + i:
      logits  = [Z^a rows of block I + B^a ; Z^b rows of block I-1 + B^b]  (per channel)
      weights = softmax of the logits over the positions (per channel)
      e       = sum(weights * [C^a rows of block I ; C^b rows of block I-1])
    then (with ``norm_weight``) the entry's RMSNorm, then RoPE on the last ``rope_dims``
    dims at position pos_offset + ratio*I.
    """
    ca = np.asarray(ca, dtype=np.float64)
    za = np.asarray(za, dtype=np.float64)
    T, D = ca.shape
    assert t0 % ratio == 0
    n = T // ratio
    if entries is None:
        entries = range(n)
    ba = np.zeros((ratio, D)) if bias_a is None else np.asarray(bias_a, dtype=np.float64)
    bb = np.zeros((ratio, D)) if bias_b is None else np.asarray(bias_b, dtype=np.float64)
    if overlap:
        cb = np.asarray(cb, dtype=np.float64)
        zb = np.asarray(zb, dtype=np.float64)
    out = []
    for i in entries:
        I = t0 // ratio + i
        vals = [ca[ratio * i: ratio * (i + 1)]]
        logits = [za[ratio * i: ratio * (i + 1)] + ba]
        if overlap:
            if i >= 1:
                vals.append(cb[ratio * (i - 1): ratio * i])
                logits.append(zb[ratio * (i - 1): ratio * i] + bb)
            elif I >= 1:
                assert prev_cb is not None and prev_zb is not None, \
                    "a CSA chunk starting after token 0 needs the previous block"
                vals.append(np.asarray(prev_cb, dtype=np.float64))
                logits.append(np.asarray(prev_zb, dtype=np.float64) + bb)
            # I == 0: no previous block, the b-branch is empty
        v = np.concatenate(vals, axis=0)          # [2m or m, D]
        lg = np.concatenate(logits, axis=0)       # [2m or m, D]
        w = np.exp(lg - lg.max(axis=0, keepdims=True))
        w = w / w.sum(axis=0, keepdims=True)
        e = (w * v).sum(axis=0)
        if norm_weight is not None:
            e = rmsnorm(e, norm_weight, norm_eps)
        out.append(rope(e, pos_offset + ratio * I, rope_dims, rope_base))
    if not out:
        return np.zeros((0, D))
    return np.stack(out, axis=0)


# ------------------------------------------------------------------ index scores


def visible_count(t: int, ratio: int, N: int) -> int:
    """Number of compressed entries visible to the query at absolute position t."""
    return max(0, min(N, t // ratio))


def index_scores(qI, wI, kI, q_pos, ratio: int) -> np.ndarray:
    """Lightning-indexer scores of one sequence.

    qI [Tq, HI, DI], wI [Tq, HI], kI [N, DI], q_pos [Tq] -> I [Tq, N] (float64),
    I[t, s] = sum_h wI[t,h] * max(0, qI[t,h] . kI[s]) for s < floor(pos_t/ratio),
    -inf for entries the query cannot see.
    """
    qI = np.asarray(qI, dtype=np.float64)
    wI = np.asarray(wI, dtype=np.float64)
    kI = np.asarray(kI, dtype=np.float64)
    Tq = qI.shape[0]
    N = kI.shape[0]
    out = np.full((Tq, N), -np.inf)
    for t in range(Tq):
        v = visible_count(int(q_pos[t]), ratio, N)
        if v == 0:
            continue
        dots = qI[t] @ kI[:v].T                     # [HI, v]
        out[t, :v] = wI[t] @ np.maximum(dots, 0.0)  # sum over heads
    return out


# ------------------------------------------------------------------------- top-k


def topk(scores, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Top-k selector over rows of scores [R, N].

    Selects the min(k, #finite) largest finite scores of each row; equal scores
    are taken in increasing index order.  Returns (idx int32 [R, k] ascending,
    padded with -1; count int32 [R]).
    """
    s = np.asarray(scores, dtype=np.float64)
    R, N = s.shape
    idx = np.full((R, k), -1, dtype=np.int32)
    cnt = np.zeros(R, dtype=np.int32)
    for r in range(R):
        cand = np.nonzero(np.isfinite(s[r]))[0]
        # primary key: score descending; secondary: index ascending
        order = cand[np.lexsort((cand, -s[r, cand]))]
        take = np.sort(order[:k])
        idx[r, :take.size] = take
        cnt[r] = take.size
    return idx, cnt


# --------------------------------------------------------------------------- MQA


def _attend_one(qr, keys, sink: float, scale: float) -> np.ndarray:
    """Attention of query heads qr [H, D] over shared keys=values [n, D] with a sink.

    weight_j = exp(z_j) / (sum_k exp(z_k) + exp(sink_h)), z = scale * q.k;
    sink = -inf drops the sink term, sink = +inf gives a zero output.
    """
    H, D = qr.shape
    z = scale * (qr @ keys.T)                        # [H, n]
    sink = np.broadcast_to(np.asarray(sink, dtype=np.float64), (H,))
    out = np.zeros((H, D))
    for h in range(H):
        if np.isposinf(sink[h]):
            continue
        zh = z[h]
        if np.isneginf(sink[h]):
            M = zh.max()
            e = np.exp(zh - M)
            denom = e.sum()
        else:
            M = max(zh.max(), sink[h]) if zh.size else sink[h]
            e = np.exp(zh - M)
            denom = e.sum() + np.exp(sink[h] - M)
        out[h] = (e @ keys) / denom
    return out


def window_positions(t: int, n_win: int) -> np.ndarray:
    return np.arange(max(0, t - n_win + 1), t + 1)


def mqa(q, q_pos, kv, sel, win, win_pos0: int, n_win: int, sink, *, scale: float,
        rope_dims: int, rope_base: float, pos_offset: int = 0, q_norm=None, kv_norm=None,
        norm_eps: float = 1e-6) -> np.ndarray:
    """Shared-KV MQA of one sequence over selected entries plus the raw window.

    q [Tq, H, D] (not roped), q_pos [Tq], kv [N, D] compressed entries (already
    roped), sel [Tq, K] entry indices (-1 = unused slot), win [Tw, D] raw entries
    (not roped) for absolute positions win_pos0 .. win_pos0+Tw-1, sink [H].
    With ``q_norm`` every query head, with ``kv_norm`` every raw window entry gets its
    RMSNorm before RoPE (the compressed entries carry theirs from the compressor).
    Returns out [Tq, H, D].
    """
    q = np.asarray(q, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    win = np.asarray(win, dtype=np.float64)
    if q_norm is not None:
        q = rmsnorm(q, q_norm, norm_eps)
    if kv_norm is not None:
        win = rmsnorm(win, kv_norm, norm_eps)
    sink = np.asarray(sink, dtype=np.float64)
    Tq, H, D = q.shape
    out = np.zeros((Tq, H, D))
    for t in range(Tq):
        pt = int(q_pos[t])
        chosen = [int(s) for s in np.asarray(sel[t]) if s >= 0]
        wpos = window_positions(pt, n_win)
        rows = wpos - win_pos0
        assert rows.min() >= 0 and rows.max() < win.shape[0], "window buffer too short"
        wkeys = rope(win[rows], wpos + pos_offset, rope_dims, rope_base)
        keys = np.concatenate([kv[chosen].reshape(-1, D), wkeys], axis=0)
        qr = rope(q[t], pos_offset + pt, rope_dims, rope_base)
        o = _attend_one(qr, keys, sink, scale)
        out[t] = rope(o, -(pos_offset + pt), rope_dims, rope_base)
    return out


def hca_dense(q, q_pos, kv, win, win_pos0: int, n_win: int, sink, *, ratio: int,
              scale: float, rope_dims: int, rope_base: float,
              pos_offset: int = 0, q_norm=None, kv_norm=None, norm_eps: float = 1e-6) -> np.ndarray:
    """HCA core attention: every visible compressed entry (i < floor(t/ratio)) + window."""
    N = np.asarray(kv).shape[0]
    Tq = np.asarray(q).shape[0]
    sel = np.full((Tq, max(1, N)), -1, dtype=np.int64)
    for t in range(Tq):
        v = visible_count(int(q_pos[t]), ratio, N)
        sel[t, :v] = np.arange(v)
    return mqa(q, q_pos, kv, sel, win, win_pos0, n_win, sink, scale=scale,
               rope_dims=rope_dims, rope_base=rope_base, pos_offset=pos_offset, q_norm=q_norm,
               kv_norm=kv_norm, norm_eps=norm_eps)


# ------------------------------------------------------------------ whole layer


def store(x, dtype: str) -> np.ndarray:
    """Value after storage in dtype ('f32' or 'bf16'), as the GPU stores stage outputs."""
    if dtype == "f32":
        return quant.round_f32(x)
    if dtype == "bf16":
        return quant.round_bf16(x)
    raise ValueError(dtype)


def _window_keys(win, win_pos0: int, p: int, n_win: int, pos_offset: int, rope_dims: int,
                 rope_base: float, kv_norm=None, norm_eps: float = 1e-6) -> np.ndarray:
    """Raw tokens of the sliding window of the query at position p, each (normalized
    and) roped at its own position ([V4-CN] §2.3.3: the last n_win uncompressed tokens,
    the query's own included)."""
    wpos = window_positions(p, n_win)
    rows = np.asarray(win, dtype=np.float64)[wpos - win_pos0]
    if kv_norm is not None:
        rows = rmsnorm(rows, kv_norm, norm_eps)
    return rope(rows, wpos + pos_offset, rope_dims, rope_base)


def _query_output(q_t, p: int, entries, wkeys, sink, scale: float, rope_dims: int, rope_base: float,
                  pos_offset: int, q_norm=None, norm_eps: float = 1e-6) -> np.ndarray:
    """Core attention of one query token ([V4-CN] §2.3.1 shared-KV MQA, §2.3.3): the
    query heads are roped at p, attend to the compressed entries it uses followed by
    its window keys in one softmax with the sink term, and the result is rotated back
    by -p."""
    keys = np.concatenate([entries.reshape(-1, wkeys.shape[1]), wkeys], axis=0)
    if q_norm is not None:
        q_t = rmsnorm(q_t, q_norm, norm_eps)
    o = _attend_one(rope(q_t, p + pos_offset, rope_dims, rope_base), keys, sink, scale)
    return rope(o, -(p + pos_offset), rope_dims, rope_base)


def csa_layer(streams, istreams, q, q_pos, qI, wI, win, win_pos0, sink, *,
              ratio: int, k: int, n_win: int, scale: float, rope_dims: int,
              rope_base: float, pos_offset: int = 0, dtype: str = "f32", q_norm=None,
              kv_norm=None, norm_eps: float = 1e-6):
    """One CSA layer forward of one sequence whose tokens start at position 0.

    From the definitions of [V4-CN] §2.3.1 and §2.3.3:
    * the compressed KV entries are the overlapped compression of the KV streams,
      with partial RoPE at each entry's position; the compressed indexer keys are the
      same compression of the indexer streams, without RoPE;
    * query t's index scores cover the entries it may see (earlier complete blocks),
      and its selected set is the top-k of those scores;
    * query t attends to its selected entries followed by its window's raw tokens,
      in one softmax with the sink term, and its output is rotated back by -t.
    streams = (Ca, Cb, Za, Zb) [T, D]; istreams = indexer-key streams [T, DI].
    Stage outputs are rounded to ``dtype`` where the device stores them
    (compressed KV, compressed indexer keys, final output).  ``q_norm`` / ``kv_norm``:
    RMSNorm weights of the query heads and of the KV entries (compressed and window),
    [V4-CN] §2.3.3; None leaves them unnormalized.
    Returns dict(kv, ik, scores, idx, count, out).
    """
    Ca, Cb, Za, Zb = streams
    kv = store(compress(Ca, Cb, Za, Zb, ratio=ratio, overlap=True, rope_dims=rope_dims,
                        rope_base=rope_base, pos_offset=pos_offset, norm_weight=kv_norm,
                        norm_eps=norm_eps), dtype)
    ICa, ICb, IZa, IZb = istreams
    ik = store(compress(ICa, ICb, IZa, IZb, ratio=ratio, overlap=True), dtype)
    scores = index_scores(qI, wI, ik, q_pos, ratio)
    idx, cnt = topk(scores, k)
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros(q.shape)
    for t in range(q.shape[0]):
        p = int(q_pos[t])
        chosen = idx[t, :cnt[t]]
        wkeys = _window_keys(win, win_pos0, p, n_win, pos_offset, rope_dims, rope_base, kv_norm, norm_eps)
        out[t] = _query_output(q[t], p, kv[chosen], wkeys, sink, scale, rope_dims, rope_base, pos_offset,
                               q_norm, norm_eps)
    return dict(kv=kv, ik=ik, scores=scores, idx=idx, count=cnt, out=store(out, dtype))


def hca_layer(streams, q, q_pos, win, win_pos0, sink, *, ratio: int, n_win: int,
              scale: float, rope_dims: int, rope_base: float, pos_offset: int = 0,
              dtype: str = "f32", q_norm=None, kv_norm=None, norm_eps: float = 1e-6):
    """One HCA layer forward of one sequence whose tokens start at position 0.

    From [V4-CN] §2.3.2 and §2.3.3: the entries are the non-overlapping compression of
    the streams (C, Z) [T, D] over blocks of ``ratio`` tokens, with partial RoPE at each
    entry's position; query t attends to every entry it may see (earlier complete
    blocks) followed by its window's raw tokens, in one softmax with the sink term,
    and its output is rotated back by -t.
    """
    C, Z = streams
    kv = store(compress(C, None, Z, None, ratio=ratio, overlap=False, rope_dims=rope_dims,
                        rope_base=rope_base, pos_offset=pos_offset, norm_weight=kv_norm,
                        norm_eps=norm_eps), dtype)
    q = np.asarray(q, dtype=np.float64)
    out = np.zeros(q.shape)
    for t in range(q.shape[0]):
        p = int(q_pos[t])
        visible = kv[:visible_count(p, ratio, kv.shape[0])]
        wkeys = _window_keys(win, win_pos0, p, n_win, pos_offset, rope_dims, rope_base, kv_norm, norm_eps)
        out[t] = _query_output(q[t], p, visible, wkeys, sink, scale, rope_dims, rope_base, pos_offset,
                               q_norm, norm_eps)
    return dict(kv=kv, out=store(out, dtype))


# ------------------------------------------------------ grouped output projection


def grouped_out_proj(o, w_group, w_out, *, dtype: str = "f32") -> np.ndarray:
    """Grouped output projection of one layer ([V4-CN] §2.3.1; group count g and
    intermediate width d_g in §4.2.1).

    o [T, n_h, c] core-attention outputs; w_group [g, d_g, (n_h / g) * c] and
    w_out [d, g * d_g] weights as [out, in] matrices.  The n_h outputs of a token are
    split into g groups of consecutive heads, group j is projected by w_group[j] to a
    d_g-dim intermediate output, and the concatenated intermediates are projected by
    w_out to d dims.  The intermediate is rounded to ``dtype`` where the device stores
    it; returns [T, d] (not rounded).
    """
    o = np.asarray(o, dtype=np.float64)
    wg = np.asarray(w_group, dtype=np.float64)
    wo = np.asarray(w_out, dtype=np.float64)
    T, n_h, c = o.shape
    g = wg.shape[0]
    per = n_h // g
    mid = np.concatenate([o[:, j * per:(j + 1) * per, :].reshape(T, per * c) @ wg[j].T for j in range(g)], axis=1)
    mid = store(mid, dtype)
    return mid @ wo.T
