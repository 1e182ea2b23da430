#!/usr/bin/env python3
"""Benchmark of the CSA / HCA attention forward on one MI355X.

Default workload (the headline): CSA decode at 128K context.
- B = 16 sequences, 131,072 tokens of context each.
- m = 4, so 32,768 compressed entries per sequence.
- Shared KV dim 512, with the last 64 dims RoPE'd.
- Lightning indexer 64 heads x 128, top-k 1024.
- 128 query heads x 512, window 128, bf16.

A decode step serves one new token per sequence with one csa_forward call: score
every entry, select the top 1024, and attend over them plus the window. Every 4th
step also compresses the newest 4-token block (KV and indexer key, one entry per
sequence), as a decoder does once per block. Steps cycle over --layers copies of
the caches, so the caches are read from HBM rather than the 256 MB Infinity Cache,
as in a multi-layer decode.

Other workloads (--config):
- 2:  CSA chunked prefill, 1M context, the last 2048 tokens as queries.
- 3d: HCA decode, B = 32, 1M context each (8192 entries).
- 3p: HCA 2048-token prefill chunk at 1M context.
- 4:  mixed-precision CSA decode, B = 8, 1M context, FP8-mixed KV cache, MXFP4
      indexer.

Inputs are seeded synthetic tensors (module synth). Caches are built by
csa_compress before timing (config 4: seeded fp32 Gaussians quantized directly).

Prints one JSON line. Stage times are measured with HIP events on the stream the
kernels run on.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from dataclasses import dataclass, field

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12            # B/s, MI355X published
MFMA_BF16_PEAK = 2.5e15      # FLOP/s dense bf16, MI355X published
MFMA_FP4_PEAK = 10.1e15      # FLOP/s dense fp4 / MXFP4
COPY_PROBE_BYTES = 1 << 30   # bytes read (and written) by one copy-probe launch
METRIC = "CSA decode tokens/s @128K ctx; indexer+MQA % MFMA peak, compress/top-k % HBM"

WORKLOAD_TAGS = {"1": "csa_decode_b16_ctx128k", "2": "csa_prefill_t2048_ctx1m", "3d": "hca_decode_b32_ctx1m",
                 "3p": "hca_prefill_t2048_ctx1m", "4": "csa_decode_b8_ctx1m_fp8kv_mxfp4idx"}
WORKLOAD_TAG = WORKLOAD_TAGS["1"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def src_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "compressed_sparse_attention_07_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_file: str, src: str):
    """Measured HBM bytes per launch from a committed PMC summary, if it matches the source."""
    path = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != src or "traffic_bytes_per_launch" not in vals:
        return None
    return float(vals["traffic_bytes_per_launch"])


def read_counters(kernel_file: str, src: str):
    """MFMA-busy and LDS figures per launch from a committed counter summary, if it
    matches the source."""
    path = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#") and not line.startswith(" "):
            k, v = line.strip().split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != src:
        return None
    out = {}
    for k in ("mfma_busy_frac", "lds_bank_conflict_frac", "valu_busy_frac", "sq_busy_cycles_per_launch"):
        if k in vals:
            out[k] = float(vals[k])
    return out or None


# ============================================================================ workloads


@dataclass
class Stage:
    run: object                 # fn(i) launching the stage on layer i % layers
    bytes: float                # algorithmic bytes per launch
    flops: float                # algorithmic FLOP per launch
    kernel: str                 # the kernels one launch of the stage runs, joined by "+"
    peak_flops: float = MFMA_BF16_PEAK


@dataclass
class Workload:
    key: str
    name: str
    cfg: object
    tokens: int                 # query tokens served per step
    desc_full: object           # csa_layer_desc of a step that compresses (T > 0), or None
    desc_attend: object         # csa_layer_desc of a step without compression
    ios: list                   # per layer: csa_forward io dict
    compress_every: int         # 1: every step compresses; 4: every 4th; 0: never
    desc_compress: object = None  # csa_layer_desc of the step's compression only (Tq = 0)
    ws: object = None
    stages: dict = field(default_factory=dict)
    build: dict = field(default_factory=dict)
    meta: dict = field(default_factory=dict)

    calls_full: list = field(default_factory=list)
    calls_attend: list = field(default_factory=list)

    def prepare(self):
        """Marshal every layer's csa_forward arguments once (the timed loop is one C call per step)."""
        import compressed_sparse_attention_07_amd as csa
        self.calls_attend = [csa.ForwardCall(self.desc_attend, io, ws=self.ws) for io in self.ios]
        if self.desc_full is not None:
            self.calls_full = [csa.ForwardCall(self.desc_full, io, ws=self.ws) for io in self.ios]

    def step(self, i):
        full = self.compress_every and (i % self.compress_every == 0)
        (self.calls_full if full else self.calls_attend)[i % len(self.ios)]()


def _copy_buf(dst, src):
    dst.data.copy_(src.data)
    if src.rope is not None:
        dst.rope.copy_(src.rope)
    if src.scale is not None:
        dst.scale.copy_(src.scale)


def _compress_bulk(csa, gens, cache, b0, tokens, D, m, overlap, R, base, bf, timer):
    """Compress tokens [0, tokens) of sequences b0 .. b0 + len(gens) - 1 into cache rows
    [0, tokens/m) with one launch (the sequences form the batch).

    Each sequence's streams are drawn from its own generator, in the same order whatever
    the batching.  The compression is idempotent: a first run touches the freshly
    allocated stream buffers, then the mean of three runs is timed.  Returns (seconds,
    bytes) of one run."""
    import torch
    nb_seq = len(gens)
    n_st = 4 if overlap else 2
    s = [torch.empty((nb_seq, tokens, D), dtype=bf, device="cuda") for _ in range(n_st)]
    for i, g in enumerate(gens):
        for j in range(n_st):
            s[j][i] = g.normal((tokens, D), dtype=bf)
    dst = csa.Buf(cache.dtype, *(None if t is None else t[b0:b0 + nb_seq] for t in (cache.data, cache.rope, cache.scale)))
    kw = dict(ratio=m, overlap=overlap, t0=0, rope_dims=R, rope_base=base)
    if overlap:
        ca, cb, za, zb = s
    else:
        ca, za = s
        cb = zb = None
    call = csa.PreparedCall(csa.csa_compress, ca, cb, za, zb, dst, **kw)
    call()  # first touch of the freshly drawn stream buffers (page-table walks); same result
    t = timer()
    for _ in range(3):
        call()
    secs = timer(t) / 3
    nbytes = nb_seq * (n_st * tokens * D * 2 + (tokens // m) * D * 2)
    del s
    return secs, nbytes


def _event_timer():
    import torch

    def timer(start=None):
        if start is None:
            # keep the GPU busy while the host records the start and enqueues the timed
            # launch, so the interval holds the launch and not the host's enqueue time
            torch.cuda._sleep(200_000)
            e0 = torch.cuda.Event(enable_timing=True)
            e0.record()
            return e0
        e1 = torch.cuda.Event(enable_timing=True)
        e1.record()
        torch.cuda.synchronize()
        return start.elapsed_time(e1) * 1e-3
    return timer


def build_workload(key: str, layers: int, dev: str = "cuda") -> Workload:
    """Inputs, caches and forward descriptors of one workload (see the module docstring)."""
    import torch

    import compressed_sparse_attention_07_amd as csa
    from synth import CONFIGS, Gen, qstd

    bf = torch.bfloat16
    timer = _event_timer()
    cfgid = {"1": 1, "2": 2, "3d": 3, "3p": 3, "4": 4}[key]
    cfg = CONFIGS[cfgid]
    D, R, HI, DI, k, H, W = cfg.D, cfg.R, cfg.HI, cfg.DI, cfg.k, cfg.H, cfg.n_win
    m, ctx, base = cfg.m, cfg.ctx, cfg.rope_base
    hca = cfg.mode == "hca"
    B = {"1": cfg.B, "2": 1, "3d": 32, "3p": 1, "4": cfg.B}[key]
    Tq = {"1": 1, "2": 2048, "3d": 1, "3p": 2048, "4": 1}[key]
    decode = Tq == 1
    L = max(1, layers)
    N = ctx // m
    kv_fmt = csa.CSA_FP8MIX if cfg.kv_format == "fp8mix" else csa.CSA_BF16
    ik_fmt = csa.CSA_MXFP4 if cfg.ik_format == "mxfp4" else csa.CSA_BF16

    # ------------------------------------------------------------------ caches (layer 0)
    kv0 = csa.Buf.empty((B, N, D), kv_fmt, rope_dims=R if kv_fmt == csa.CSA_FP8MIX else 0)
    ik0 = None if hca else csa.Buf.empty((B, N, DI), ik_fmt)
    # decode: the step recompresses the newest block (t0 = ctx - m); prefill: the last 2048 tokens
    T_step = 0 if key in ("3d", "4") else (m if decode else Tq)
    t0 = ctx - T_step
    build_secs, build_bytes = 0.0, 0
    log(f"[{key}] building caches: B={B} ctx={ctx} N={N} layers={L}")
    # stream memory of one sequence's cache build; sequences are compressed together in
    # launches of at most 16 GiB of streams
    tokens = t0 if T_step else ctx
    seq_bytes = (4 if not hca else 2) * tokens * (D + (0 if hca else DI)) * 2
    per_launch = max(1, min(B, (16 << 30) // max(1, seq_bytes)))
    if key != "4":
        for b0 in range(0, B, per_launch):
            bs = range(b0, min(B, b0 + per_launch))
            gens = [Gen(cfg.seed * 1000 + b, dev) for b in bs]
            sec, nb = _compress_bulk(csa, gens, kv0, b0, tokens, D, m, not hca, R, base, bf, timer)
            build_secs += sec
            build_bytes += nb
            if not hca:
                sec, nb = _compress_bulk(csa, gens, ik0, b0, tokens, DI, m, True, 0, base, bf, timer)
                build_secs += sec
                build_bytes += nb
    for b in range(B):
        g = Gen(cfg.seed * 1000 + b, dev)
        if key == "4":
            # seeded fp32 Gaussians quantized directly into the storage formats
            for r0 in range(0, N, 1 << 16):
                r1 = min(N, r0 + (1 << 16))
                x = g.normal((r1 - r0, D))
                csa.csa_quantize(x, csa.Buf(kv0.dtype, kv0.data[b, r0:r1], kv0.rope[b, r0:r1], kv0.scale[b, r0:r1]),
                                 rope_dims=R)
                xi = g.normal((r1 - r0, DI))
                csa.csa_quantize(xi, csa.Buf(ik0.dtype, ik0.data[b, r0:r1], None, ik0.scale[b, r0:r1]))
    torch.cuda.synchronize()

    # ------------------------------------------------------------------ step inputs
    g = Gen(cfg.seed, dev)
    pos = (torch.full((B, Tq), ctx, dtype=torch.int64, device=dev) if decode else
           torch.arange(ctx - Tq, ctx, dtype=torch.int64, device=dev).expand(B, Tq).contiguous())
    p_last = ctx if decode else ctx - 1
    p_first = ctx if decode else ctx - Tq
    wfirst = max(0, p_first - W + 1)
    Tw = p_last - wfirst + 1
    ios = []
    for li in range(L):
        if li == 0:
            kv, ik = kv0, ik0
        else:
            kv = csa.Buf.empty((B, N, D), kv_fmt, rope_dims=R if kv_fmt == csa.CSA_FP8MIX else 0)
            _copy_buf(kv, kv0)
            ik = None
            if not hca:
                ik = csa.Buf.empty((B, N, DI), ik_fmt)
                _copy_buf(ik, ik0)
        io = dict(kv_cache=kv, q_pos=pos, win_pos0=torch.full((B,), wfirst, dtype=torch.int64, device=dev),
                  q=g.normal((B, Tq, H, D), qstd(D), dtype=bf), sink=g.normal((H,)),
                  out=torch.empty((B, Tq, H, D), dtype=bf, device=dev))
        if T_step:
            nst = 2 if hca else 4
            st = [g.normal((B, T_step, D), dtype=bf) for _ in range(nst)]
            prev = [g.normal((B, m, D), dtype=bf) for _ in range(2)] if not hca else [None, None]
            io.update(ca=st[0], za=st[1] if hca else st[2])
            if not hca:
                io.update(cb=st[1], zb=st[3], prev_cb=prev[0], prev_zb=prev[1])
                ist = [g.normal((B, T_step, DI), dtype=bf) for _ in range(4)]
                iprev = [g.normal((B, m, DI), dtype=bf) for _ in range(2)]
                io.update(ica=ist[0], icb=ist[1], iza=ist[2], izb=ist[3], iprev_cb=iprev[0], iprev_zb=iprev[1])
        if kv_fmt == csa.CSA_FP8MIX:
            win = csa.Buf.empty((B, Tw, D), kv_fmt, rope_dims=R)
            csa.csa_quantize(g.normal((B, Tw, D)), win, rope_dims=R)
        else:
            win = g.normal((B, Tw, D), dtype=bf)
        io["win"] = win
        if not hca:
            if ik_fmt == csa.CSA_MXFP4:
                qI = csa.Buf.empty((B, Tq, HI, DI), ik_fmt)
                csa.csa_quantize(g.normal((B, Tq, HI, DI), qstd(DI)), qI)
            else:
                qI = g.normal((B, Tq, HI, DI), qstd(DI), dtype=bf)
            io.update(ik_cache=ik, qI=qI, wI=g.uniform((B, Tq, HI)))
        ios.append(io)

    def desc(T, Tq=Tq):
        return csa.layer_desc(mode=csa.CSA_MODE_HCA if hca else csa.CSA_MODE_CSA, B=B, T=T, t0=ctx - T if T else ctx,
                              Tq=Tq, cache_rows=N, Tw=Tw, D=D, H=H, HI=HI, DI=DI, ratio=m, topk=k, n_win=W,
                              rope_dims=R, rope_base=base, softmax_scale=cfg.softmax_scale, pos_offset=0,
                              stream_dtype=csa.CSA_BF16)

    desc_full = desc(T_step) if T_step else None
    desc_att = desc(0)
    desc_compress = desc(T_step, Tq=0) if T_step else None  # the step's compression launch alone
    every = 0 if not T_step else (4 if decode else 1)
    wl = Workload(key=key, name=WORKLOAD_TAGS[key], cfg=cfg, tokens=B * Tq, desc_full=desc_full,
                  desc_attend=desc_att, ios=ios, compress_every=every, desc_compress=desc_compress)
    need = csa.csa_forward_workspace_size(desc_full if desc_full is not None else desc_att)
    wl.ws = torch.empty(max(1, need), dtype=torch.uint8, device=dev)
    wl.meta = dict(B=B, Tq=Tq, ctx=ctx, m=m, N=N, D=D, R=R, HI=HI, DI=DI, k=k, H=H, W=W, T_step=T_step, Tw=Tw,
                   kv_format=cfg.kv_format, ik_format=cfg.ik_format, mode=cfg.mode)
    if build_secs > 0:
        wl.build = dict(us=round(build_secs * 1e6, 1), bytes=build_bytes,
                        GBps=round(build_bytes / build_secs / 1e9, 1),
                        hbm_frac=round(build_bytes / build_secs / HBM_PEAK, 4))
    _add_stages(wl, csa, torch, dev)
    _prepare_stages(wl, csa)
    wl.prepare()
    return wl


def _attn_kernels(ws, M, sparse: bool) -> str:
    """The attention kernels one call launches: the main kernel, plus the combine kernel
    when the key range is split (the call then needs a workspace for the partials)."""
    # D = 512 with 64 RoPE dims takes the LDS-DMA kernels (bf16 or FP8MIX cache; FP8MIX
    # with 4 or 8 waves); sparse bf16 launches with fewer than 256 query tokens per
    # sequence (128 heads) and at most 4096 key slots per query take the wave-pair kernel
    dma = M["D"] == 512 and M["R"] == 64 and (M["kv_format"] != "fp8mix" or M["H"] % 64 == 0)
    pair = (dma and sparse and M["kv_format"] != "fp8mix" and M["Tq"] * max(1, M["H"] // 128) < 256 and
            M["k"] + M["W"] <= 4096)
    main = "attn_pair_kernel" if pair else ("attn_dma_kernel" if dma else "attn_mfma_kernel")
    return main + ("+attn_combine_kernel" if ws.numel() > 1 else "")


def _add_stages(wl: Workload, csa, torch, dev):
    """Per-stage launches with the step's shapes, and their algorithmic work."""
    M = wl.meta
    B, Tq, N, D, R, HI, DI, k, H, W, m = (M[x] for x in ("B", "Tq", "N", "D", "R", "HI", "DI", "k", "H", "W", "m"))
    hca = M["mode"] == "hca"
    T = M["T_step"]
    ctx = M["ctx"]
    L = len(wl.ios)
    kv_entry = (D - R) + 2 * R + 4 if M["kv_format"] == "fp8mix" else 2 * D
    ik_entry = DI // 2 + DI // 32 if M["ik_format"] == "mxfp4" else 2 * DI
    q_entry = ik_entry
    pos = wl.ios[0]["q_pos"].cpu()
    vis = [[min(N, int(p) // m) for p in row] for row in pos.tolist()]
    sum_vis = sum(sum(r) for r in vis)
    cfg = wl.cfg

    if T:
        def st_compress(i):
            # the same fused launch (KV entries and indexer keys) the step makes
            csa.csa_forward(wl.desc_compress, wl.ios[i % L], ws=wl.ws)
        nst = 2 if hca else 4
        cb = B * (nst * T * D * 2 + (T // m) * kv_entry)
        if not hca:
            cb += B * (4 * T * DI * 2 + (T // m) * ik_entry)
        wl.stages["compress"] = Stage(st_compress, cb, 0.0, "compress_kernel")

    if not hca:
        scores = torch.empty((B, Tq, N), dtype=torch.float32, device=dev)
        idx = torch.empty((B, Tq, k), dtype=torch.int32, device=dev)

        def st_index(i):
            io = wl.ios[i % L]
            csa.csa_index_scores(io["qI"], io["wI"], io["ik_cache"], io["q_pos"], scores, ratio=m)

        def st_topk(i):
            csa.csa_topk(scores, k, idx)

        mx = M["ik_format"] == "mxfp4"
        wl.stages["index_scores"] = Stage(
            st_index, B * N * ik_entry + B * Tq * (HI * q_entry + HI * 4 + N * 4), 2.0 * HI * DI * sum_vis,
            "index_mxfp4_kernel" if mx else ("index_prefill_kernel" if Tq >= 16 else
                                             ("index_stream_kernel" if DI <= 128 else "index_mfma_kernel")),
            MFMA_FP4_PEAK if mx else MFMA_BF16_PEAK)
        wl.stages["topk"] = Stage(st_topk, B * Tq * (N * 4 + k * 4), 0.0, "topk_kernel")
        mqa_ws = torch.empty(max(1, csa.lib().csa_sparse_mqa_workspace_size(B, Tq, H, D, k, W)), dtype=torch.uint8,
                             device=dev)
        outs = torch.empty((B, Tq, H, D), dtype=torch.bfloat16, device=dev)

        def st_attn(i):
            io = wl.ios[i % L]
            csa.csa_sparse_mqa(io["q"], io["q_pos"], io["kv_cache"], idx, io["win"], io["win_pos0"], io["sink"],
                               outs, N=N, n_win=W, softmax_scale=cfg.softmax_scale, rope_dims=R,
                               rope_base=cfg.rope_base, ws=mqa_ws)
        keys = [min(k, v) + min(W, int(p) + 1) for row, prow in zip(vis, pos.tolist()) for v, p in zip(row, prow)]
        # algorithmic bytes: every distinct entry once (a prefill chunk's selections overlap), q, out, indices
        uniq = min(sum(keys), B * (N + M["Tw"]))
        wl.stages["sparse_mqa"] = Stage(st_attn, uniq * kv_entry + B * Tq * (4 * H * D + 4 * k),
                                        4.0 * H * D * sum(keys), _attn_kernels(mqa_ws, M, True))
        wl.stages["_prime"] = Stage(lambda i: (st_index(i), st_topk(i)), 0, 0, "")
    else:
        mqa_ws = torch.empty(max(1, csa.lib().hca_dense_attn_workspace_size(B, Tq, H, D, N, W)), dtype=torch.uint8,
                             device=dev)
        outs = torch.empty((B, Tq, H, D), dtype=torch.bfloat16, device=dev)

        def st_attn(i):
            io = wl.ios[i % L]
            csa.hca_dense_attn(io["q"], io["q_pos"], io["kv_cache"], io["win"], io["win_pos0"], io["sink"], outs, N=N,
                               ratio=m, n_win=W, softmax_scale=cfg.softmax_scale, rope_dims=R,
                               rope_base=cfg.rope_base, ws=mqa_ws)
        keys = [v + min(W, int(p) + 1) for row, prow in zip(vis, pos.tolist()) for v, p in zip(row, prow)]
        uniq = B * (N + M["Tw"]) if Tq > 1 else sum(keys)
        wl.stages["dense_attn"] = Stage(st_attn, uniq * kv_entry + B * Tq * 4 * H * D, 4.0 * H * D * sum(keys),
                                        _attn_kernels(mqa_ws, M, False))


def _prepare_stages(wl: Workload, csa):
    """Marshal each stage's launches once per layer, so timing sees the GPU and not Python."""
    L = len(wl.ios)
    for st in wl.stages.values():
        calls = [csa.PreparedCall(st.run, j) for j in range(L)]
        st.run = lambda i, calls=calls: calls[i % len(calls)]()


def time_stage(fn, reps):
    import torch
    for i in range(2):
        fn(i)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        fn(i)
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps * 1e-3


# ============================================================================ profiles


def _short(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").replace("void ", "").replace("csa::", "").split("(")[0]


def summarize_trace(db_path: str, out: str, command: str, kernel: str = ""):
    """Per-kernel duration summary of a `rocprofv3 --kernel-trace` database (rocpd SQLite).

    With `kernel` ("a" or "a+b": the kernels one stage launch runs), a last line gives
    the sum of their average durations, the figure bench.py's roofline time matches."""
    import sqlite3
    cur = sqlite3.connect(db_path).cursor()
    rows = cur.execute("select name, count(*), avg(duration), min(duration), max(duration), "
                       "sum(duration), avg(grid_x / workgroup_x) from kernels group by name "
                       "order by sum(duration) desc").fetchall()
    lines = ["# rocprofv3 kernel-trace summary", f"# command: {command}",
             f"# {'kernel':58s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_us':>10s} {'wgs':>7s}"]
    avg = {}
    for n, c, av, mn, mx, tot, wgs in rows:
        lines.append(f"{_short(n)[:60]:60s} {c:6d} {av / 1e3:9.2f} {mn / 1e3:9.2f} {mx / 1e3:9.2f} "
                     f"{tot / 1e3:10.1f} {wgs:7.0f}")
        avg.setdefault(_short(n).split("<")[0], av / 1e3)
    if kernel:
        parts = [avg.get(kn, float("nan")) for kn in kernel.split("+")]
        lines.append(f"# stage kernels {kernel}: average durations {' + '.join(f'{p:.2f}' for p in parts)} = "
                     f"{sum(parts):.2f} us per launch")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines[:16] + lines[-1:]))


def summarize_pmc(fetch_csv: str, write_csv: str, kernel: str, src: str, out: str, command: str, workload: str):
    """HBM traffic per launch of `kernel` (or of kernels "a+b" launched together) from
    FETCH_SIZE / WRITE_SIZE counter runs.

    Both counters (KiB per dispatch) are scaled by what they read for the copy probe
    (torch.neg over 1 GiB: 1 GiB read, 1 GiB written).  Dispatches of each kernel are
    grouped by grid size and the most frequent grid (the timed step's) is reported;
    the traffic of kernels launched together is summed.
    """
    import collections
    import csv

    names = kernel.split("+")

    def load(path, counter):
        per = collections.defaultdict(list)
        probe = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            if "neg_kernel" in name:  # only the copy probe calls torch.neg
                probe.append(v)
            else:
                for kn in names:
                    if _short(name).startswith(kn):
                        per[(kn, _short(name), int(r["Grid_Size"]))].append(v)
        return per, probe

    fetch, pf = load(fetch_csv, "FETCH_SIZE")
    write, pw = load(write_csv, "WRITE_SIZE")
    if not pf or not pw or not fetch:
        raise SystemExit(f"missing probe or kernel dispatches (probe {len(pf)}/{len(pw)}, kernel {len(fetch)})")
    kib = COPY_PROBE_BYTES / 1024
    f_fac = kib / (sum(pf) / len(pf))
    w_fac = kib / (sum(pw) / len(pw))
    lines = [f"# HBM traffic per launch of {kernel}, workload {workload}",
             f"# command (FETCH_SIZE pass): {command.replace('@COUNTER@', 'FETCH_SIZE')}",
             f"# command (WRITE_SIZE pass): {command.replace('@COUNTER@', 'WRITE_SIZE')}",
             f"# summarised by: python bench.py --summarize-pmc <fetch.csv> <write.csv> --kernel {kernel}",
             f"probe_fetch_kib = {sum(pf) / len(pf):.1f}", f"probe_write_kib = {sum(pw) / len(pw):.1f}",
             f"fetch_scale = {f_fac:.4f}", f"write_scale = {w_fac:.4f}"]
    traffic = 0.0
    for kn in names:
        keys = [kk for kk in fetch if kk[0] == kn]
        if not keys:
            raise SystemExit(f"no dispatches of {kn}")
        key = max(keys, key=lambda kk: len(fetch[kk]))
        f_avg = sum(fetch[key]) / len(fetch[key])
        w_avg = sum(write[key]) / len(write[key]) if write.get(key) else 0.0
        t = (f_avg * f_fac + w_avg * w_fac) * 1024
        traffic += t
        lines += [f"kernel = {key[1]} (most frequent grid: {key[2]} threads, {len(fetch[key])} dispatches)",
                  f"  fetch_kib_per_dispatch = {f_avg:.1f}", f"  write_kib_per_dispatch = {w_avg:.1f}",
                  f"  traffic_bytes = {t:.0f}"]
    lines += [f"traffic_bytes_per_launch = {traffic:.0f}", f"source_hash = {src}"]
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


COUNTERS = ("SQ_BUSY_CYCLES", "SQ_WAVE_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_VALU_MFMA_MOPS_BF16",
            "SQ_INSTS_LDS", "SQ_LDS_IDX_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_WAIT_INST_LDS", "GRBM_GUI_ACTIVE")
N_CU = 256
N_XCD = 8


def summarize_counters(csv_path: str, kernel: str, src: str, out: str, command: str, workload: str):
    """MFMA and LDS behaviour of `kernel` per dispatch from one `rocprofv3 --pmc` run of the
    COUNTERS (summed over the device by the profiler).

    mfma_busy_frac = SQ_VALU_MFMA_BUSY_CYCLES / (4 SIMDs x 256 CUs x GRBM_GUI_ACTIVE / 8): the
    share of SIMD-cycles the matrix cores were busy while the GPU ran the kernel (the
    profiler sums GRBM_GUI_ACTIVE over the 8 XCDs; at the clock the GPU actually ran, so
    it reads above the FLOP fraction of the 2.4 GHz spec peak);
    lds_bank_conflict_frac = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE: the share of the
    cycles the LDS was addressed that a bank conflict stalled; mfma_flop =
    SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 (the counter counts bf16 matrix work in units of
    512 FLOP).  The most frequent grid of the kernel (the timed step's) is reported."""
    import collections
    import csv

    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for r in csv.DictReader(open(csv_path)):
        name = _short(r["Kernel_Name"])
        if not name.startswith(kernel):
            continue
        per[(name, int(r["Grid_Size"]))][r["Counter_Name"]].append(float(r["Counter_Value"]))
    if not per:
        raise SystemExit(f"no dispatches of {kernel}")
    key = max(per, key=lambda k: len(per[k].get("GRBM_GUI_ACTIVE", [])))
    avg = {c: sum(v) / len(v) for c, v in per[key].items()}
    gui = avg.get("GRBM_GUI_ACTIVE", float("nan")) / N_XCD  # cycles the GPU was active
    mfma_frac = avg.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (4 * N_CU * gui)
    lds_frac = avg.get("SQ_LDS_BANK_CONFLICT", 0.0) / max(1.0, avg.get("SQ_LDS_IDX_ACTIVE", 0.0))
    lines = [f"# counters per dispatch of {kernel}, workload {workload}",
             f"# command: {command}",
             f"# summarised by: python bench.py --summarize-counters <counter_collection.csv> --kernel {kernel}",
             f"kernel = {key[0]} (most frequent grid: {key[1]} threads, "
             f"{len(per[key].get('GRBM_GUI_ACTIVE', []))} dispatches)"]
    lines += [f"  {c} = {avg[c]:.0f}" for c in COUNTERS if c in avg]
    lines += [f"mfma_busy_frac = {mfma_frac:.4f}", f"lds_bank_conflict_frac = {lds_frac:.4f}",
              f"mfma_flop_per_dispatch = {avg.get('SQ_INSTS_VALU_MFMA_MOPS_BF16', 0.0) * 512:.4g}",
              f"gpu_active_cycles_per_launch = {gui:.0f}",
              f"sq_busy_cycles_per_launch = {avg.get('SQ_BUSY_CYCLES', 0.0):.0f}",
              f"source_hash = {src}"]
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


# the sources a kernel's code comes from: its own file and the headers it includes
_HDR = ("device_common.h", "launch.h", "rmsnorm.h")
_HDR_SEL = _HDR + ("topk_select.h",)
KERNEL_SOURCES = {"attn_dma_kernel": ("mqa.hip",) + _HDR, "attn_mfma_kernel": ("mqa.hip",) + _HDR,
                  "attn_pair_kernel": ("mqa.hip",) + _HDR, "attn_combine_kernel": ("mqa.hip",) + _HDR,
                  "index_mfma_kernel": ("indexer.hip",) + _HDR_SEL, "index_stream_kernel": ("indexer.hip",) + _HDR_SEL,
                  "index_mxfp4_kernel": ("indexer.hip",) + _HDR_SEL, "index_prefill_kernel": ("indexer.hip",) + _HDR_SEL,
                  "topk_kernel": ("topk.hip",) + _HDR_SEL,
                  "compress_kernel": ("compress.hip",) + _HDR, "state_append_kernel": ("compress.hip",) + _HDR,
                  "gemm_few_kernel": ("proj.hip",) + _HDR, "gemm_tiled_kernel": ("proj.hip",) + _HDR,
                  "gemm_reduce_kernel": ("proj.hip",) + _HDR}


def kernel_src_hash(kernels: str) -> str:
    """Hash of the sources of the kernels named (joined by "+"): a committed profile
    counts only while it matches."""
    return src_hash(*sorted({f for kn in kernels.split("+") for f in KERNEL_SOURCES[kn]}))


# ============================================================================ runs


def run_workload(key: str, steps: int, warmup: int, layers: int, reps: int):
    """Build one workload, time `steps` whole steps (after `warmup`) and each stage alone.

    Returns (workload, tokens/s, ms per step, per-stage figures, dominant-stage roofline)."""
    import torch

    wl = build_workload(key, layers)
    for i in range(warmup):
        wl.step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        wl.step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e0.elapsed_time(e1) / steps
    value = wl.tokens / (ms_per_step * 1e-3)
    log(f"[{key}] step {ms_per_step * 1e3:.1f} us ({wall / steps * 1e6:.1f} us wall) -> {value:,.0f} tokens/s")

    if "_prime" in wl.stages:
        wl.stages.pop("_prime").run(0)
    torch.cuda.synchronize()
    stage_out = {}
    times = {}
    for name, s in wl.stages.items():
        t = time_stage(s.run, reps)
        times[name] = t
        gbs = s.bytes / t / 1e9
        tfs = s.flops / t / 1e12
        bound = "mfma" if s.flops / s.peak_flops > s.bytes / HBM_PEAK else "hbm"
        stage_out[name] = dict(us=round(t * 1e6, 2), GBps=round(gbs, 1), TFLOPs=round(tfs, 2),
                               hbm_frac=round(s.bytes / t / HBM_PEAK, 4),
                               mfma_frac=round(s.flops / t / s.peak_flops, 4), bound=bound, kernel=s.kernel,
                               algorithmic_bytes=int(s.bytes), algorithmic_flops=int(s.flops))
        log(f"  {name:13s} {t * 1e6:9.2f} us  {gbs:8.1f} GB/s  {tfs:7.2f} TFLOP/s  ({bound}-bound)")
    dom_name = max(wl.stages, key=lambda n: times[n])
    dom = wl.stages[dom_name]
    if stage_out[dom_name]["bound"] == "hbm":
        achieved, peak, unit = dom.bytes / times[dom_name] / 1e9, HBM_PEAK / 1e9, "GB/s"
    else:
        achieved, peak, unit = dom.flops / times[dom_name] / 1e12, dom.peak_flops / 1e12, "TFLOP/s"
    kern = dom.kernel
    traffic = read_traffic(f"{kern}_{wl.name}_pmc.txt", kernel_src_hash(kern))
    roofline = dict(kernel=kern, stage=dom_name, bound=stage_out[dom_name]["bound"], achieved=round(achieved, 2),
                    peak=peak, unit=unit, frac=round(achieved / peak, 4), traffic=traffic,
                    algorithmic_bytes=int(dom.bytes), algorithmic_flops=int(dom.flops),
                    avg_launch_us=round(times[dom_name] * 1e6, 2))
    counters = read_counters(f"{kern.split('+')[0]}_{wl.name}_counters.txt", kernel_src_hash(kern.split('+')[0]))
    if counters:
        roofline["counters"] = counters
    return wl, value, ms_per_step, stage_out, roofline


def layer_edges(wl: Workload, steps: int, reps: int):
    """The steps either side of core attention, timed apart from the step: the same
    forward steps with Q/KV RMSNorm (query heads, compressed entries and window rows),
    and the grouped output projection of the step's tokens at the large model's widths
    (128 heads x 512 -> 16 groups x 1024 -> 7168; bf16 weights, seeded)."""

    import torch

    import compressed_sparse_attention_07_amd as csa
    from synth import Gen

    M = wl.meta
    if M["mode"] != "csa" or M["kv_format"] == "fp8mix":
        return None
    g = Gen(wl.cfg.seed + 77, "cuda")
    D = M["D"]
    q_norm, kv_norm = g.uniform((D,), 0.5, 1.5), g.uniform((D,), 0.5, 1.5)

    def with_norm(d):
        if d is None:
            return None
        d2 = csa._lib.csa_layer_desc.from_buffer_copy(d)
        d2.flags |= csa.CSA_FLAG_QKV_NORM
        d2.norm_eps = 1e-6
        return d2

    dfull, datt = with_norm(wl.desc_full), with_norm(wl.desc_attend)
    ws = torch.empty(max(1, csa.csa_forward_workspace_size(dfull if dfull is not None else datt)), dtype=torch.uint8,
                     device="cuda")
    ios = [dict(io, q_norm=q_norm, kv_norm=kv_norm) for io in wl.ios]
    att = [csa.ForwardCall(datt, io, ws=ws) for io in ios]
    full = [csa.ForwardCall(dfull, io, ws=ws) for io in ios] if dfull is not None else att

    def step(i):
        f = wl.compress_every and (i % wl.compress_every == 0)
        (full if f else att)[i % len(ios)]()

    for i in range(4):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    out = {"qkv_norm_step": dict(ms_per_step=round(ms, 5), value=round(wl.tokens / (ms * 1e-3), 1),
                                 unit="tokens/s")}
    log(f"  with Q/KV RMSNorm: step {ms * 1e3:.1f} us")
    del att, full, ws

    # BF16 index scores ([V4-CN] §3.4): the same attend-only step with the scores rounded
    # to bf16 before the selection, and the recall of the exact (fp32) selection
    def flagged(d, f):
        d2 = csa._lib.csa_layer_desc.from_buffer_copy(d)
        d2.flags |= f
        return d2

    k, B, Tq = M["k"], M["B"], M["Tq"]
    sel = []
    for f in (0, csa.CSA_FLAG_BF16_SCORES):
        idx = torch.empty((B, Tq, k), dtype=torch.int32, device="cuda")
        d = flagged(wl.desc_attend, f)
        w = torch.empty(max(1, csa.csa_forward_workspace_size(d)), dtype=torch.uint8, device="cuda")
        csa.csa_forward(d, dict(wl.ios[0], idx_out=idx), ws=w)
        sel.append(idx.cpu().numpy().reshape(B * Tq, k))
    hits = total = 0
    for r in range(B * Tq):
        e = set(int(x) for x in sel[0][r] if x >= 0)
        hits += len(e & set(int(x) for x in sel[1][r] if x >= 0))
        total += len(e)
    times = []
    for f in (0, csa.CSA_FLAG_BF16_SCORES):
        d = flagged(wl.desc_attend, f)
        w = torch.empty(max(1, csa.csa_forward_workspace_size(d)), dtype=torch.uint8, device="cuda")
        calls = [csa.ForwardCall(d, io, ws=w) for io in wl.ios]
        times.append(time_stage(lambda i: calls[i % len(calls)](), reps))
        del calls, w
    out["bf16_scores"] = dict(attend_step_us=round(times[1] * 1e6, 2), attend_step_us_fp32=round(times[0] * 1e6, 2),
                              recall=round(hits / max(1, total), 5), selections=B * Tq, k=k)
    log(f"  BF16 scores: attend-only step {times[1] * 1e6:.1f} us (fp32 scores {times[0] * 1e6:.1f} us), "
        f"recall of the exact selection {hits / max(1, total):.4f}")

    T = M["B"] * M["Tq"]
    n_h, c, ng, d_g, d = 128, 512, 16, 1024, 7168
    o = g.normal((T, n_h, c), dtype=torch.bfloat16)
    wg = g.normal((ng, d_g, (n_h // ng) * c), ((n_h // ng) * c) ** -0.5, dtype=torch.bfloat16)
    wo = g.normal((d, ng * d_g), (ng * d_g) ** -0.5, dtype=torch.bfloat16)
    y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    pws = torch.empty(max(1, csa.csa_grouped_out_proj_workspace_size(T, n_h, c, ng, d_g, d)), dtype=torch.uint8,
                      device="cuda")
    call = csa.PreparedCall(csa.csa_grouped_out_proj, o, wg, wo, y, ws=pws)
    t = time_stage(lambda i: call(), reps)
    nbytes = (wg.numel() + wo.numel() + o.numel() + y.numel()) * 2
    flops = 2.0 * T * (n_h * c * d_g + ng * d_g * d)
    bound = "mfma" if flops / MFMA_BF16_PEAK > nbytes / HBM_PEAK else "hbm"
    out["grouped_out_proj"] = dict(us=round(t * 1e6, 2), tokens=T, GBps=round(nbytes / t / 1e9, 1),
                                   TFLOPs=round(flops / t / 1e12, 2), hbm_frac=round(nbytes / t / HBM_PEAK, 4),
                                   mfma_frac=round(flops / t / MFMA_BF16_PEAK, 4), bound=bound,
                                   kernel=("gemm_few_kernel+gemm_reduce_kernel" if T <= 32 else
                                           "gemm_tiled_kernel" if T >= 128 else "gemm_bf16_kernel"),
                                   algorithmic_bytes=int(nbytes), algorithmic_flops=int(flops))
    log(f"  grouped output projection ({T} tokens): {t * 1e6:.1f} us, {nbytes / t / 1e9:.0f} GB/s, "
        f"{flops / t / 1e12:.1f} TFLOP/s ({bound}-bound)")
    return out


def fp8_query_edge(wl: Workload, reps: int):
    """The sparse attention stage over an FP8MIX cache with bf16 queries and with FP8MIX
    queries (QK products of the codes on fp8 MFMA), same selections; plus the cost of
    quantizing the step's queries.  CSA workloads with an FP8MIX cache, or prefill chunks
    (whose bf16 cache is quantized for the comparison); None otherwise."""
    import torch

    import compressed_sparse_attention_07_amd as csa

    M = wl.meta
    fp8_cache = M["kv_format"] == "fp8mix"
    if M["mode"] != "csa" or not (fp8_cache or M["Tq"] > 1) or M["D"] != 512 or M["R"] != 64:
        return None
    B, Tq, H, D, R, N, k, W = (M[x] for x in ("B", "Tq", "H", "D", "R", "N", "k", "W"))
    io = wl.ios[0]
    cfg = wl.cfg

    def quantized(x):  # [.., D] bf16 or fp32 tensor -> FP8MIX Buf of the same rows
        rows = x.numel() // D
        b = csa.Buf.empty(tuple(x.shape), csa.CSA_FP8MIX, rope_dims=R)
        flat = csa.Buf(b.dtype, b.data.view(rows, D - R), b.rope.view(rows, R), b.scale.view(rows))
        xv = x.reshape(rows, D)
        for r0 in range(0, rows, 1 << 16):
            r1 = min(rows, r0 + (1 << 16))
            csa.csa_quantize(xv[r0:r1].float().contiguous(),
                             csa.Buf(b.dtype, flat.data[r0:r1], flat.rope[r0:r1], flat.scale[r0:r1]), rope_dims=R)
        return b

    kv8 = io["kv_cache"] if fp8_cache else quantized(io["kv_cache"].data if isinstance(io["kv_cache"], csa.Buf)
                                                     else io["kv_cache"])
    win8 = io["win"] if fp8_cache else quantized(io["win"].data if isinstance(io["win"], csa.Buf) else io["win"])
    q = io["q"]
    q8 = quantized(q)
    idx = torch.empty((B, Tq, k), dtype=torch.int32, device="cuda")
    w = torch.empty(max(1, csa.csa_forward_workspace_size(wl.desc_attend)), dtype=torch.uint8, device="cuda")
    csa.csa_forward(wl.desc_attend, dict(io, idx_out=idx), ws=w)
    del w
    mqa_ws = torch.empty(max(1, csa.lib().csa_sparse_mqa_workspace_size(B, Tq, H, D, k, W)), dtype=torch.uint8,
                         device="cuda")
    outs = [torch.empty((B, Tq, H, D), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    calls = [csa.PreparedCall(csa.csa_sparse_mqa, qq, io["q_pos"], kv8, idx, win8, io["win_pos0"], io["sink"], o,
                              N=N, n_win=W, softmax_scale=cfg.softmax_scale, rope_dims=R, rope_base=cfg.rope_base,
                              ws=mqa_ws) for qq, o in ((q, outs[0]), (q8, outs[1]))]
    t_bf16 = time_stage(lambda i: calls[0](), reps)
    t_fp8 = time_stage(lambda i: calls[1](), reps)
    qrows = B * Tq * H
    qf32 = q.reshape(qrows, D).float().contiguous() if qrows <= (1 << 16) else None
    t_quant = None
    if qf32 is not None:
        qb = csa.Buf(q8.dtype, q8.data.view(qrows, D - R), q8.rope.view(qrows, R), q8.scale.view(qrows))
        qcall = csa.PreparedCall(csa.csa_quantize, qf32, qb, rope_dims=R)
        t_quant = time_stage(lambda i: qcall(), reps)
    torch.cuda.synchronize()
    diff = (outs[0].float() - outs[1].float()).abs().max().item()
    flops = wl.stages["sparse_mqa"].flops
    res = dict(attend_us_bf16_query=round(t_bf16 * 1e6, 2), attend_us_fp8_query=round(t_fp8 * 1e6, 2),
               mfma_frac_bf16_query=round(flops / t_bf16 / MFMA_BF16_PEAK, 4),
               mfma_frac_fp8_query_vs_bf16_peak=round(flops / t_fp8 / MFMA_BF16_PEAK, 4),
               query_quantize_us=None if t_quant is None else round(t_quant * 1e6, 2),
               max_abs_diff_vs_bf16_query=round(diff, 5),
               cache="FP8MIX" if fp8_cache else "FP8MIX quantized from the workload's bf16 cache",
               kernel="attn_dma_kernel (fp8 query products)")
    log(f"  FP8MIX cache: attention {t_bf16 * 1e6:.1f} us with bf16 queries, {t_fp8 * 1e6:.1f} us with FP8MIX "
        f"queries (max |diff| {diff:.4f})")
    return res


def decode_state_bench(wl: Workload, steps: int, warmup: int):
    """The same decode layer served by csa_decode_step from a state pool and paged caches
    (ragged lengths near the workload's context; every step appends one token per
    sequence, so blocks complete and windows roll over as in serving).  Returns the
    step rate, or None for workloads it does not cover."""
    import torch

    import compressed_sparse_attention_07_amd as csa
    from synth import Gen, qstd

    M = wl.meta
    if M["Tq"] != 1:
        return None
    csa_mode = M["mode"] == "csa"
    B, D, H, HI, DI, k, W, m, ctx, R = (M[x] for x in ("B", "D", "H", "HI", "DI", "k", "W", "m", "ctx", "R"))
    cfg = wl.cfg
    page_tokens = 2048 if csa_mode else 4096
    total = steps + warmup + 4
    # ragged lengths just below the context, so that every query sees at most the
    # workload's entry count (the row length the top-k planner is shaped for)
    lengths = [ctx - total - 2 * m - (b * 37) % 509 for b in range(B)]
    max_pages = -(-ctx // page_tokens)
    pages = B * max_pages
    g = Gen(cfg.seed + 991, "cuda")
    bf = torch.bfloat16
    kvd = csa.CSA_FP8MIX if M["kv_format"] == "fp8mix" else csa.CSA_BF16
    ikd = csa.CSA_MXFP4 if M["ik_format"] == "mxfp4" else csa.CSA_BF16
    pool = csa.DecodePool(mode=csa.CSA_MODE_CSA if csa_mode else csa.CSA_MODE_HCA, slots=B, pages=pages,
                          max_pages=max_pages, page_tokens=page_tokens, D=D, DI=DI, ratio=m, n_win=W,
                          stream_dtype=csa.CSA_BF16, kv_dtype=kvd, ik_dtype=ikd, rope_dims=R)
    gen = torch.Generator().manual_seed(cfg.seed)
    pool.block_table.copy_(torch.randperm(pages, generator=gen).view(B, max_pages).to(torch.int32))

    def fill(buf, std):
        # seeded Gaussians; quantized formats take fp32 rows through the library's quantizer
        b = csa.Buf.of(buf)
        flat = lambda t, k: None if t is None else t.reshape((-1,) + tuple(t.shape[k:]))
        lead = len(b.data.shape) - 1
        data, rope, scale = flat(b.data, lead), flat(b.rope, lead), flat(b.scale, lead)
        for r0 in range(0, data.shape[0], 1 << 15):
            r1 = min(data.shape[0], r0 + (1 << 15))
            if b.dtype == csa.CSA_BF16:
                data[r0:r1].copy_(g.normal(data[r0:r1].shape, std, dtype=bf))
                continue
            width = b.shape[-1]
            part = csa.Buf(b.dtype, data[r0:r1], None if rope is None else rope[r0:r1], scale[r0:r1])
            csa.csa_quantize(g.normal((r1 - r0, width), std), part, rope_dims=R if b.dtype == csa.CSA_FP8MIX else 0)

    fill(pool.kv_pages, 0.5)
    if csa_mode:
        fill(pool.ik_pages, 0.5)
    fill(pool.win, 0.5)
    for x in (pool.tail, pool.itail):
        if x is not None:
            for r0 in range(0, x.shape[0], 64):
                x[r0:r0 + 64].copy_(g.normal(x[r0:r0 + 64].shape, 0.5, dtype=bf))
    pool.length.copy_(torch.tensor(lengths, dtype=torch.int64))
    pool.win_pos0.copy_(torch.tensor([n - W + 1 for n in lengths], dtype=torch.int64))
    ns = 4 if csa_mode else 2
    st = [g.normal((B, D), dtype=bf) for _ in range(ns)]
    kv_raw = csa.Buf.empty((B, D), kvd, rope_dims=R)
    fill(kv_raw.data if kvd == csa.CSA_BF16 else kv_raw, 1.0)
    io = dict(pool.io(), slot=torch.arange(B, dtype=torch.int32, device="cuda"), kv_raw=kv_raw,
              q=g.normal((B, H, D), qstd(D), dtype=bf), sink=g.normal((H,)),
              out=torch.empty((B, H, D), dtype=bf, device="cuda"))
    if csa_mode:
        ist = [g.normal((B, DI), dtype=bf) for _ in range(4)]
        qI = csa.Buf.empty((B, HI, DI), ikd)
        if ikd == csa.CSA_BF16:
            qI.data.copy_(g.normal((B, HI, DI), qstd(DI), dtype=bf))
        else:
            csa.csa_quantize(g.normal((B * HI, DI), qstd(DI)), csa.Buf(ikd, qI.data.view(B * HI, -1), None,
                                                                       qI.scale.view(B * HI, -1)))
        io.update(ca=st[0], cb=st[1], za=st[2], zb=st[3], ica=ist[0], icb=ist[1], iza=ist[2], izb=ist[3],
                  qI=qI, wI=g.uniform((B, HI)))
    else:
        io.update(ca=st[0], za=st[1])
    desc = csa.decode_desc(mode=csa.CSA_MODE_CSA if csa_mode else csa.CSA_MODE_HCA, B=B, slots=B, pages=pages,
                           max_pages=max_pages, page_tokens=page_tokens, D=D, H=H, HI=HI, DI=DI, ratio=m, topk=k,
                           n_win=W, rope_dims=R, rope_base=cfg.rope_base, softmax_scale=cfg.softmax_scale,
                           stream_dtype=csa.CSA_BF16)
    ws = torch.empty(max(1, csa.csa_decode_step_workspace_size(desc)), dtype=torch.uint8, device="cuda")
    call = csa.PreparedCall(csa.csa_decode_step, desc, io, ws=ws)
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        call()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    log(f"  decode state step (ragged, paged {page_tokens}-token blocks): {ms * 1e3:.1f} us")
    return dict(ms_per_step=round(ms, 5), value=round(B / (ms * 1e-3), 1), unit="tokens/s", B=B,
                lengths=f"{min(lengths)}..{max(lengths)}", page_tokens=page_tokens,
                step="csa_decode_step: append + (index + top-k) + attention")


# ============================================================================ main


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: 48 decode, 6 prefill)")
    ap.add_argument("--warmup", type=int, default=None)
    ap.add_argument("--config", default="1", choices=sorted(WORKLOAD_TAGS))
    ap.add_argument("--layers", type=int, default=None, help="cache copies cycled over (default: 4 decode, 1 prefill)")
    ap.add_argument("--stage-reps", type=int, default=None)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU time spent on the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="time only --config (not the other workloads)")
    ap.add_argument("--no-edges", action="store_true",
                    help="skip the layer-edge, FP8-query and decode-state legs (profiling runs)")
    ap.add_argument("--copy-probe", action="store_true", help="also run a plain 1 GiB device copy (PMC calibration)")
    ap.add_argument("--summarize-trace", metavar="DB", help="write a kernel-trace summary (no GPU work)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write an HBM-traffic summary from two counter runs (no GPU work)")
    ap.add_argument("--summarize-counters", metavar="CSV",
                    help="write an MFMA / LDS counter summary from one counter run (no GPU work)")
    ap.add_argument("--kernel", default="attn_dma_kernel")
    ap.add_argument("--profile-cmd", default="", help="command recorded in the summary")
    ap.add_argument("--out", help="summary file")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.profile_cmd, args.kernel)
        return
    if args.summarize_counters:
        tag = WORKLOAD_TAGS[args.config]
        out = args.out or os.path.join(ROOT, "profiles", f"{args.kernel}_{tag}_counters.txt")
        summarize_counters(args.summarize_counters, args.kernel, kernel_src_hash(args.kernel), out,
                           args.profile_cmd, tag)
        return
    if args.summarize_pmc:
        tag = WORKLOAD_TAGS[args.config]
        out = args.out or os.path.join(ROOT, "profiles", f"{args.kernel}_{tag}_pmc.txt")
        summarize_pmc(*args.summarize_pmc, args.kernel, kernel_src_hash(args.kernel), out, args.profile_cmd, tag)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): there is no multi-GPU path; "
              "decode shards by sequence, each GPU serving its own sequences", file=sys.stderr)
        sys.exit(2)

    import torch

    import compressed_sparse_attention_07_amd as csa

    if not os.path.exists(csa.LIB_PATH):
        from compressed_sparse_attention_07_amd import build
        build.build()
    assert csa.lib().csa_device_check() == 0, csa.lib().csa_last_error()
    decode = args.config in ("1", "3d", "4")
    steps = args.steps if args.steps is not None else (48 if decode else 6)
    warmup = args.warmup if args.warmup is not None else (8 if decode else 2)
    layers = args.layers if args.layers is not None else (4 if decode else 1)
    reps = args.stage_reps if args.stage_reps is not None else (20 if decode else 4)

    wl, value, ms_per_step, stage_out, roofline = run_workload(args.config, steps, warmup, layers, reps)
    edges = fq = dstate = None
    if not args.no_edges:
        edges = layer_edges(wl, steps, reps)
        fq = fp8_query_edge(wl, reps)
        dstate = decode_state_bench(wl, steps, warmup)

    if args.copy_probe:
        # a plain elementwise kernel of known traffic (reads 1 GiB, writes 1 GiB): the
        # reference for scaling the FETCH_SIZE / WRITE_SIZE counters
        src = torch.zeros(COPY_PROBE_BYTES // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("copy probe: 3 x neg over 1 GiB done")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds)

    M = wl.meta
    config = {"workload": wl.cfg.name if args.config in ("1", "2", "4") else
              ("HCA decode bf16, B=32, 1M context, m'=128, D=512, H=128" if args.config == "3d" else
               "HCA prefill bf16, 2048-token chunk at 1M context, m'=128, D=512, H=128"),
              "B": M["B"], "context": M["ctx"], "query_tokens_per_seq": M["Tq"], "m": M["m"], "entries": M["N"],
              "D": M["D"], "rope_dims": M["R"], "heads": M["H"], "window": M["W"], "kv_format": M["kv_format"],
              "layers_cycled": len(wl.ios)}
    if M["mode"] == "csa":
        config.update(indexer=f"{M['HI']}x{M['DI']}", topk=M["k"], ik_format=M["ik_format"])
    config["step"] = ("csa_forward per new token; the newest block is compressed every 4th step" if decode and
                      wl.compress_every == 4 else
                      "csa_forward over the chunk (compress + attend)" if not decode else "csa_forward (attend only)")
    line = {
        "metric": METRIC if args.config == "1" else f"{wl.name} tokens/s; per-stage % of HBM / MFMA peak",
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if M["kv_format"] != "fp8mix" else "bf16+fp8kv+mxfp4idx",
        "data": "synthetic", "config": config, "roofline": roofline, "cpu_baseline": cpu, "stages": stage_out,
    }
    if wl.build:
        line["cache_build_compress"] = wl.build
    if edges:
        line["layer_edges"] = edges
    if fq:
        line["fp8_query"] = fq
    if dstate:
        line["decode_state"] = dstate
    if not args.no_others:
        # the other workloads at their full sizes, fewer steps each: their step rate,
        # every stage's time and fraction of peak, and the dominant stage's roofline
        others = {}
        key0, tag0 = args.config, wl.name
        del wl
        for key in [k for k in ("1", "2", "3d", "3p", "4") if k != key0]:
            torch.cuda.empty_cache()
            dec = key in ("1", "3d", "4")
            w2, v2, ms2, st2, rf2 = run_workload(key, 16 if dec else 3, 4 if dec else 1, 4 if dec else 1,
                                                 10 if dec else 3)
            others[WORKLOAD_TAGS[key]] = dict(value=round(v2, 1), unit="tokens/s", ms_per_step=round(ms2, 5),
                                              build_compress=w2.build or None, roofline=rf2, stages=st2)
            e2 = layer_edges(w2, 16 if dec else 3, 10 if dec else 3)
            if e2:
                others[WORKLOAD_TAGS[key]]["layer_edges"] = e2
            f2 = fp8_query_edge(w2, 10 if dec else 3)
            if f2:
                others[WORKLOAD_TAGS[key]]["fp8_query"] = f2
            d2 = decode_state_bench(w2, 16, 4) if dec else None
            if d2:
                others[WORKLOAD_TAGS[key]]["decode_state"] = d2
            del w2
        line["other_workloads"] = others
    print(json.dumps(line), flush=True)


def cpu_baseline(wl: Workload, seconds: float):
    """Time the fp64 oracle on a bounded sample of the workload, for about `seconds`.

    Decode: the oracle builds one sequence's caches from the same seeded streams
    (untimed), then times decode steps with fresh seeded inputs -- compress the newest
    block, score every entry, top-k, MQA over the selection and the window.
    Other workloads: the oracle's per-query work (index scores, top-k, attention) for
    a sample of query tokens over the GPU-built caches, read back once.
    """
    import numpy as np
    import torch

    from oracle import csa_oracle as O
    from synth import Gen, qstd

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    cores = len(os.sched_getaffinity(0))
    f = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
    M, cfg = wl.meta, wl.cfg
    m, D, R, ctx, DI, W, H, HI, k = M["m"], M["D"], M["R"], M["ctx"], M["DI"], M["W"], M["H"], M["HI"], M["k"]
    bf = torch.bfloat16
    total, steps = 0.0, 0
    if wl.key == "1":
        t0 = ctx - m
        g = Gen(cfg.seed * 1000, "cuda")
        s = [f(g.normal((1, ctx, D), dtype=bf)[0]) for _ in range(4)]
        si = [f(g.normal((1, ctx, DI), dtype=bf)[0]) for _ in range(4)]
        log("cpu baseline: oracle cache build for sequence 0 (untimed)")
        kv = O.compress(*s, ratio=m, overlap=True, rope_dims=R, rope_base=cfg.rope_base)
        ik = O.compress(*si, ratio=m, overlap=True)
        del s, si
        pos = np.array([ctx])
        while total < seconds and steps < 100000:
            g = Gen(cfg.seed * 7919 + steps, "cuda")
            blk = [f(g.normal((m, D), dtype=bf)) for _ in range(6)]
            iblk = [f(g.normal((m, DI), dtype=bf)) for _ in range(6)]
            q = f(g.normal((1, H, D), qstd(D), dtype=bf))
            qI = f(g.normal((1, HI, DI), qstd(DI), dtype=bf))
            wI = f(g.uniform((1, HI)))
            win = f(g.normal((W, D), dtype=bf))
            sink = f(g.normal((H,)))
            tic = time.perf_counter()
            if steps % 4 == 0:  # the newest block, every 4th step as in the timed loop
                e = O.compress(*blk[:4], ratio=m, overlap=True, t0=t0, prev_cb=blk[4], prev_zb=blk[5],
                               rope_dims=R, rope_base=cfg.rope_base)
                kv[-1] = e[0]
                ei = O.compress(*iblk[:4], ratio=m, overlap=True, t0=t0, prev_cb=iblk[4], prev_zb=iblk[5])
                ik[-1] = ei[0]
            sc = O.index_scores(qI, wI, ik, pos, m)
            idx, _ = O.topk(sc, k)
            O.mqa(q, pos, kv, idx, win, ctx - W + 1, W, sink, scale=cfg.softmax_scale, rope_dims=R,
                  rope_base=cfg.rope_base)
            total += time.perf_counter() - tic
            steps += 1
        sample = (f"{steps} decode steps of sequence 0 (fresh seeded block, queries, window and sink per step; the "
                  f"block compressed every 4th step): score {ctx // m} entries, top-{k}, MQA over {k}+{W} keys; the "
                  "oracle's caches are built once, untimed")
    else:
        from oracle import quant as Q
        io = wl.ios[0]
        hca = M["mode"] == "hca"

        def deq(buf, b):
            if buf.dtype == 2:  # FP8MIX
                return Q.fp8mix_dequantize(buf.data[b].cpu().numpy(), buf.rope[b].view(torch.int16).cpu().numpy()
                                           .view(np.uint16), buf.scale[b].cpu().numpy())
            if buf.dtype == 3:  # MXFP4
                return Q.mxfp4_dequantize(buf.data[b].cpu().numpy(), buf.scale[b].cpu().numpy())
            return f(buf.data[b])

        def dense(x, b):
            return deq(x, b) if not isinstance(x, torch.Tensor) else f(x[b])
        Tq, B = M["Tq"], M["B"]
        order = np.random.default_rng(0).permutation(Tq)
        for b in range(B):
            if total >= seconds:
                break
            log(f"cpu baseline: reading caches of sequence {b} back (untimed)")
            kv = deq(io["kv_cache"], b)
            ik = None if hca else deq(io["ik_cache"], b)
            qI_all = None if hca else dense(io["qI"], b)
            pos = io["q_pos"][b].cpu().numpy()
            win = dense(io["win"], b)
            wp0 = int(io["win_pos0"][b])
            sink = f(io["sink"])
            for t in order:
                if total >= seconds:
                    break
                t = int(t)
                q = f(io["q"][b, t:t + 1])
                p = pos[t:t + 1]
                tic = time.perf_counter()
                if hca:
                    O.hca_dense(q, p, kv, win, wp0, W, sink, ratio=m, scale=cfg.softmax_scale, rope_dims=R,
                                rope_base=cfg.rope_base)
                else:
                    sc = O.index_scores(qI_all[t:t + 1], f(io["wI"][b, t:t + 1]), ik, p, m)
                    idx, _ = O.topk(sc, k)
                    O.mqa(q, p, kv, idx, win, wp0, W, sink, scale=cfg.softmax_scale, rope_dims=R,
                          rope_base=cfg.rope_base)
                total += time.perf_counter() - tic
                steps += 1
            del kv, ik
        sample = (f"{steps} query tokens ({'dense attention' if hca else 'index, top-k, MQA'}) over the GPU-built "
                  "caches, read back per sequence untimed; the chunk's compression is not in the sample")
    rate = steps / total
    log(f"cpu baseline: {steps} units in {total:.2f} s -> {rate:.2f} tokens/s ({threads} BLAS threads, {cores} cores)")
    return dict(value=round(rate, 3), unit="tokens/s", cores=threads, host_cores=cores, kind="oracle",
                seconds=round(total, 2), sample=sample)


if __name__ == "__main__":
    main()
