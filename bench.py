#!/usr/bin/env python3
"""Benchmark of the CSA decode step at 128K context on one MI355X.

Workload (the headline configuration): B = 16 sequences, 131,072 tokens of context
each, CSA with m = 4 (32,768 compressed entries per sequence), shared KV dim 512
(last 64 dims RoPE), lightning indexer 64 heads x 128, top-k 1024, 128 query heads
x 512, window 128, bf16.  Inputs are seeded synthetic tensors (synth module); the
KV and indexer-key caches are built by csa_compress from each sequence's streams
before timing.

One step = one csa_forward call for the new token of every sequence: compress the
newest 4-token block (one entry per sequence; a real decoder does this every 4th
step, so this over-counts), score all 32,768 entries, select the top 1024, and
attend over them plus the 128-token window.  Each step uses the caches of a
different "layer" (--layers copies, cycled) so that caches are read from HBM, not
from the 256 MB Infinity Cache, as in a multi-layer decode.

Prints one JSON line (see the keys below).  Stage times are measured with HIP
events on the stream the kernels run on.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12            # B/s, MI355X published
MFMA_BF16_PEAK = 2.5e15      # FLOP/s dense bf16, MI355X published
COPY_PROBE_BYTES = 1 << 30  # bytes read (and written) by one copy-probe launch
WORKLOAD_TAG = "csa_decode_b16_ctx128k"
METRIC = "CSA decode tokens/s @128K ctx; indexer+MQA % MFMA peak, compress/top-k % HBM"


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


def _short(name: str) -> str:
    return name.replace("(anonymous namespace)::", "").replace("void ", "").replace("csa::", "").split("(")[0]


def summarize_trace(db_path: str, out: str, command: str):
    """Per-kernel duration summary of a `rocprofv3 --kernel-trace` database (rocpd SQLite)."""
    import sqlite3
    cur = sqlite3.connect(db_path).cursor()
    rows = cur.execute("select name, count(*), avg(duration), min(duration), max(duration), "
                       "sum(duration), avg(grid_x / workgroup_x) from kernels group by name "
                       "order by sum(duration) desc").fetchall()
    lines = [f"# rocprofv3 kernel-trace summary", f"# command: {command}",
             f"# {'kernel':58s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s} {'total_us':>10s} {'wgs':>7s}"]
    for n, c, av, mn, mx, tot, wgs in rows:
        lines.append(f"{_short(n)[:60]:60s} {c:6d} {av / 1e3:9.2f} {mn / 1e3:9.2f} {mx / 1e3:9.2f} "
                     f"{tot / 1e3:10.1f} {wgs:7.0f}")
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines[:14]))


def summarize_pmc(fetch_csv: str, write_csv: str, kernel: str, src: str, out: str, command: str):
    """HBM traffic per launch of `kernel` from FETCH_SIZE / WRITE_SIZE counter runs.

    Both counters (KiB per dispatch) are scaled by what they read for the copy probe
    (torch.neg over 1 GiB: 1 GiB read, 1 GiB written).  Dispatches of `kernel` are
    grouped by grid size and the most frequent grid (the decode step's) is reported.
    """
    import collections
    import csv

    def load(path, counter):
        per = collections.defaultdict(list)
        probe = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            name, v = r["Kernel_Name"], float(r["Counter_Value"])
            if "neg_kernel" in name:  # only the copy probe calls torch.neg
                probe.append(v)
            elif _short(name).startswith(kernel):
                per[(_short(name), int(r["Grid_Size"]))].append(v)
        return per, probe

    fetch, pf = load(fetch_csv, "FETCH_SIZE")
    write, pw = load(write_csv, "WRITE_SIZE")
    if not pf or not pw or not fetch:
        raise SystemExit(f"missing probe or kernel dispatches (probe {len(pf)}/{len(pw)}, kernel {len(fetch)})")
    key = max(fetch, key=lambda k: len(fetch[k]))
    kib = COPY_PROBE_BYTES / 1024
    f_fac = kib / (sum(pf) / len(pf))
    w_fac = kib / (sum(pw) / len(pw))
    f_avg = sum(fetch[key]) / len(fetch[key])
    w_avg = sum(write[key]) / len(write[key]) if write.get(key) else 0.0
    traffic = (f_avg * f_fac + w_avg * w_fac) * 1024
    lines = [f"# HBM traffic per launch of {key[0]} (grid {key[1]} threads), decode step of the headline workload",
             f"# command (FETCH_SIZE pass): {command.replace('@COUNTER@', 'FETCH_SIZE')}",
             f"# command (WRITE_SIZE pass): {command.replace('@COUNTER@', 'WRITE_SIZE')}",
             f"# summarised by: python bench.py --summarize-pmc <fetch.csv> <write.csv> --kernel {kernel}",
             f"kernel = {key[0]}", f"grid_threads = {key[1]}", f"dispatches = {len(fetch[key])}",
             f"fetch_kib_per_dispatch = {f_avg:.1f}", f"write_kib_per_dispatch = {w_avg:.1f}",
             f"probe_fetch_kib = {sum(pf) / len(pf):.1f}", f"probe_write_kib = {sum(pw) / len(pw):.1f}",
             f"fetch_scale = {f_fac:.4f}", f"write_scale = {w_fac:.4f}",
             f"traffic_bytes_per_launch = {traffic:.0f}", f"source_hash = {src}"]
    open(out, "w").write("\n".join(lines) + "\n")
    print("\n".join(lines))


KERNEL_SOURCES = {"attn_mfma_kernel": ("mqa.hip",), "attn_combine_kernel": ("mqa.hip",),
                  "index_mfma_kernel": ("indexer.hip",), "topk_kernel": ("topk.hip",),
                  "compress_kernel": ("compress.hip",)}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--stage-reps", type=int, default=20)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU time spent on the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", action="store_true", help="also run a plain 1 GiB device copy (PMC calibration)")
    ap.add_argument("--summarize-trace", metavar="DB", help="write a kernel-trace summary (no GPU work)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write an HBM-traffic summary from two counter runs (no GPU work)")
    ap.add_argument("--kernel", default="attn_mfma_kernel")
    ap.add_argument("--profile-cmd", default="", help="command recorded in the summary")
    ap.add_argument("--out", help="summary file")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.out, args.profile_cmd)
        return
    if args.summarize_pmc:
        out = args.out or os.path.join(ROOT, "profiles", f"{args.kernel}_{WORKLOAD_TAG}_pmc.txt")
        summarize_pmc(*args.summarize_pmc, args.kernel, src_hash(*KERNEL_SOURCES[args.kernel]), out,
                      args.profile_cmd)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this build has no multi-GPU path; "
              "the decode workload shards by sequence (see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import torch

    import compressed_sparse_attention_07_amd as csa
    from synth import CONFIGS, Gen, qstd

    if not os.path.exists(csa.LIB_PATH):
        from compressed_sparse_attention_07_amd import build
        build.build()
    dev = "cuda"
    assert csa.lib().csa_device_check() == 0, csa.lib().csa_last_error()
    cfg = CONFIGS[1]
    B, ctx, m, D, R, HI, DI, k, H, W = cfg.B, cfg.ctx, cfg.m, cfg.D, cfg.R, cfg.HI, cfg.DI, cfg.k, cfg.H, cfg.n_win
    N = ctx // m
    bf = torch.bfloat16
    L = max(1, args.layers)
    t_new = ctx                      # position of the new token
    t0 = ctx - m                     # the newest complete block, recompressed every step

    # ---------------------------------------------------------------- caches
    log(f"building caches: B={B} ctx={ctx} N={N} layers={L}")
    kv = [csa.Buf.empty((B, N, D), csa.CSA_BF16) for _ in range(L)]
    ik = [csa.Buf.empty((B, N, DI), csa.CSA_BF16) for _ in range(L)]
    ev = lambda: torch.cuda.Event(enable_timing=True)
    build_ms = 0.0
    build_bytes = 0
    for b in range(B):
        g = Gen(cfg.seed * 1000 + b, dev)
        s = [g.normal((1, ctx, D), dtype=bf) for _ in range(4)]
        si = [g.normal((1, ctx, DI), dtype=bf) for _ in range(4)]
        e0, e1 = ev(), ev()
        e0.record()
        csa.csa_compress(s[0], s[1], s[2], s[3], _seq(kv[0], b), ratio=m,
                         overlap=True, rope_dims=R, rope_base=cfg.rope_base)
        csa.csa_compress(si[0], si[1], si[2], si[3], _seq(ik[0], b), ratio=m, overlap=True)
        e1.record()
        torch.cuda.synchronize()
        build_ms += e0.elapsed_time(e1)
        build_bytes += 4 * ctx * (D + DI) * 2 + N * (D + DI) * 2
        del s, si
    for li in range(1, L):
        kv[li].data.copy_(kv[0].data)
        ik[li].data.copy_(ik[0].data)
    torch.cuda.synchronize()

    # ---------------------------------------------------------------- step inputs
    g = Gen(cfg.seed, dev)
    steps_in = []
    for li in range(L):
        d = dict(
            ca=g.normal((B, m, D), dtype=bf), cb=g.normal((B, m, D), dtype=bf), za=g.normal((B, m, D), dtype=bf),
            zb=g.normal((B, m, D), dtype=bf), prev_cb=g.normal((B, m, D), dtype=bf),
            prev_zb=g.normal((B, m, D), dtype=bf),
            ica=g.normal((B, m, DI), dtype=bf), icb=g.normal((B, m, DI), dtype=bf),
            iza=g.normal((B, m, DI), dtype=bf), izb=g.normal((B, m, DI), dtype=bf),
            iprev_cb=g.normal((B, m, DI), dtype=bf), iprev_zb=g.normal((B, m, DI), dtype=bf),
            q=g.normal((B, 1, H, D), qstd(D), dtype=bf), qI=g.normal((B, 1, HI, DI), qstd(DI), dtype=bf),
            wI=g.uniform((B, 1, HI)), win=g.normal((B, W, D), dtype=bf), sink=g.normal((H,)),
        )
        d.update(kv_cache=kv[li], ik_cache=ik[li], q_pos=torch.full((B, 1), t_new, dtype=torch.int64, device=dev),
                 win_pos0=torch.full((B,), t_new - W + 1, dtype=torch.int64, device=dev),
                 out=torch.empty((B, 1, H, D), dtype=bf, device=dev))
        steps_in.append(d)
    desc = csa.layer_desc(mode=csa.CSA_MODE_CSA, B=B, T=m, t0=t0, Tq=1, cache_rows=N, Tw=W, D=D, H=H, HI=HI, DI=DI,
                          ratio=m, topk=k, n_win=W, rope_dims=R, rope_base=cfg.rope_base,
                          softmax_scale=cfg.softmax_scale, pos_offset=0, stream_dtype=csa.CSA_BF16)
    ws = torch.empty(csa.csa_forward_workspace_size(desc), dtype=torch.uint8, device=dev)

    def step(i):
        csa.csa_forward(desc, steps_in[i % L], ws=ws)

    # ---------------------------------------------------------------- timed steps
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = ev(), ev()
    wall0 = time.perf_counter()
    e0.record()
    for i in range(args.steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = e0.elapsed_time(e1) / args.steps
    value = B / (ms_per_step * 1e-3)
    log(f"decode step {ms_per_step * 1e3:.1f} us ({wall / args.steps * 1e6:.1f} us wall) -> {value:,.0f} tokens/s")

    # ---------------------------------------------------------------- stages
    scores = torch.empty((B, 1, N), dtype=torch.float32, device=dev)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    outs = torch.empty((B, 1, H, D), dtype=bf, device=dev)
    mqa_ws = torch.empty(max(1, csa.lib().csa_sparse_mqa_workspace_size(B, 1, H, D, k, W)), dtype=torch.uint8,
                         device=dev)

    def st_compress(i):
        d = steps_in[i % L]
        csa.csa_compress(d["ca"], d["cb"], d["za"], d["zb"], kv[i % L], ratio=m, overlap=True, t0=t0,
                         prev_cb=d["prev_cb"], prev_zb=d["prev_zb"], rope_dims=R, rope_base=cfg.rope_base)
        csa.csa_compress(d["ica"], d["icb"], d["iza"], d["izb"], ik[i % L], ratio=m, overlap=True, t0=t0,
                         prev_cb=d["iprev_cb"], prev_zb=d["iprev_zb"])

    def st_index(i):
        d = steps_in[i % L]
        csa.csa_index_scores(d["qI"], d["wI"], ik[i % L], d["q_pos"], scores, ratio=m)

    def st_topk(i):
        csa.csa_topk(scores, k, idx)

    def st_mqa(i):
        d = steps_in[i % L]
        csa.csa_sparse_mqa(d["q"], d["q_pos"], kv[i % L], idx, d["win"], d["win_pos0"], d["sink"], outs, N=N,
                           n_win=W, softmax_scale=cfg.softmax_scale, rope_dims=R, rope_base=cfg.rope_base, ws=mqa_ws)

    def timeit(fn, reps):
        for i in range(3):
            fn(i)
        torch.cuda.synchronize()
        a, b_ = ev(), ev()
        a.record()
        for i in range(reps):
            fn(i)
        b_.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b_) / reps * 1e-3  # seconds per call

    st_index(0)
    st_topk(0)
    torch.cuda.synchronize()
    reps = args.stage_reps
    t_comp = timeit(st_compress, reps)
    t_idx = timeit(st_index, reps)
    t_topk = timeit(st_topk, reps)
    t_mqa = timeit(st_mqa, reps)

    # algorithmic work per launch (what the method must move / compute)
    stages = {
        "compress": dict(t=t_comp, bytes=B * (2 * m * 2 * (D + DI) * 2 + (D + DI) * 2), flops=0.0,
                         kernel="compress_kernel", src=("compress.hip",)),
        "index_scores": dict(t=t_idx, bytes=B * (N * DI * 2 + HI * DI * 2 + HI * 4 + N * 4),
                             flops=2.0 * B * HI * DI * N, kernel="index_mfma_kernel", src=("indexer.hip",)),
        "topk": dict(t=t_topk, bytes=B * (N * 4 + k * 4), flops=0.0, kernel="topk_kernel", src=("topk.hip",)),
        "sparse_mqa": dict(t=t_mqa, bytes=B * ((k + W) * D * 2 + 2 * H * D * 2 + k * 4),
                           flops=4.0 * B * H * (k + W) * D, kernel="attn_mfma_kernel", src=("mqa.hip",)),
    }
    stage_out = {}
    for name, s in stages.items():
        gbs = s["bytes"] / s["t"] / 1e9
        tfs = s["flops"] / s["t"] / 1e12
        bound = "mfma" if s["flops"] / MFMA_BF16_PEAK > s["bytes"] / HBM_PEAK else "hbm"
        stage_out[name] = dict(us=round(s["t"] * 1e6, 2), GBps=round(gbs, 1), TFLOPs=round(tfs, 2),
                               hbm_frac=round(s["bytes"] / s["t"] / HBM_PEAK, 4),
                               mfma_frac=round(s["flops"] / s["t"] / MFMA_BF16_PEAK, 4), bound=bound)
        log(f"  {name:13s} {s['t'] * 1e6:8.2f} us  {gbs:8.1f} GB/s  {tfs:7.2f} TFLOP/s  ({bound}-bound)")
    dom_name = max(stages, key=lambda n: stages[n]["t"])
    dom = stages[dom_name]
    if stage_out[dom_name]["bound"] == "hbm":
        achieved, peak, unit = dom["bytes"] / dom["t"] / 1e9, HBM_PEAK / 1e9, "GB/s"
    else:
        achieved, peak, unit = dom["flops"] / dom["t"] / 1e12, MFMA_BF16_PEAK / 1e12, "TFLOP/s"
    traffic = read_traffic(f"{dom['kernel']}_{WORKLOAD_TAG}_pmc.txt", src_hash(*dom["src"]))
    roofline = dict(kernel=dom["kernel"], stage=dom_name, bound=stage_out[dom_name]["bound"],
                    achieved=round(achieved, 2), peak=peak, unit=unit, frac=round(achieved / peak, 4),
                    traffic=traffic, algorithmic_bytes=dom["bytes"], avg_launch_us=round(dom["t"] * 1e6, 2))

    if args.copy_probe:
        # a plain elementwise kernel of known traffic (reads 1 GiB, writes 1 GiB): the
        # reference for scaling the FETCH_SIZE / WRITE_SIZE counters
        src = torch.zeros(COPY_PROBE_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        log("copy probe: 3 x neg over 1 GiB done")

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, args.cpu_seconds, dev)

    cache_build = dict(us=round(build_ms * 1e3, 1), GBps=round(build_bytes / (build_ms * 1e-3) / 1e9, 1),
                       hbm_frac=round(build_bytes / (build_ms * 1e-3) / HBM_PEAK, 4),
                       bytes=build_bytes)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": cfg.name, "B": B, "context": ctx, "m": m, "entries": N, "D": D, "rope_dims": R,
                   "indexer": f"{HI}x{DI}", "topk": k, "heads": H, "window": W, "layers_cycled": L,
                   "step": "csa_forward: compress newest block + index + top-k + sparse MQA"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "stages": stage_out,
        "cache_build_compress": cache_build,
    }
    print(json.dumps(line), flush=True)


def _seq(buf, b):
    """csa_buf view of sequence b of a [B, rows, D] buffer (as a batch of one)."""
    import compressed_sparse_attention_07_amd as csa
    sl = lambda t: None if t is None else t[b:b + 1]
    return csa.Buf(buf.dtype, sl(buf.data), sl(buf.rope), sl(buf.scale))


def cpu_baseline(cfg, seconds, dev):
    """Time the fp64 oracle's decode step (same workload) for about `seconds` of CPU work.

    The oracle builds sequence 0's caches from the same seeded streams (untimed).
    Then decode steps with fresh seeded inputs (new block, queries, window, sink)
    are timed one after another -- compress the newest block, score every entry,
    top-k, MQA over the selection and the window -- until `seconds` have been spent.
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
    m, D, R, ctx, DI, W = cfg.m, cfg.D, cfg.R, cfg.ctx, cfg.DI, cfg.n_win
    bf = torch.bfloat16
    t0 = ctx - m
    g = Gen(cfg.seed * 1000, dev)
    s = [f(g.normal((1, ctx, D), dtype=bf)[0]) for _ in range(4)]
    si = [f(g.normal((1, ctx, DI), dtype=bf)[0]) for _ in range(4)]
    log("cpu baseline: oracle cache build for sequence 0 (untimed)")
    kv = O.compress(*s, ratio=m, overlap=True, rope_dims=R, rope_base=cfg.rope_base)
    ik = O.compress(*si, ratio=m, overlap=True)
    del s, si
    pos = np.array([ctx])
    total, steps = 0.0, 0
    while total < seconds and steps < 100000:
        g = Gen(cfg.seed * 7919 + steps, dev)
        blk = [f(g.normal((m, D), dtype=bf)) for _ in range(6)]
        iblk = [f(g.normal((m, DI), dtype=bf)) for _ in range(6)]
        q = f(g.normal((1, cfg.H, D), qstd(D), dtype=bf))
        qI = f(g.normal((1, cfg.HI, DI), qstd(DI), dtype=bf))
        wI = f(g.uniform((1, cfg.HI)))
        win = f(g.normal((W, D), dtype=bf))
        sink = f(g.normal((cfg.H,)))
        tic = time.perf_counter()
        e = O.compress(*blk[:4], ratio=m, overlap=True, t0=t0, prev_cb=blk[4], prev_zb=blk[5], rope_dims=R,
                       rope_base=cfg.rope_base)
        kv[-1] = e[0]
        ei = O.compress(*iblk[:4], ratio=m, overlap=True, t0=t0, prev_cb=iblk[4], prev_zb=iblk[5])
        ik[-1] = ei[0]
        sc = O.index_scores(qI, wI, ik, pos, m)
        idx, _ = O.topk(sc, cfg.k)
        O.mqa(q, pos, kv, idx, win, ctx - W + 1, W, sink, scale=cfg.softmax_scale, rope_dims=R,
              rope_base=cfg.rope_base)
        total += time.perf_counter() - tic
        steps += 1
    rate = steps / total
    log(f"cpu baseline: {steps} decode steps in {total:.2f} s -> {rate:.2f} tokens/s ({threads} BLAS threads, "
        f"{cores} cores)")
    return dict(value=round(rate, 3), unit="tokens/s", cores=threads, host_cores=cores, kind="oracle",
                seconds=round(total, 2),
                sample=f"{steps} decode steps of sequence 0 (fresh seeded block, queries, window and sink per "
                       f"step): compress the newest block, score {ctx // m} entries, top-{cfg.k}, MQA over "
                       f"{cfg.k}+{W} keys; the oracle's caches are built once, untimed")


if __name__ == "__main__":
    main()
