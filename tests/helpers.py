"""Shared test utilities: library loading, tolerance checks, top-k tie rule."""

from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def ensure_built():
    """Load the in-tree library; build it only if nothing is built."""
    from compressed_sparse_attention_07_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from compressed_sparse_attention_07_amd import build
        build.build()
    return _lib.lib()


def f64(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


# tolerances: |got - want| <= atol + rtol * |want|
TOL = {
    "f32": dict(rtol=1e-4, atol_rms=1e-4),
    "bf16": dict(rtol=2e-2, atol=2e-2),
    "fp8": dict(rtol=5e-2, atol=5e-2),
}


def assert_close(got, want, kind: str, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    t = TOL[kind]
    if "atol_rms" in t:
        rms = np.sqrt(np.mean(want ** 2)) if want.size else 0.0
        atol = t["atol_rms"] * rms
    else:
        atol = t["atol"]
    err = np.abs(got - want)
    bad = ~(err <= atol + t["rtol"] * np.abs(want))
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err, -1)), err.shape)
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside {kind} tolerance; "
                             f"worst at {i}: got {got[i]!r} want {want[i]!r}")


def topk_sets_agree(gpu_idx, gpu_cnt, oracle_scores, k, band_rel=1e-4, band_abs=None):
    """Compare a GPU top-k row with the oracle's scores under the near-tie rule.

    Returns (ok, exact): counts must match; every index in the symmetric difference
    of the two sets must have an oracle score within the band of the k-th score.
    """
    s = np.asarray(oracle_scores, dtype=np.float64)
    fin = np.isfinite(s)
    want_cnt = min(k, int(fin.sum()))
    if int(gpu_cnt) != want_cnt:
        return False, False
    g = set(int(x) for x in gpu_idx[:want_cnt])
    if any(x < 0 for x in g) or len(g) != want_cnt:
        return False, False
    order = np.nonzero(fin)[0]
    order = order[np.lexsort((order, -s[order]))]
    o = set(int(x) for x in order[:want_cnt])
    diff = g ^ o
    if not diff:
        return True, True
    kth = s[order[want_cnt - 1]]
    band = band_rel * abs(kth) + (band_abs or 0.0)
    ok = all(np.isfinite(s[i]) and abs(s[i] - kth) <= band for i in diff)
    return ok, False
