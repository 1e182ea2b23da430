"""ctypes binding of libcsa.so: argument marshalling only.

Every function here forwards torch tensors (device memory owned by the caller) and
the current HIP stream to the C entry point of the same name in include/csa.h.
No step of the computation happens in Python; if the library is missing the call
raises instead of falling back to anything else.
"""

from __future__ import annotations

import ctypes as C
import os

import torch

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libcsa.so")

CSA_F32, CSA_BF16, CSA_FP8MIX, CSA_MXFP4 = 0, 1, 2, 3
CSA_MODE_CSA, CSA_MODE_HCA = 0, 1
CSA_FLAG_BF16_SCORES = 1
CSA_FLAG_QKV_NORM = 2
STATUS = {0: "CSA_OK", 1: "CSA_ERR_NULL", 2: "CSA_ERR_SHAPE", 3: "CSA_ERR_DTYPE",
          4: "CSA_ERR_WORKSPACE", 5: "CSA_ERR_DEVICE", 6: "CSA_ERR_UNSUPPORTED"}

EXPORTS = ["csa_abi_version", "csa_last_error", "csa_device_check", "csa_compress", "csa_compress_norm", "csa_rmsnorm",
           "csa_grouped_out_proj_workspace_size", "csa_grouped_out_proj", "csa_quantize",
           "csa_index_scores", "csa_topk_workspace_size", "csa_topk", "csa_index_topk_workspace_size", "csa_index_topk", "csa_sparse_mqa_workspace_size",
           "csa_sparse_mqa", "csa_sparse_mqa_noalloc", "csa_sparse_mqa_noalloc_limit", "hca_dense_attn_workspace_size",
           "hca_dense_attn",
           "csa_forward_workspace_size", "csa_forward", "csa_decode_step_workspace_size", "csa_decode_step"]


class CSAError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


class csa_buf(C.Structure):
    _fields_ = [("data", C.c_void_p), ("rope", C.c_void_p), ("scale", C.c_void_p),
                ("dtype", C.c_int32), ("reserved", C.c_int32)]


class csa_layer_desc(C.Structure):
    _fields_ = [("struct_size", C.c_int32), ("mode", C.c_int32),
                ("B", C.c_int64), ("T", C.c_int64), ("t0", C.c_int64), ("Tq", C.c_int64),
                ("cache_rows", C.c_int64), ("Tw", C.c_int64),
                ("D", C.c_int32), ("H", C.c_int32), ("HI", C.c_int32), ("DI", C.c_int32),
                ("ratio", C.c_int32), ("topk", C.c_int32), ("n_win", C.c_int32), ("rope_dims", C.c_int32),
                ("rope_base", C.c_float), ("softmax_scale", C.c_float), ("pos_offset", C.c_int64),
                ("stream_dtype", C.c_int32), ("flags", C.c_int32), ("norm_eps", C.c_float),
                ("reserved", C.c_int32)]


class csa_forward_io(C.Structure):
    _fields_ = [("ca", C.c_void_p), ("cb", C.c_void_p), ("za", C.c_void_p), ("zb", C.c_void_p),
                ("bias_a", C.c_void_p), ("bias_b", C.c_void_p), ("prev_cb", C.c_void_p), ("prev_zb", C.c_void_p),
                ("ica", C.c_void_p), ("icb", C.c_void_p), ("iza", C.c_void_p), ("izb", C.c_void_p),
                ("ibias_a", C.c_void_p), ("ibias_b", C.c_void_p), ("iprev_cb", C.c_void_p), ("iprev_zb", C.c_void_p),
                ("kv_cache", csa_buf), ("ik_cache", csa_buf), ("q", csa_buf), ("q_pos", C.c_void_p),
                ("qI", csa_buf), ("wI", C.c_void_p), ("win", csa_buf), ("win_pos0", C.c_void_p),
                ("sink", C.c_void_p), ("out", csa_buf), ("scores_out", C.c_void_p), ("idx_out", C.c_void_p),
                ("q_norm", C.c_void_p), ("kv_norm", C.c_void_p)]


class csa_decode_desc(C.Structure):
    _fields_ = [("struct_size", C.c_int32), ("mode", C.c_int32), ("B", C.c_int64), ("slots", C.c_int64),
                ("pages", C.c_int64), ("max_pages", C.c_int32), ("page_tokens", C.c_int32),
                ("D", C.c_int32), ("H", C.c_int32), ("HI", C.c_int32), ("DI", C.c_int32),
                ("ratio", C.c_int32), ("topk", C.c_int32), ("n_win", C.c_int32), ("rope_dims", C.c_int32),
                ("rope_base", C.c_float), ("softmax_scale", C.c_float), ("pos_offset", C.c_int64),
                ("stream_dtype", C.c_int32), ("flags", C.c_int32), ("norm_eps", C.c_float), ("reserved", C.c_int32)]


class csa_decode_io(C.Structure):
    _fields_ = [("slot", C.c_void_p), ("length", C.c_void_p),
                ("ca", C.c_void_p), ("cb", C.c_void_p), ("za", C.c_void_p), ("zb", C.c_void_p),
                ("bias_a", C.c_void_p), ("bias_b", C.c_void_p),
                ("ica", C.c_void_p), ("icb", C.c_void_p), ("iza", C.c_void_p), ("izb", C.c_void_p),
                ("ibias_a", C.c_void_p), ("ibias_b", C.c_void_p), ("kv_raw", csa_buf),
                ("tail", C.c_void_p), ("itail", C.c_void_p), ("win", csa_buf), ("win_pos0", C.c_void_p),
                ("kv_pages", csa_buf), ("ik_pages", csa_buf), ("block_table", C.c_void_p),
                ("q", csa_buf), ("qI", csa_buf), ("wI", C.c_void_p), ("sink", C.c_void_p), ("out", csa_buf),
                ("q_norm", C.c_void_p), ("kv_norm", C.c_void_p), ("idx_out", C.c_void_p), ("scores_out", C.c_void_p)]


_lib = None


def lib():
    """Load libcsa.so (built in-tree); raise loudly if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m compressed_sparse_attention_07_amd.build`")
        L = C.CDLL(LIB_PATH)
        vp, i32, i64, f32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t
        bp = C.POINTER(csa_buf)
        L.csa_abi_version.restype = C.c_int
        L.csa_last_error.restype = C.c_char_p
        L.csa_device_check.restype = C.c_int
        L.csa_compress.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, i64, i64, i32, i32, i32, i64, i32, f32, i64,
                                   bp, i64, vp]
        L.csa_compress_norm.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, vp, i64, i64, i32, i32, i32, i64, i32, f32,
                                        i64, vp, f32, bp, i64, vp]
        L.csa_rmsnorm.argtypes = [bp, i64, i32, vp, f32, bp, vp]
        L.csa_grouped_out_proj_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
        L.csa_grouped_out_proj_workspace_size.restype = sz
        L.csa_grouped_out_proj.argtypes = [bp, vp, vp, i64, i32, i32, i32, i32, i32, bp, vp, sz, vp]
        L.csa_quantize.argtypes = [vp, i64, i32, i32, bp, vp]
        L.csa_index_scores.argtypes = [bp, vp, bp, vp, i64, i64, i32, i32, i64, i64, i32, vp, vp]
        L.csa_topk_workspace_size.argtypes = [i64, i64, i32]
        L.csa_topk_workspace_size.restype = sz
        L.csa_topk.argtypes = [vp, i64, i64, i32, vp, vp, vp, sz, vp]
        L.csa_index_topk_workspace_size.argtypes = [i64, i64, i32, i32, i64, i32, i32, i32]
        L.csa_index_topk_workspace_size.restype = sz
        L.csa_index_topk.argtypes = [bp, vp, bp, vp, i64, i64, i32, i32, i64, i64, i32, i32, i32, vp, vp, vp, vp, sz, vp]
        L.csa_sparse_mqa_workspace_size.argtypes = [i64, i64, i32, i32, i32, i32]
        L.csa_sparse_mqa_workspace_size.restype = sz
        L.csa_sparse_mqa.argtypes = [bp, vp, bp, i64, vp, i32, bp, vp, i64, vp, f32, i32, f32, i64, i64, i64, i32,
                                     i32, i64, i32, bp, vp, sz, vp]
        L.csa_sparse_mqa_noalloc.argtypes = [bp, vp, bp, i64, vp, i32, bp, vp, i64, vp, f32, i32, f32, i64, i64, i64,
                                             i32, i32, i64, i32, bp, vp]
        L.csa_sparse_mqa_noalloc_limit.argtypes = []
        L.csa_sparse_mqa_noalloc_limit.restype = sz
        L.hca_dense_attn_workspace_size.argtypes = [i64, i64, i32, i32, i64, i32]
        L.hca_dense_attn_workspace_size.restype = sz
        L.hca_dense_attn.argtypes = [bp, vp, bp, i64, i32, bp, vp, i64, vp, f32, i32, f32, i64, i64, i64, i32, i32,
                                     i64, i32, bp, vp, sz, vp]
        L.csa_forward_workspace_size.argtypes = [C.POINTER(csa_layer_desc)]
        L.csa_forward_workspace_size.restype = sz
        L.csa_forward.argtypes = [C.POINTER(csa_layer_desc), C.POINTER(csa_forward_io), vp, sz, vp]
        L.csa_decode_step_workspace_size.argtypes = [C.POINTER(csa_decode_desc)]
        L.csa_decode_step_workspace_size.restype = sz
        L.csa_decode_step.argtypes = [C.POINTER(csa_decode_desc), C.POINTER(csa_decode_io), vp, sz, vp]
        for name in EXPORTS:
            if name not in ("csa_topk_workspace_size", "csa_sparse_mqa_workspace_size", "csa_index_topk_workspace_size",
                            "csa_grouped_out_proj_workspace_size", "csa_decode_step_workspace_size",
                            "csa_sparse_mqa_noalloc_limit",
                            "hca_dense_attn_workspace_size", "csa_forward_workspace_size",
                            "csa_last_error", "csa_abi_version"):
                getattr(L, name).restype = C.c_int
        _lib = L
    return _lib


def check(status: int) -> None:
    if status != 0:
        raise CSAError(status, lib().csa_last_error().decode())


# While a PreparedCall is being built, entry points record their C call here instead
# of making it.
_recording: list | None = None


def _invoke(name: str, *args, keep=()) -> None:
    fn = getattr(lib(), name)
    if _recording is not None:
        _recording.append((fn, args, keep))
        return
    check(fn(*args))


def ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def stream_handle(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


# ------------------------------------------------------------------ buffers


class Buf:
    """A tensor (or tensor triple) in one of the library's storage formats."""

    def __init__(self, dtype: int, data, rope=None, scale=None):
        self.dtype, self.data, self.rope, self.scale = dtype, data, rope, scale

    @property
    def shape(self):
        if self.dtype in (CSA_F32, CSA_BF16):
            return tuple(self.data.shape)
        if self.dtype == CSA_FP8MIX:
            return tuple(self.data.shape[:-1]) + (self.data.shape[-1] + self.rope.shape[-1],)
        return tuple(self.data.shape[:-1]) + (2 * self.data.shape[-1],)

    def rows(self, lo: int, hi: int) -> "Buf":
        """View of rows [lo, hi) along dim 1 (the per-sequence row axis)."""
        sl = lambda t: None if t is None else t[:, lo:hi]
        return Buf(self.dtype, sl(self.data), sl(self.rope), sl(self.scale))

    def c(self) -> csa_buf:
        return csa_buf(ptr(self.data), ptr(self.rope), ptr(self.scale), self.dtype, 0)

    @staticmethod
    def of(t) -> "Buf":
        if isinstance(t, Buf):
            return t
        if t.dtype == torch.float32:
            return Buf(CSA_F32, t)
        if t.dtype == torch.bfloat16:
            return Buf(CSA_BF16, t)
        raise TypeError(f"unsupported tensor dtype {t.dtype}")

    @staticmethod
    def empty(shape, dtype: int, rope_dims: int = 0, device="cuda") -> "Buf":
        *lead, D = shape
        lead = tuple(lead)
        if dtype == CSA_F32:
            return Buf(dtype, torch.empty(lead + (D,), dtype=torch.float32, device=device))
        if dtype == CSA_BF16:
            return Buf(dtype, torch.empty(lead + (D,), dtype=torch.bfloat16, device=device))
        if dtype == CSA_FP8MIX:
            return Buf(dtype, torch.empty(lead + (D - rope_dims,), dtype=torch.uint8, device=device),
                       torch.empty(lead + (rope_dims,), dtype=torch.bfloat16, device=device),
                       torch.empty(lead, dtype=torch.float32, device=device))
        if dtype == CSA_MXFP4:
            return Buf(dtype, torch.empty(lead + (D // 2,), dtype=torch.uint8, device=device), None,
                       torch.empty(lead + (D // 32,), dtype=torch.uint8, device=device))
        raise ValueError(dtype)


def _ws(nbytes: int, device, ws=None):
    if nbytes == 0:
        return None, 0
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def _dt(t) -> int:
    return Buf.of(t).dtype


# ------------------------------------------------------------------ entry points


def csa_compress(ca, cb, za, zb, out: Buf, *, ratio: int, overlap: bool, t0: int = 0, bias_a=None, bias_b=None,
                 prev_cb=None, prev_zb=None, rope_dims: int = 0, rope_base: float = 10000.0, pos_offset: int = 0,
                 stream=None) -> None:
    B, T, D = ca.shape
    out_rows = out.shape[1]
    bo = out.c()
    _invoke("csa_compress", ptr(ca), ptr(cb), ptr(za), ptr(zb), _dt(ca), ptr(bias_a), ptr(bias_b), ptr(prev_cb),
            ptr(prev_zb), B, T, D, ratio, 1 if overlap else 0, t0, rope_dims, rope_base, pos_offset, C.byref(bo),
            out_rows, stream_handle(stream))


def csa_compress_norm(ca, cb, za, zb, out: Buf, *, ratio: int, overlap: bool, norm_weight, norm_eps: float = 1e-6,
                      t0: int = 0, bias_a=None, bias_b=None, prev_cb=None, prev_zb=None, rope_dims: int = 0,
                      rope_base: float = 10000.0, pos_offset: int = 0, stream=None) -> None:
    B, T, D = ca.shape
    out_rows = out.shape[1]
    bo = out.c()
    _invoke("csa_compress_norm", ptr(ca), ptr(cb), ptr(za), ptr(zb), _dt(ca), ptr(bias_a), ptr(bias_b), ptr(prev_cb),
            ptr(prev_zb), B, T, D, ratio, 1 if overlap else 0, t0, rope_dims, rope_base, pos_offset,
            ptr(norm_weight), norm_eps, C.byref(bo), out_rows, stream_handle(stream))


def csa_rmsnorm(x, weight, out, *, eps: float = 1e-6, stream=None) -> None:
    xb, ob = Buf.of(x), Buf.of(out)
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    cx, co = xb.c(), ob.c()
    _invoke("csa_rmsnorm", C.byref(cx), rows, D, ptr(weight), eps, C.byref(co), stream_handle(stream))


def csa_grouped_out_proj_workspace_size(T: int, n_h: int, c: int, g: int, d_g: int, d: int) -> int:
    return lib().csa_grouped_out_proj_workspace_size(T, n_h, c, g, d_g, d)


def csa_grouped_out_proj(o, w_group, w_out, out, *, ws=None, stream=None) -> None:
    """o [T, n_h, c] bf16; w_group [g, d_g, (n_h/g) c] bf16; w_out [d, g d_g] bf16; out [T, d]."""
    T, n_h, c = o.shape
    g, d_g, _ = w_group.shape
    d = w_out.shape[0]
    need = csa_grouped_out_proj_workspace_size(T, n_h, c, g, d_g, d)
    w, wbytes = _ws(need, o.device, ws)
    co, cout = Buf.of(o).c(), Buf.of(out).c()
    _invoke("csa_grouped_out_proj", C.byref(co), ptr(w_group), ptr(w_out), T, n_h, c, g, d_g, d, C.byref(cout),
            ptr(w), wbytes, stream_handle(stream), keep=(w,))


def csa_quantize(x, out: Buf, *, rope_dims: int = 0, stream=None) -> None:
    D = x.shape[-1]
    rows = x.numel() // D
    bo = out.c()
    _invoke("csa_quantize", ptr(x), rows, D, rope_dims, C.byref(bo), stream_handle(stream))


def csa_index_scores(qI, wI, kI, q_pos, scores, *, ratio: int, stream=None) -> None:
    qb, kb = Buf.of(qI), Buf.of(kI)
    B, Tq, HI, DI = qb.shape
    _, kI_rows, _ = kb.shape
    N = scores.shape[-1]
    cq, ck = qb.c(), kb.c()
    _invoke("csa_index_scores", C.byref(cq), ptr(wI), C.byref(ck), ptr(q_pos), B, Tq, HI, DI, N, kI_rows, ratio,
            ptr(scores), stream_handle(stream))


def csa_topk(scores, k: int, idx, count=None, *, ws=None, stream=None) -> None:
    N = scores.shape[-1]
    rows = 1
    for d in scores.shape[:-1]:
        rows *= d
    need = lib().csa_topk_workspace_size(rows, N, k)
    w, wb = _ws(need, scores.device, ws)
    _invoke("csa_topk", ptr(scores), rows, N, k, ptr(idx), ptr(count), ptr(w), wb, stream_handle(stream), keep=(w,))


def csa_index_topk(qI, wI, kI, q_pos, k: int, idx, count=None, scores=None, *, N: int, ratio: int, flags: int = 0,
                   ws=None, stream=None) -> None:
    qb, kb = Buf.of(qI), Buf.of(kI)
    B, Tq, HI, DI = qb.shape
    _, kI_rows, _ = kb.shape
    need = lib().csa_index_topk_workspace_size(B, Tq, HI, DI, N, k, qb.dtype, flags)
    w, wbytes = _ws(need, qb.data.device, ws)
    cq, ck = qb.c(), kb.c()
    _invoke("csa_index_topk", C.byref(cq), ptr(wI), C.byref(ck), ptr(q_pos), B, Tq, HI, DI, N, kI_rows, ratio, k, flags,
            ptr(idx), ptr(count), ptr(scores), ptr(w), wbytes, stream_handle(stream), keep=(w,))


def csa_sparse_mqa(q, q_pos, kv, idx, win, win_pos0, sink, out, *, N: int, n_win: int, softmax_scale: float,
                   rope_dims: int, rope_base: float = 10000.0, pos_offset: int = 0, ws=None, stream=None) -> None:
    qb, kvb, wb_, ob = Buf.of(q), Buf.of(kv), Buf.of(win), Buf.of(out)
    B, Tq, H, D = qb.shape
    kv_rows = kvb.shape[1]
    Tw = wb_.shape[1]
    K = idx.shape[-1]
    need = lib().csa_sparse_mqa_workspace_size(B, Tq, H, D, K, n_win)
    w, wbytes = _ws(need, q.device if not isinstance(q, Buf) else q.data.device, ws)
    cq, ck, cw, co = qb.c(), kvb.c(), wb_.c(), ob.c()
    _invoke("csa_sparse_mqa", C.byref(cq), ptr(q_pos), C.byref(ck), kv_rows, ptr(idx), K, C.byref(cw),
            ptr(win_pos0), Tw, ptr(sink), softmax_scale, rope_dims, rope_base, pos_offset, B, Tq, H, D, N, n_win,
            C.byref(co), ptr(w), wbytes, stream_handle(stream), keep=(w,))


def csa_sparse_mqa_noalloc(q, q_pos, kv, idx, win, win_pos0, sink, out, *, N: int, n_win: int, softmax_scale: float,
                           rope_dims: int, rope_base: float = 10000.0, pos_offset: int = 0, stream=None) -> None:
    qb, kvb, wb_, ob = Buf.of(q), Buf.of(kv), Buf.of(win), Buf.of(out)
    B, Tq, H, D = qb.shape
    kv_rows = kvb.shape[1]
    Tw = wb_.shape[1]
    K = idx.shape[-1]
    cq, ck, cw, co = qb.c(), kvb.c(), wb_.c(), ob.c()
    _invoke("csa_sparse_mqa_noalloc", C.byref(cq), ptr(q_pos), C.byref(ck), kv_rows, ptr(idx), K, C.byref(cw),
            ptr(win_pos0), Tw, ptr(sink), softmax_scale, rope_dims, rope_base, pos_offset, B, Tq, H, D, N, n_win,
            C.byref(co), stream_handle(stream))


def hca_dense_attn(q, q_pos, kv, win, win_pos0, sink, out, *, N: int, ratio: int, n_win: int, softmax_scale: float,
                   rope_dims: int, rope_base: float = 10000.0, pos_offset: int = 0, ws=None, stream=None) -> None:
    qb, kvb, wb_, ob = Buf.of(q), Buf.of(kv), Buf.of(win), Buf.of(out)
    B, Tq, H, D = qb.shape
    kv_rows = kvb.shape[1]
    Tw = wb_.shape[1]
    need = lib().hca_dense_attn_workspace_size(B, Tq, H, D, N, n_win)
    w, wbytes = _ws(need, qb.data.device, ws)
    cq, ck, cw, co = qb.c(), kvb.c(), wb_.c(), ob.c()
    _invoke("hca_dense_attn", C.byref(cq), ptr(q_pos), C.byref(ck), kv_rows, ratio, C.byref(cw), ptr(win_pos0),
            Tw, ptr(sink), softmax_scale, rope_dims, rope_base, pos_offset, B, Tq, H, D, N, n_win, C.byref(co),
            ptr(w), wbytes, stream_handle(stream), keep=(w,))


def layer_desc(**kw) -> csa_layer_desc:
    d = csa_layer_desc()
    d.struct_size = C.sizeof(csa_layer_desc)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def csa_forward_workspace_size(desc: csa_layer_desc) -> int:
    return lib().csa_forward_workspace_size(C.byref(desc))


def _forward_io(io: dict) -> csa_forward_io:
    cio = csa_forward_io()
    for name, val in io.items():
        if val is None:
            continue
        if isinstance(val, Buf) or (name in ("kv_cache", "ik_cache", "q", "qI", "win", "out")):
            setattr(cio, name, Buf.of(val).c())
        else:
            setattr(cio, name, ptr(val))
    return cio


def csa_forward(desc: csa_layer_desc, io: dict, *, ws=None, stream=None) -> None:
    """io maps csa_forward_io field names to tensors / Buf objects (missing = NULL)."""
    cio = _forward_io(io)
    need = csa_forward_workspace_size(desc)
    dev = Buf.of(io["q"]).data.device
    w, wbytes = _ws(need, dev, ws)
    _invoke("csa_forward", C.byref(desc), C.byref(cio), ptr(w), wbytes, stream_handle(stream), keep=(w, io))


def decode_desc(**kw) -> csa_decode_desc:
    d = csa_decode_desc()
    d.struct_size = C.sizeof(csa_decode_desc)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def csa_decode_step_workspace_size(desc: csa_decode_desc) -> int:
    return lib().csa_decode_step_workspace_size(C.byref(desc))


_DECODE_BUFS = ("kv_raw", "win", "kv_pages", "ik_pages", "q", "qI", "out")


def _decode_io(io: dict) -> csa_decode_io:
    cio = csa_decode_io()
    for name, val in io.items():
        if val is None:
            continue
        if name in _DECODE_BUFS:
            setattr(cio, name, Buf.of(val).c())
        else:
            setattr(cio, name, ptr(val))
    return cio


def csa_decode_step(desc: csa_decode_desc, io: dict, *, ws=None, stream=None) -> None:
    """io maps csa_decode_io field names to tensors / Buf objects (missing = NULL)."""
    cio = _decode_io(io)
    need = csa_decode_step_workspace_size(desc)
    dev = Buf.of(io["q"]).data.device
    w, wbytes = _ws(need, dev, ws)
    _invoke("csa_decode_step", C.byref(desc), C.byref(cio), ptr(w), wbytes, stream_handle(stream), keep=(w, io))


class DecodePool:
    """Device memory of a decode state pool and its paged caches, laid out as
    csa_decode_step documents (allocation only; every field is a plain tensor)."""

    def __init__(self, *, mode: int, slots: int, pages: int, max_pages: int, page_tokens: int, D: int, DI: int,
                 ratio: int, n_win: int, stream_dtype: int, kv_dtype: int, ik_dtype: int, rope_dims: int = 0,
                 device="cuda"):
        import torch
        st = torch.float32 if stream_dtype == CSA_F32 else torch.bfloat16
        kt = torch.float32 if kv_dtype == CSA_F32 else torch.bfloat16
        P = page_tokens // ratio
        csa_mode = mode == CSA_MODE_CSA
        self.P = P
        self.length = torch.zeros(slots, dtype=torch.int64, device=device)
        ring, nst = (2 * ratio, 4) if csa_mode else (ratio, 2)
        self.tail = torch.zeros((slots, ring, nst, D), dtype=st, device=device)
        self.itail = torch.zeros((slots, ring, 4, DI), dtype=st, device=device) if csa_mode else None
        if kv_dtype == CSA_FP8MIX:
            self.win = Buf.empty((slots, 2 * n_win, D), kv_dtype, rope_dims=rope_dims, device=device)
        else:
            self.win = torch.zeros((slots, 2 * n_win, D), dtype=kt, device=device)
        self.win_pos0 = torch.zeros(slots, dtype=torch.int64, device=device)
        self.kv_pages = Buf.empty((pages, P, D), kv_dtype, rope_dims=rope_dims, device=device)
        self.ik_pages = Buf.empty((pages, P, DI), ik_dtype, device=device) if csa_mode else None
        self.block_table = torch.full((slots, max_pages), -1, dtype=torch.int32, device=device)

    def io(self) -> dict:
        return dict(length=self.length, tail=self.tail, itail=self.itail, win=self.win, win_pos0=self.win_pos0,
                    kv_pages=self.kv_pages, ik_pages=self.ik_pages, block_table=self.block_table)


class ForwardCall:
    """A csa_forward call with its arguments marshalled once (for repeated launches).

    Holds references to every tensor it points at; the call itself is one C call."""

    def __init__(self, desc: csa_layer_desc, io: dict, *, ws=None, stream=None):
        self.desc = desc
        self.io = dict(io)
        self.cio = _forward_io(self.io)
        need = csa_forward_workspace_size(desc)
        self.w, self.wbytes = _ws(need, Buf.of(io["q"]).data.device, ws)
        self.wptr = ptr(self.w)
        self.stream = stream_handle(stream)
        self.fn = lib().csa_forward
        self.args = (C.byref(self.desc), C.byref(self.cio), self.wptr, self.wbytes, self.stream)

    def __call__(self) -> None:
        st = self.fn(*self.args)
        if st != 0:
            check(st)


class PreparedCall:
    """One entry-point call with its arguments marshalled once, for repeated launches.

    ``PreparedCall(csa_topk, scores, k, idx)`` runs the binding's argument handling
    once and records the C call it would make; calling the object repeats that C call
    on the same buffers. The object holds the tensors the call points at (and any
    workspace the binding allocated) for as long as it lives."""

    def __init__(self, entry, *args, **kwargs):
        global _recording
        if _recording is not None:
            raise RuntimeError("PreparedCall cannot nest")
        _recording = []
        try:
            entry(*args, **kwargs)
            self.calls = _recording
        finally:
            _recording = None
        self.refs = (args, kwargs)

    def __call__(self) -> None:
        for fn, args, _ in self.calls:
            st = fn(*args)
            if st != 0:
                check(st)
