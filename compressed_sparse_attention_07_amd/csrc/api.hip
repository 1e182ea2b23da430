// Host side of libcsa: argument validation, workspace planning and kernel
// launches for every entry point declared in include/csa.h.  Validation is pure
// host arithmetic on the scalar arguments (no device queries apart from one cached
// architecture check per device), so a rejected call costs well under a microsecond
// and launches nothing.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "launch.h"

using namespace csa;

namespace {

thread_local std::string g_err;

csa_status fail(csa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

csa_status ok() {
  g_err.clear();
  return CSA_OK;
}

std::atomic<int> g_dev_state[64];  // 0 unknown, 1 gfx950, 2 other

csa_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return fail(CSA_ERR_DEVICE, "no HIP device is available");
  }
  if (dev < 64) {
    int st = g_dev_state[dev].load(std::memory_order_relaxed);
    if (st == 1) return CSA_OK;
    if (st == 2) return fail(CSA_ERR_DEVICE, "device %d is not a gfx950 (MI355X) GPU", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(CSA_ERR_DEVICE, "cannot query device %d", dev);
  }
  const bool good = std::string(prop.gcnArchName).rfind("gfx950", 0) == 0;
  if (dev < 64) g_dev_state[dev].store(good ? 1 : 2, std::memory_order_relaxed);
  if (!good) return fail(CSA_ERR_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  return CSA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

const char* dt_name(int d) {
  switch (d) {
    case CSA_F32: return "F32";
    case CSA_BF16: return "BF16";
    case CSA_FP8MIX: return "FP8MIX";
    case CSA_MXFP4: return "MXFP4";
  }
  return "?";
}

// Check that a csa_buf carries the pointers its format needs.
csa_status check_buf(const csa_buf* b, const char* name) {
  if (!b) return fail(CSA_ERR_NULL, "%s is NULL", name);
  if (b->dtype < CSA_F32 || b->dtype > CSA_MXFP4) return fail(CSA_ERR_DTYPE, "%s has unknown dtype %d", name, b->dtype);
  if (!b->data) return fail(CSA_ERR_NULL, "%s.data is NULL", name);
  if (b->dtype == CSA_FP8MIX && !b->scale) return fail(CSA_ERR_NULL, "%s (FP8MIX) needs a scale pointer", name);
  if (b->dtype == CSA_MXFP4 && !b->scale) return fail(CSA_ERR_NULL, "%s (MXFP4) needs a scale pointer", name);
  if (!aligned16(b->data) || (b->rope && !aligned16(b->rope)))
    return fail(CSA_ERR_SHAPE, "%s pointers must be 16-byte aligned", name);
  return CSA_OK;
}

csa_status check_rope(int32_t D, int32_t R, float base) {
  if (R < 0 || R > D || (R & 1) || ((D - R) & 1))
    return fail(CSA_ERR_SHAPE, "rope_dims=%d must be even, <= D=%d, with D-rope_dims even", R, D);
  if (R > 128) return fail(CSA_ERR_UNSUPPORTED, "rope_dims=%d: at most 128 RoPE dims are supported", R);
  if (R > 0 && !(base > 0.f && std::isfinite(base))) return fail(CSA_ERR_SHAPE, "rope_base must be positive");
  return CSA_OK;
}

#define CSA_TRY(x)                    \
  do {                                \
    csa_status _s = (x);              \
    if (_s != CSA_OK) return _s;      \
  } while (0)

csa_status validate_compress(const void* ca, const void* cb, const void* za, const void* zb, int32_t in_dtype,
                             const float* bias_a, const float* bias_b, const void* prev_cb, const void* prev_zb,
                             int64_t B, int64_t T, int32_t D, int32_t ratio, int32_t overlap, int64_t t0,
                             int32_t rope_dims, float rope_base, const csa_buf* out, int64_t out_rows) {
  if (!ca || !za) return fail(CSA_ERR_NULL, "ca and za are required");
  if (overlap != 0 && overlap != 1) return fail(CSA_ERR_SHAPE, "overlap must be 0 or 1");
  if (overlap && (!cb || !zb)) return fail(CSA_ERR_NULL, "overlapped compression needs cb and zb");
  if (overlap && t0 > 0 && (!prev_cb || !prev_zb))
    return fail(CSA_ERR_NULL, "overlapped compression from t0 > 0 needs prev_cb and prev_zb");
  CSA_TRY(check_buf(out, "out"));
  if (in_dtype != CSA_F32 && in_dtype != CSA_BF16)
    return fail(CSA_ERR_DTYPE, "compress inputs must be F32 or BF16, got %s", dt_name(in_dtype));
  if (ratio < 1 || ratio > 1024) return fail(CSA_ERR_SHAPE, "ratio=%d out of [1, 1024]", ratio);
  if (D < 8 || D > 2048 || D % 8) return fail(CSA_ERR_SHAPE, "D=%d must be a multiple of 8 in [8, 2048]", D);
  if (B < 0 || T < 0 || t0 < 0) return fail(CSA_ERR_SHAPE, "B, T, t0 must be non-negative");
  if (T % ratio) return fail(CSA_ERR_SHAPE, "T=%lld is not a multiple of ratio=%d", (long long)T, ratio);
  if (t0 % ratio) return fail(CSA_ERR_SHAPE, "t0=%lld is not a multiple of ratio=%d", (long long)t0, ratio);
  CSA_TRY(check_rope(D, rope_dims, rope_base));
  if (out->dtype == CSA_FP8MIX && (D - rope_dims) % 8)
    return fail(CSA_ERR_SHAPE, "FP8MIX output needs D - rope_dims to be a multiple of 8");
  if (out->dtype == CSA_FP8MIX && rope_dims > 0 && !out->rope)
    return fail(CSA_ERR_NULL, "FP8MIX output with rope_dims > 0 needs a rope pointer");
  if (out->dtype == CSA_MXFP4 && D % 32) return fail(CSA_ERR_SHAPE, "MXFP4 output needs D %% 32 == 0");
  if (out_rows < (t0 + T) / ratio)
    return fail(CSA_ERR_SHAPE, "out_rows=%lld < (t0+T)/ratio=%lld", (long long)out_rows, (long long)((t0 + T) / ratio));
  const void* ptrs[] = {ca, cb, za, zb, prev_cb, prev_zb, bias_a, bias_b};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(CSA_ERR_SHAPE, "compress inputs must be 16-byte aligned");
  return CSA_OK;
}

csa_status validate_attn(const csa_buf* q, const int64_t* q_pos, const csa_buf* kv, int64_t kv_rows,
                         const csa_buf* win, const int64_t* win_pos0, int64_t Tw, const float* sink,
                         int32_t rope_dims, float rope_base, int64_t B, int64_t Tq, int32_t H, int32_t D, int64_t N,
                         int32_t n_win, const csa_buf* out) {
  CSA_TRY(check_buf(q, "q"));
  CSA_TRY(check_buf(kv, "kv"));
  CSA_TRY(check_buf(win, "win"));
  CSA_TRY(check_buf(out, "out"));
  if (!q_pos || !win_pos0 || !sink) return fail(CSA_ERR_NULL, "q_pos, win_pos0 and sink are required");
  if (q->dtype != CSA_F32 && q->dtype != CSA_BF16) return fail(CSA_ERR_DTYPE, "q must be F32 or BF16");
  if (out->dtype != q->dtype) return fail(CSA_ERR_DTYPE, "out must have the dtype of q");
  if (kv->dtype == CSA_MXFP4) return fail(CSA_ERR_DTYPE, "attention cache cannot be MXFP4");
  if (win->dtype != kv->dtype) return fail(CSA_ERR_DTYPE, "win must have the dtype of kv");
  if (D < 8 || D > 1024 || D % 8) return fail(CSA_ERR_SHAPE, "D=%d must be a multiple of 8 in [8, 1024]", D);
  if (H < 1 || H > 256) return fail(CSA_ERR_SHAPE, "H=%d out of [1, 256]", H);
  if (B < 0 || Tq < 0 || N < 0 || Tw < 0) return fail(CSA_ERR_SHAPE, "sizes must be non-negative");
  if (kv_rows < N) return fail(CSA_ERR_SHAPE, "kv_rows < N");
  if (n_win < 1) return fail(CSA_ERR_SHAPE, "n_win must be >= 1 (the window holds the query's own token)");
  if (Tw < 1 && B * Tq > 0) return fail(CSA_ERR_SHAPE, "the window buffer is empty");
  CSA_TRY(check_rope(D, rope_dims, rope_base));
  if (kv->dtype == CSA_FP8MIX && (D - rope_dims) % 8) return fail(CSA_ERR_SHAPE, "FP8MIX needs (D - rope_dims) %% 8 == 0");
  if (kv->dtype == CSA_FP8MIX && rope_dims > 0 && (!kv->rope || !win->rope))
    return fail(CSA_ERR_NULL, "FP8MIX caches with rope_dims > 0 need rope pointers");
  return CSA_OK;
}

AttnLaunch make_attn(const csa_buf* q, const int64_t* q_pos, const csa_buf* kv, int64_t kv_rows, int sparse,
                     const int32_t* idx, int32_t K, int32_t ratio, const csa_buf* win, const int64_t* win_pos0,
                     int64_t Tw, const float* sink, float scale, int32_t rope_dims, float rope_base,
                     int64_t pos_offset, int64_t B, int64_t Tq, int32_t H, int32_t D, int64_t N, int32_t n_win,
                     const csa_buf* out) {
  AttnLaunch L{};
  L.q = *q;
  L.q_pos = q_pos;
  L.kv = *kv;
  L.kv_rows = kv_rows;
  L.sparse = sparse;
  L.idx = idx;
  L.K = K;
  L.ratio = ratio;
  L.win = *win;
  L.win_pos0 = win_pos0;
  L.Tw = Tw;
  L.sink = sink;
  L.scale = scale;
  L.rope_dims = rope_dims;
  L.log2_base = rope_dims > 0 ? std::log2(static_cast<double>(rope_base)) : 0.0;
  L.pos_offset = pos_offset;
  L.B = B;
  L.Tq = Tq;
  L.N = N;
  L.H = H;
  L.D = D;
  L.n_win = n_win;
  L.out = *out;
  return L;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

csa_status launched(int rc, const char* what) {
  if (rc == 0) return ok();
  if (rc == -3) return fail(CSA_ERR_WORKSPACE, "%s: workspace too small", what);
  if (rc == -2) return fail(CSA_ERR_UNSUPPORTED, "%s: dtype combination not implemented", what);
  if (rc == -4) return fail(CSA_ERR_SHAPE, "%s: 2^32 or more workgroups", what);
  return fail(CSA_ERR_DEVICE, "%s: kernel launch failed (%s)", what, hipGetErrorString(hipGetLastError()));
}

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_last_error(void) { return g_err.c_str(); }

csa_status csa_device_check(void) {
  csa_status s = check_device();
  return s == CSA_OK ? ok() : s;
}

csa_status csa_compress(const void* ca, const void* cb, const void* za, const void* zb, int32_t in_dtype,
                        const float* bias_a, const float* bias_b, const void* prev_cb, const void* prev_zb,
                        int64_t B, int64_t T, int32_t D, int32_t ratio, int32_t overlap, int64_t t0,
                        int32_t rope_dims, float rope_base, int64_t pos_offset, const csa_buf* out,
                        int64_t out_rows, void* stream) {
  CSA_TRY(validate_compress(ca, cb, za, zb, in_dtype, bias_a, bias_b, prev_cb, prev_zb, B, T, D, ratio, overlap, t0,
                            rope_dims, rope_base, out, out_rows));
  CSA_TRY(check_device());
  CompressLaunch L{};
  L.ca = ca;
  L.cb = overlap ? cb : nullptr;
  L.za = za;
  L.zb = overlap ? zb : nullptr;
  L.bias_a = bias_a;
  L.bias_b = overlap ? bias_b : nullptr;
  L.prev_cb = (overlap && t0 > 0) ? prev_cb : nullptr;
  L.prev_zb = (overlap && t0 > 0) ? prev_zb : nullptr;
  L.stream_dtype = in_dtype;
  L.B = B;
  L.T = T;
  L.t0 = t0;
  L.D = D;
  L.ratio = ratio;
  L.overlap = overlap;
  L.rope_dims = rope_dims;
  L.log2_base = rope_dims > 0 ? std::log2(static_cast<double>(rope_base)) : 0.0;
  L.pos_offset = pos_offset;
  L.out = *out;
  L.out_rows = out_rows;
  return launched(launch_compress(L, static_cast<hipStream_t>(stream)), "csa_compress");
}

csa_status csa_quantize(const float* x, int64_t rows, int32_t D, int32_t rope_dims, const csa_buf* out,
                        void* stream) {
  if (!x) return fail(CSA_ERR_NULL, "x is NULL");
  CSA_TRY(check_buf(out, "out"));
  if (out->dtype != CSA_BF16 && out->dtype != CSA_FP8MIX && out->dtype != CSA_MXFP4)
    return fail(CSA_ERR_DTYPE, "csa_quantize targets BF16, FP8MIX or MXFP4");
  if (rows < 0) return fail(CSA_ERR_SHAPE, "rows must be non-negative");
  if (D < 8 || D > 2048 || D % 8) return fail(CSA_ERR_SHAPE, "D=%d must be a multiple of 8 in [8, 2048]", D);
  if (out->dtype == CSA_FP8MIX) {
    CSA_TRY(check_rope(D, rope_dims, 10000.f));
    if ((D - rope_dims) % 8) return fail(CSA_ERR_SHAPE, "FP8MIX needs (D - rope_dims) %% 8 == 0");
    if (rope_dims > 0 && !out->rope) return fail(CSA_ERR_NULL, "FP8MIX with rope_dims > 0 needs a rope pointer");
  }
  if (out->dtype == CSA_MXFP4 && D % 32) return fail(CSA_ERR_SHAPE, "MXFP4 needs D %% 32 == 0");
  if (!aligned16(x)) return fail(CSA_ERR_SHAPE, "x must be 16-byte aligned");
  CSA_TRY(check_device());
  return launched(launch_quantize(x, rows, D, rope_dims, *out, static_cast<hipStream_t>(stream)), "csa_quantize");
}

csa_status csa_index_scores(const csa_buf* qI, const float* wI, const csa_buf* kI, const int64_t* q_pos, int64_t B,
                            int64_t Tq, int32_t HI, int32_t DI, int64_t N, int64_t kI_rows, int32_t ratio,
                            float* scores, void* stream) {
  CSA_TRY(check_buf(qI, "qI"));
  CSA_TRY(check_buf(kI, "kI"));
  if (!wI || !q_pos || !scores) return fail(CSA_ERR_NULL, "wI, q_pos and scores are required");
  if (qI->dtype != kI->dtype) return fail(CSA_ERR_DTYPE, "qI and kI must share a dtype");
  if (qI->dtype == CSA_FP8MIX) return fail(CSA_ERR_DTYPE, "the indexer takes F32, BF16 or MXFP4");
  if (HI < 1 || HI > 128) return fail(CSA_ERR_SHAPE, "HI=%d out of [1, 128]", HI);
  if (DI < 8 || DI > 512 || DI % 8) return fail(CSA_ERR_SHAPE, "DI=%d must be a multiple of 8 in [8, 512]", DI);
  if (qI->dtype == CSA_MXFP4 && DI % 32) return fail(CSA_ERR_SHAPE, "MXFP4 needs DI %% 32 == 0");
  if (!aligned16(qI->data) || !aligned16(kI->data)) return fail(CSA_ERR_SHAPE, "qI and kI must be 16-byte aligned");
  if (qI->dtype == CSA_MXFP4 && ((reinterpret_cast<uintptr_t>(qI->scale) | reinterpret_cast<uintptr_t>(kI->scale)) & 3))
    return fail(CSA_ERR_SHAPE, "MXFP4 scale planes must be 4-byte aligned");
  if (B < 0 || Tq < 0 || N < 0) return fail(CSA_ERR_SHAPE, "sizes must be non-negative");
  if (kI_rows < N) return fail(CSA_ERR_SHAPE, "kI_rows < N");
  if (ratio < 1) return fail(CSA_ERR_SHAPE, "ratio must be >= 1");
  CSA_TRY(check_device());
  IndexLaunch L{};
  L.qI = *qI;
  L.wI = wI;
  L.kI = *kI;
  L.q_pos = q_pos;
  L.B = B;
  L.Tq = Tq;
  L.N = N;
  L.kI_rows = kI_rows;
  L.HI = HI;
  L.DI = DI;
  L.ratio = ratio;
  L.scores = scores;
  return launched(launch_index_scores(L, static_cast<hipStream_t>(stream)), "csa_index_scores");
}

size_t csa_topk_workspace_size(int64_t rows, int64_t N, int32_t k) { return topk_workspace_bytes(rows, N, k); }

csa_status csa_topk(const float* scores, int64_t rows, int64_t N, int32_t k, int32_t* idx, int32_t* count, void* ws,
                    size_t ws_bytes, void* stream) {
  if (!idx || (!scores && rows > 0 && N > 0)) return fail(CSA_ERR_NULL, "scores and idx are required");
  if (rows < 0 || N < 0 || N >= (static_cast<int64_t>(1) << 31)) return fail(CSA_ERR_SHAPE, "N out of range");
  if (k < 1 || k > 4096) return fail(CSA_ERR_SHAPE, "k=%d out of [1, 4096]", k);
  const size_t need = topk_workspace_bytes(rows, N, k);
  if (need > 0 && (!ws || ws_bytes < need)) return fail(CSA_ERR_WORKSPACE, "csa_topk needs %zu workspace bytes", need);
  CSA_TRY(check_device());
  return launched(launch_topk(scores, rows, N, k, idx, count, ws, static_cast<hipStream_t>(stream)), "csa_topk");
}

size_t csa_sparse_mqa_workspace_size(int64_t B, int64_t Tq, int32_t H, int32_t D, int32_t K, int32_t n_win) {
  return attn_workspace_bytes(B, Tq, H, D, static_cast<int64_t>(K) + n_win, true);
}

csa_status csa_sparse_mqa(const csa_buf* q, const int64_t* q_pos, const csa_buf* kv, int64_t kv_rows,
                          const int32_t* idx, int32_t K, const csa_buf* win, const int64_t* win_pos0, int64_t Tw,
                          const float* sink, float softmax_scale, int32_t rope_dims, float rope_base,
                          int64_t pos_offset, int64_t B, int64_t Tq, int32_t H, int32_t D, int64_t N, int32_t n_win,
                          const csa_buf* out, void* ws, size_t ws_bytes, void* stream) {
  CSA_TRY(validate_attn(q, q_pos, kv, kv_rows, win, win_pos0, Tw, sink, rope_dims, rope_base, B, Tq, H, D, N, n_win,
                        out));
  if (K < 0 || K > (1 << 20)) return fail(CSA_ERR_SHAPE, "K out of range");
  if (K > 0 && !idx) return fail(CSA_ERR_NULL, "idx is required when K > 0");
  AttnLaunch L = make_attn(q, q_pos, kv, kv_rows, 1, idx, K, 1, win, win_pos0, Tw, sink, softmax_scale, rope_dims,
                           rope_base, pos_offset, B, Tq, H, D, N, n_win, out);
  const size_t need = attn_uses_mfma(L) ? attn_workspace_bytes(B, Tq, H, D, static_cast<int64_t>(K) + n_win, true) : 0;
  if (need > ws_bytes || (need > 0 && !ws))
    return fail(CSA_ERR_WORKSPACE, "csa_sparse_mqa needs %zu workspace bytes, got %zu", need, ws_bytes);
  CSA_TRY(check_device());
  return launched(launch_attn(L, ws, ws_bytes, static_cast<hipStream_t>(stream)), "csa_sparse_mqa");
}

size_t hca_dense_attn_workspace_size(int64_t B, int64_t Tq, int32_t H, int32_t D, int64_t N, int32_t n_win) {
  return attn_workspace_bytes(B, Tq, H, D, N + n_win, false);
}

csa_status hca_dense_attn(const csa_buf* q, const int64_t* q_pos, const csa_buf* kv, int64_t kv_rows, int32_t ratio,
                          const csa_buf* win, const int64_t* win_pos0, int64_t Tw, const float* sink,
                          float softmax_scale, int32_t rope_dims, float rope_base, int64_t pos_offset, int64_t B,
                          int64_t Tq, int32_t H, int32_t D, int64_t N, int32_t n_win, const csa_buf* out, void* ws,
                          size_t ws_bytes, void* stream) {
  CSA_TRY(validate_attn(q, q_pos, kv, kv_rows, win, win_pos0, Tw, sink, rope_dims, rope_base, B, Tq, H, D, N, n_win,
                        out));
  if (ratio < 1) return fail(CSA_ERR_SHAPE, "ratio must be >= 1");
  AttnLaunch L = make_attn(q, q_pos, kv, kv_rows, 0, nullptr, 0, ratio, win, win_pos0, Tw, sink, softmax_scale,
                           rope_dims, rope_base, pos_offset, B, Tq, H, D, N, n_win, out);
  const size_t need = attn_uses_mfma(L) ? attn_workspace_bytes(B, Tq, H, D, N + n_win, false) : 0;
  if (need > ws_bytes || (need > 0 && !ws))
    return fail(CSA_ERR_WORKSPACE, "hca_dense_attn needs %zu workspace bytes, got %zu", need, ws_bytes);
  CSA_TRY(check_device());
  return launched(launch_attn(L, ws, ws_bytes, static_cast<hipStream_t>(stream)), "hca_dense_attn");
}

// ------------------------------------------------------------------ csa_forward

namespace {

struct FwdPlan {
  int64_t N;
  size_t scores_off, scores_bytes, idx_off, idx_bytes, topk_off, topk_bytes, attn_off, attn_bytes, total;
};

FwdPlan plan_forward(const csa_layer_desc* L, bool have_scores, bool have_idx) {
  FwdPlan p{};
  p.N = (L->t0 + L->T) / L->ratio;
  size_t off = 0;
  if (L->mode == CSA_MODE_CSA) {
    p.scores_bytes = have_scores ? 0 : align256(static_cast<size_t>(L->B * L->Tq * p.N) * sizeof(float));
    p.scores_off = off;
    off += p.scores_bytes;
    p.idx_bytes = have_idx ? 0 : align256(static_cast<size_t>(L->B * L->Tq * L->topk) * sizeof(int32_t));
    p.idx_off = off;
    off += p.idx_bytes;
    p.topk_bytes = align256(topk_workspace_bytes(L->B * L->Tq, p.N, L->topk));
    p.topk_off = off;
    off += p.topk_bytes;
    p.attn_bytes = align256(attn_workspace_bytes(L->B, L->Tq, L->H, L->D, static_cast<int64_t>(L->topk) + L->n_win, true));
  } else {
    p.attn_bytes = align256(attn_workspace_bytes(L->B, L->Tq, L->H, L->D, p.N + L->n_win, false));
  }
  p.attn_off = off;
  off += p.attn_bytes;
  p.total = off;
  return p;
}

csa_status validate_desc(const csa_layer_desc* L) {
  if (!L) return fail(CSA_ERR_NULL, "layer descriptor is NULL");
  if (L->struct_size != static_cast<int32_t>(sizeof(csa_layer_desc)))
    return fail(CSA_ERR_SHAPE, "csa_layer_desc.struct_size=%d, expected %zu", L->struct_size, sizeof(csa_layer_desc));
  if (L->mode != CSA_MODE_CSA && L->mode != CSA_MODE_HCA) return fail(CSA_ERR_SHAPE, "unknown mode %d", L->mode);
  if (L->ratio < 1 || L->ratio > 1024) return fail(CSA_ERR_SHAPE, "ratio out of [1, 1024]");
  if (L->B < 0 || L->T < 0 || L->t0 < 0 || L->Tq < 0) return fail(CSA_ERR_SHAPE, "sizes must be non-negative");
  if (L->T % L->ratio || L->t0 % L->ratio) return fail(CSA_ERR_SHAPE, "T and t0 must be multiples of ratio");
  if (L->cache_rows < (L->t0 + L->T) / L->ratio) return fail(CSA_ERR_SHAPE, "cache_rows < (t0+T)/ratio");
  if (L->mode == CSA_MODE_CSA && (L->topk < 1 || L->topk > 4096)) return fail(CSA_ERR_SHAPE, "topk out of [1, 4096]");
  return CSA_OK;
}

}  // namespace

size_t csa_forward_workspace_size(const csa_layer_desc* L) {
  if (validate_desc(L) != CSA_OK) return 0;
  return plan_forward(L, false, false).total;
}

csa_status csa_forward(const csa_layer_desc* L, const csa_forward_io* io, void* ws, size_t ws_bytes, void* stream) {
  CSA_TRY(validate_desc(L));
  if (!io) return fail(CSA_ERR_NULL, "io is NULL");
  const bool csa_mode = L->mode == CSA_MODE_CSA;
  const int64_t N = (L->t0 + L->T) / L->ratio;
  // validate every stage before launching any
  if (L->T > 0) {
    CSA_TRY(validate_compress(io->ca, io->cb, io->za, io->zb, L->stream_dtype, io->bias_a, io->bias_b, io->prev_cb,
                              io->prev_zb, L->B, L->T, L->D, L->ratio, csa_mode ? 1 : 0, L->t0, L->rope_dims,
                              L->rope_base, &io->kv_cache, L->cache_rows));
    if (csa_mode)
      CSA_TRY(validate_compress(io->ica, io->icb, io->iza, io->izb, L->stream_dtype, io->ibias_a, io->ibias_b,
                                io->iprev_cb, io->iprev_zb, L->B, L->T, L->DI, L->ratio, 1, L->t0, 0, 1.f,
                                &io->ik_cache, L->cache_rows));
  }
  CSA_TRY(validate_attn(&io->q, io->q_pos, &io->kv_cache, L->cache_rows, &io->win, io->win_pos0, L->Tw, io->sink,
                        L->rope_dims, L->rope_base, L->B, L->Tq, L->H, L->D, N, L->n_win, &io->out));
  if (csa_mode) {
    CSA_TRY(check_buf(&io->qI, "qI"));
    CSA_TRY(check_buf(&io->ik_cache, "ik_cache"));
    if (!io->wI) return fail(CSA_ERR_NULL, "wI is required");
    if (io->qI.dtype != io->ik_cache.dtype) return fail(CSA_ERR_DTYPE, "qI and ik_cache must share a dtype");
    if (L->HI < 1 || L->HI > 128 || L->DI < 8 || L->DI > 512 || L->DI % 8)
      return fail(CSA_ERR_SHAPE, "indexer shape HI=%d DI=%d unsupported", L->HI, L->DI);
    if (io->qI.dtype == CSA_FP8MIX) return fail(CSA_ERR_DTYPE, "the indexer takes F32, BF16 or MXFP4");
    if (io->qI.dtype == CSA_MXFP4 && L->DI % 32) return fail(CSA_ERR_SHAPE, "MXFP4 needs DI %% 32 == 0");
    if (!aligned16(io->qI.data) || !aligned16(io->ik_cache.data))
      return fail(CSA_ERR_SHAPE, "qI and ik_cache must be 16-byte aligned");
    if (io->qI.dtype == CSA_MXFP4 &&
        ((reinterpret_cast<uintptr_t>(io->qI.scale) | reinterpret_cast<uintptr_t>(io->ik_cache.scale)) & 3))
      return fail(CSA_ERR_SHAPE, "MXFP4 scale planes must be 4-byte aligned");
  }
  const FwdPlan P = plan_forward(L, io->scores_out != nullptr, io->idx_out != nullptr);
  if (P.total > 0 && (!ws || ws_bytes < P.total))
    return fail(CSA_ERR_WORKSPACE, "csa_forward needs %zu workspace bytes, got %zu", P.total, ws_bytes);
  CSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  const double log2_base = L->rope_dims > 0 ? std::log2(static_cast<double>(L->rope_base)) : 0.0;

  if (L->T > 0) {
    CompressLaunch C{};
    C.ca = io->ca;
    C.cb = csa_mode ? io->cb : nullptr;
    C.za = io->za;
    C.zb = csa_mode ? io->zb : nullptr;
    C.bias_a = io->bias_a;
    C.bias_b = csa_mode ? io->bias_b : nullptr;
    C.prev_cb = (csa_mode && L->t0 > 0) ? io->prev_cb : nullptr;
    C.prev_zb = (csa_mode && L->t0 > 0) ? io->prev_zb : nullptr;
    C.stream_dtype = L->stream_dtype;
    C.B = L->B;
    C.T = L->T;
    C.t0 = L->t0;
    C.D = L->D;
    C.ratio = L->ratio;
    C.overlap = csa_mode ? 1 : 0;
    C.rope_dims = L->rope_dims;
    C.log2_base = log2_base;
    C.pos_offset = L->pos_offset;
    C.out = io->kv_cache;
    C.out_rows = L->cache_rows;
    if (csa_mode) {
      CompressLaunch I = C;
      I.ca = io->ica;
      I.cb = io->icb;
      I.za = io->iza;
      I.zb = io->izb;
      I.bias_a = io->ibias_a;
      I.bias_b = io->ibias_b;
      I.prev_cb = L->t0 > 0 ? io->iprev_cb : nullptr;
      I.prev_zb = L->t0 > 0 ? io->iprev_zb : nullptr;
      I.D = L->DI;
      I.rope_dims = 0;
      I.out = io->ik_cache;
      if (launch_compress2(C, I, s) != 0) return launched(-1, "csa_forward/compress");
    } else if (launch_compress(C, s) != 0) {
      return launched(-1, "csa_forward/compress");
    }
  }
  if (csa_mode) {
    float* scores = io->scores_out ? io->scores_out : reinterpret_cast<float*>(w + P.scores_off);
    int32_t* idx = io->idx_out ? io->idx_out : reinterpret_cast<int32_t*>(w + P.idx_off);
    IndexLaunch X{};
    X.qI = io->qI;
    X.wI = io->wI;
    X.kI = io->ik_cache;
    X.q_pos = io->q_pos;
    X.B = L->B;
    X.Tq = L->Tq;
    X.N = N;
    X.kI_rows = L->cache_rows;
    X.HI = L->HI;
    X.DI = L->DI;
    X.ratio = L->ratio;
    X.scores = scores;
    int rc = launch_index_scores(X, s);
    if (rc != 0) return launched(rc, "csa_forward/index_scores");
    rc = launch_topk(scores, L->B * L->Tq, N, L->topk, idx, nullptr, w + P.topk_off, s);
    if (rc != 0) return launched(rc, "csa_forward/topk");
    AttnLaunch A = make_attn(&io->q, io->q_pos, &io->kv_cache, L->cache_rows, 1, idx, L->topk, 1, &io->win, io->win_pos0,
                             L->Tw, io->sink, L->softmax_scale, L->rope_dims, L->rope_base, L->pos_offset, L->B, L->Tq,
                             L->H, L->D, N, L->n_win, &io->out);
    return launched(launch_attn(A, w + P.attn_off, P.attn_bytes, s), "csa_forward/sparse_mqa");
  }
  AttnLaunch A = make_attn(&io->q, io->q_pos, &io->kv_cache, L->cache_rows, 0, nullptr, 0, L->ratio, &io->win,
                           io->win_pos0, L->Tw, io->sink, L->softmax_scale, L->rope_dims, L->rope_base, L->pos_offset,
                           L->B, L->Tq, L->H, L->D, N, L->n_win, &io->out);
  return launched(launch_attn(A, w + P.attn_off, P.attn_bytes, s), "csa_forward/hca_dense_attn");
}

}  // extern "C"
