// Host side of libcsa: argument validation, workspace planning and kernel
// launches for every entry point declared in include/csa.h.  Validation is pure
// host arithmetic on the scalar arguments (no device queries apart from one cached
// architecture check per device), so a rejected call costs well under a microsecond
// and launches nothing.
#include <hip/hip_runtime.h>

#include <algorithm>
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

// The query and output formats: F32 or BF16 queries with an output of the same dtype,
// or FP8MIX queries (e4m3 codes of the D - R leading dims, bf16 RoPE dims, a scale per
// head) with an FP8MIX cache, whose QK products then run on fp8 MFMA, and a BF16 output
csa_status check_query(const csa_buf* q, int32_t kv_dtype, const csa_buf* out, int32_t D, int32_t rope_dims,
                       int32_t H) {
  if (q->dtype == CSA_FP8MIX) {
    if (kv_dtype != CSA_FP8MIX) return fail(CSA_ERR_UNSUPPORTED, "FP8MIX queries need an FP8MIX cache");
    if (D != 512 || rope_dims != 64 || (H != 64 && H != 128 && H != 256))
      return fail(CSA_ERR_UNSUPPORTED, "FP8MIX queries need D = 512, rope_dims = 64 and H in {64, 128, 256}");
    if (!q->rope) return fail(CSA_ERR_NULL, "FP8MIX queries need a rope pointer");
    if (reinterpret_cast<uintptr_t>(q->scale) & 3) return fail(CSA_ERR_SHAPE, "the query scales must be 4-byte aligned");
    if (out->dtype != CSA_BF16) return fail(CSA_ERR_DTYPE, "out must be BF16 for FP8MIX queries");
    return CSA_OK;
  }
  if (q->dtype != CSA_F32 && q->dtype != CSA_BF16) return fail(CSA_ERR_DTYPE, "q must be F32, BF16 or FP8MIX");
  if (out->dtype != q->dtype) return fail(CSA_ERR_DTYPE, "out must have the dtype of q");
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
  CSA_TRY(check_query(q, kv->dtype, out, D, rope_dims, H));
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

// Lightning indexer followed by top-k.  Decode-shaped bf16 launches take the selecting
// indexer (each slice's top-k kept while scoring) and one merge level; everything else
// scores the rows into the workspace (or the caller's score buffer) and runs csa_topk.
struct IdxTopkPlan {
  int sel;       // slices per row of the selecting indexer, 0 for the two-call path
  size_t bytes;  // workspace
};

// dtype_known = false (a size query without the operands) sizes for either path
IdxTopkPlan plan_index_topk(IndexLaunch X, int k, bool have_scores, bool dtype_known) {
  X.sel_k = k;
  const size_t rows = static_cast<size_t>(X.B * X.Tq);
  const int sel = index_select_slices(X);
  const size_t cand = sel > 0 ? align256(rows * sel * k * (sizeof(float) + sizeof(int32_t))) : 0;
  const size_t two = (have_scores ? 0 : align256(rows * X.N * sizeof(float))) +
                     align256(topk_workspace_bytes(X.B * X.Tq, X.N, k));
  IdxTopkPlan p{};
  p.sel = dtype_known ? sel : 0;
  p.bytes = !dtype_known ? std::max(cand, two) : (sel > 0 ? cand : two);
  return p;
}

// side: a normalization job riding on the final selection launch, or NULL; out_map:
// the selected entries are written as pool rows of a paged cache
int run_index_topk(IndexLaunch X, int k, const IdxTopkPlan& P, int32_t* idx, int32_t* count, float* scores_out,
                   char* w, hipStream_t s, const char** stage, const AttnNormArgs* side = nullptr,
                   const PageMap* out_map = nullptr) {
  X.sel_k = k;
  const int64_t rows = X.B * X.Tq;
  if (rows == 0 || X.N == 0) {
    // nothing to score: every selection is empty (idx all -1, counts 0)
    *stage = "topk";
    return launch_topk(nullptr, rows, 0, k, idx, count, nullptr, s, side, out_map, X.Tq);
  }
  if (P.sel > 0) {
    const size_t nc = static_cast<size_t>(rows) * P.sel * k;
    X.scores = scores_out;
    X.sel_val = reinterpret_cast<float*>(w);
    X.sel_idx = reinterpret_cast<int32_t*>(w + nc * sizeof(float));
    *stage = "index_select";
    int rc = launch_index_select(X, s);
    if (rc != 0) return rc;
    *stage = "topk_merge";
    return launch_topk_merge(X.sel_val, X.sel_idx, rows, P.sel, k, idx, count, s, side, out_map, X.Tq);
  }
  X.scores = scores_out ? scores_out : reinterpret_cast<float*>(w);
  *stage = "index_scores";
  int rc = launch_index_scores(X, s);
  if (rc != 0) return rc;
  *stage = "topk";
  void* tws = w + (scores_out ? 0 : align256(static_cast<size_t>(rows * X.N) * sizeof(float)));
  return launch_topk(X.scores, rows, X.N, k, idx, count, tws, s, side, out_map, X.Tq);
}

}  // namespace

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_last_error(void) { return g_err.c_str(); }

csa_status csa_device_check(void) {
  csa_status s = check_device();
  return s == CSA_OK ? ok() : s;
}

csa_status csa_compress_norm(const void* ca, const void* cb, const void* za, const void* zb, int32_t in_dtype,
                             const float* bias_a, const float* bias_b, const void* prev_cb, const void* prev_zb,
                             int64_t B, int64_t T, int32_t D, int32_t ratio, int32_t overlap, int64_t t0,
                             int32_t rope_dims, float rope_base, int64_t pos_offset, const float* norm_weight,
                             float norm_eps, const csa_buf* out, int64_t out_rows, void* stream) {
  CSA_TRY(validate_compress(ca, cb, za, zb, in_dtype, bias_a, bias_b, prev_cb, prev_zb, B, T, D, ratio, overlap, t0,
                            rope_dims, rope_base, out, out_rows));
  if (norm_weight && (!aligned16(norm_weight) || !(norm_eps >= 0.f) || !std::isfinite(norm_eps)))
    return fail(CSA_ERR_SHAPE, "norm_weight must be 16-byte aligned and norm_eps finite and >= 0");
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
  L.norm_w = norm_weight;
  L.norm_eps = norm_eps;
  return launched(launch_compress(L, static_cast<hipStream_t>(stream)), "csa_compress");
}

csa_status csa_compress(const void* ca, const void* cb, const void* za, const void* zb, int32_t in_dtype,
                        const float* bias_a, const float* bias_b, const void* prev_cb, const void* prev_zb,
                        int64_t B, int64_t T, int32_t D, int32_t ratio, int32_t overlap, int64_t t0,
                        int32_t rope_dims, float rope_base, int64_t pos_offset, const csa_buf* out,
                        int64_t out_rows, void* stream) {
  return csa_compress_norm(ca, cb, za, zb, in_dtype, bias_a, bias_b, prev_cb, prev_zb, B, T, D, ratio, overlap, t0,
                           rope_dims, rope_base, pos_offset, nullptr, 0.f, out, out_rows, stream);
}

csa_status csa_rmsnorm(const csa_buf* x, int64_t rows, int32_t D, const float* weight, float eps,
                       const csa_buf* out, void* stream) {
  if (!x || !out) return fail(CSA_ERR_NULL, "x and out are required");
  if (!weight) return fail(CSA_ERR_NULL, "weight is required");
  if (x->dtype != out->dtype || (x->dtype != CSA_F32 && x->dtype != CSA_BF16))
    return fail(CSA_ERR_DTYPE, "x and out must share a dtype, F32 or BF16");
  if (rows < 0) return fail(CSA_ERR_SHAPE, "rows < 0");
  if (D < 8 || D > 2048 || D % 8) return fail(CSA_ERR_SHAPE, "D=%d must be a multiple of 8 in [8, 2048]", D);
  if (!(eps >= 0.f) || !std::isfinite(eps)) return fail(CSA_ERR_SHAPE, "eps must be finite and >= 0");
  if (rows == 0) return ok();  // no rows: the buffers may be empty (NULL)
  CSA_TRY(check_buf(x, "x"));
  CSA_TRY(check_buf(out, "out"));
  if (!aligned16(x->data) || !aligned16(out->data)) return fail(CSA_ERR_SHAPE, "x and out must be 16-byte aligned");
  CSA_TRY(check_device());
  return launched(launch_rmsnorm(*x, rows, D, weight, eps, *out, static_cast<hipStream_t>(stream)), "csa_rmsnorm");
}

size_t csa_grouped_out_proj_workspace_size(int64_t T, int32_t n_h, int32_t c, int32_t g, int32_t d_g, int32_t d) {
  if (T < 0 || n_h < 1 || c < 1 || g < 1 || d_g < 1 || d < 1 || n_h % g) return 0;
  return grouped_out_proj_workspace_bytes(T, n_h, c, g, d_g, d);
}

csa_status csa_grouped_out_proj(const csa_buf* o, const void* w_group, const void* w_out, int64_t T, int32_t n_h,
                                int32_t c, int32_t g, int32_t d_g, int32_t d, const csa_buf* out, void* ws,
                                size_t ws_bytes, void* stream) {
  if (!o || !out) return fail(CSA_ERR_NULL, "o and out are required");
  if (!w_group || !w_out) return fail(CSA_ERR_NULL, "w_group and w_out are required");
  if (o->dtype != CSA_BF16) return fail(CSA_ERR_DTYPE, "o must be BF16");
  if (out->dtype != CSA_BF16 && out->dtype != CSA_F32) return fail(CSA_ERR_DTYPE, "out must be BF16 or F32");
  if (T < 0 || n_h < 1 || c < 1 || g < 1 || d_g < 1 || d < 1 || n_h % g || g > 1024)
    return fail(CSA_ERR_SHAPE, "sizes must be positive and g (<= 1024) must divide n_h");
  if ((static_cast<int64_t>(n_h / g) * c) % 32 || (static_cast<int64_t>(g) * d_g) % 32)
    return fail(CSA_ERR_UNSUPPORTED, "(n_h / g) * c and g * d_g must be multiples of 32");
  if (T > (int64_t(1) << 22)) return fail(CSA_ERR_SHAPE, "T=%lld above 2^22", static_cast<long long>(T));
  if (!aligned16(w_group) || !aligned16(w_out)) return fail(CSA_ERR_SHAPE, "the weights must be 16-byte aligned");
  if (T == 0) return ok();  // no rows: o and out may be empty (NULL)
  CSA_TRY(check_buf(o, "o"));
  CSA_TRY(check_buf(out, "out"));
  if (!ws || !aligned16(ws)) return fail(CSA_ERR_WORKSPACE, "workspace required, 16-byte aligned");
  const size_t need = csa_grouped_out_proj_workspace_size(T, n_h, c, g, d_g, d);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "csa_grouped_out_proj needs %zu workspace bytes, got %zu", need, ws_bytes);
  CSA_TRY(check_device());
  GroupedProjLaunch L{};
  L.o = o->data;
  L.w_group = w_group;
  L.w_out = w_out;
  L.mid = ws;
  L.out = out->data;
  L.T = T;
  L.n_h = n_h;
  L.c = c;
  L.g = g;
  L.d_g = d_g;
  L.d = d;
  L.out_f32 = out->dtype == CSA_F32;
  return launched(launch_grouped_out_proj(L, static_cast<hipStream_t>(stream)), "csa_grouped_out_proj");
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

size_t csa_index_topk_workspace_size(int64_t B, int64_t Tq, int32_t HI, int32_t DI, int64_t N, int32_t k,
                                     int32_t qI_dtype, int32_t flags) {
  if (B < 0 || Tq < 0 || N < 0 || HI < 1 || DI < 1 || k < 1) return 0;
  IndexLaunch X{};
  X.qI.dtype = X.kI.dtype = qI_dtype;
  X.B = B;
  X.Tq = Tq;
  X.N = N;
  X.HI = HI;
  X.DI = DI;
  X.score_bf16 = (flags & CSA_FLAG_BF16_SCORES) ? 1 : 0;
  return plan_index_topk(X, k, false, true).bytes;
}

csa_status csa_index_topk(const csa_buf* qI, const float* wI, const csa_buf* kI, const int64_t* q_pos, int64_t B,
                          int64_t Tq, int32_t HI, int32_t DI, int64_t N, int64_t kI_rows, int32_t ratio, int32_t k,
                          int32_t flags, int32_t* idx, int32_t* count, float* scores, void* ws, size_t ws_bytes,
                          void* stream) {
  CSA_TRY(check_buf(qI, "qI"));
  CSA_TRY(check_buf(kI, "kI"));
  if (!wI || !q_pos || !idx) return fail(CSA_ERR_NULL, "wI, q_pos and idx are required");
  if (qI->dtype != kI->dtype) return fail(CSA_ERR_DTYPE, "qI and kI must share a dtype");
  if (qI->dtype == CSA_FP8MIX) return fail(CSA_ERR_DTYPE, "the indexer takes F32, BF16 or MXFP4");
  if (HI < 1 || HI > 128) return fail(CSA_ERR_SHAPE, "HI=%d out of [1, 128]", HI);
  if (DI < 8 || DI > 512 || DI % 8) return fail(CSA_ERR_SHAPE, "DI=%d must be a multiple of 8 in [8, 512]", DI);
  if (qI->dtype == CSA_MXFP4 && DI % 32) return fail(CSA_ERR_SHAPE, "MXFP4 needs DI %% 32 == 0");
  if (!aligned16(qI->data) || !aligned16(kI->data)) return fail(CSA_ERR_SHAPE, "qI and kI must be 16-byte aligned");
  if (qI->dtype == CSA_MXFP4 && ((reinterpret_cast<uintptr_t>(qI->scale) | reinterpret_cast<uintptr_t>(kI->scale)) & 3))
    return fail(CSA_ERR_SHAPE, "MXFP4 scale planes must be 4-byte aligned");
  if (B < 0 || Tq < 0 || N < 0 || N >= (static_cast<int64_t>(1) << 31)) return fail(CSA_ERR_SHAPE, "sizes out of range");
  if (kI_rows < N) return fail(CSA_ERR_SHAPE, "kI_rows < N");
  if (ratio < 1) return fail(CSA_ERR_SHAPE, "ratio must be >= 1");
  if (k < 1 || k > 4096) return fail(CSA_ERR_SHAPE, "k=%d out of [1, 4096]", k);
  if (flags & ~CSA_FLAG_BF16_SCORES) return fail(CSA_ERR_SHAPE, "unknown flags 0x%x", flags);
  IndexLaunch X{};
  X.qI = *qI;
  X.wI = wI;
  X.kI = *kI;
  X.q_pos = q_pos;
  X.B = B;
  X.Tq = Tq;
  X.N = N;
  X.kI_rows = kI_rows;
  X.HI = HI;
  X.DI = DI;
  X.ratio = ratio;
  X.score_bf16 = (flags & CSA_FLAG_BF16_SCORES) ? 1 : 0;
  const IdxTopkPlan P = plan_index_topk(X, k, scores != nullptr, true);
  if (P.bytes > 0 && (!ws || ws_bytes < P.bytes))
    return fail(CSA_ERR_WORKSPACE, "csa_index_topk needs %zu workspace bytes, got %zu", P.bytes, ws_bytes);
  CSA_TRY(check_device());
  const char* stage = "";
  const int rc = run_index_topk(X, k, P, idx, count, scores, static_cast<char*>(ws), static_cast<hipStream_t>(stream),
                                &stage);
  return launched(rc, stage);
}

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

// ------------------------------------------------------------------ allocation-free attention
//
// csa_sparse_mqa_noalloc keeps the split partials in this file-scope device array
// instead of a caller workspace.  Each GPU the library runs on holds its own copy until
// the process ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current, and that
// address is what the kernels receive.  Every call on one GPU shares the array, so calls
// that overlap on one GPU race; nothing in it needs to start at zero (each split writes
// its partial rows and statistics in full before the merge reads them).

}  // extern "C"

namespace {

constexpr size_t kNoAllocScratchBytes = size_t{32} << 20;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];

csa_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return fail(CSA_ERR_DEVICE, "no usable HIP device for the scratch array");
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();
      return fail(CSA_ERR_DEVICE, "hipGetSymbolAddress failed for the scratch array on device %d", dev);
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status csa_sparse_mqa_noalloc(const csa_buf* q, const int64_t* q_pos, const csa_buf* kv, int64_t kv_rows,
                                  const int32_t* idx, int32_t K, const csa_buf* win, const int64_t* win_pos0,
                                  int64_t Tw, const float* sink, float softmax_scale, int32_t rope_dims,
                                  float rope_base, int64_t pos_offset, int64_t B, int64_t Tq, int32_t H, int32_t D,
                                  int64_t N, int32_t n_win, const csa_buf* out, void* stream) {
  CSA_TRY(validate_attn(q, q_pos, kv, kv_rows, win, win_pos0, Tw, sink, rope_dims, rope_base, B, Tq, H, D, N, n_win,
                        out));
  if (K < 0 || K > (1 << 20)) return fail(CSA_ERR_SHAPE, "K out of range");
  if (K > 0 && !idx) return fail(CSA_ERR_NULL, "idx is required when K > 0");
  AttnLaunch L = make_attn(q, q_pos, kv, kv_rows, 1, idx, K, 1, win, win_pos0, Tw, sink, softmax_scale, rope_dims,
                           rope_base, pos_offset, B, Tq, H, D, N, n_win, out);
  const size_t need = attn_uses_mfma(L) ? attn_workspace_bytes(B, Tq, H, D, static_cast<int64_t>(K) + n_win, true) : 0;
  if (need > kNoAllocScratchBytes)
    return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_noalloc: %zu scratch bytes needed, the limit is %zu", need,
                kNoAllocScratchBytes);
  CSA_TRY(check_device());
  void* ws = nullptr;
  CSA_TRY(scratch_address(&ws));
  return launched(launch_attn(L, ws, kNoAllocScratchBytes, static_cast<hipStream_t>(stream)),
                  "csa_sparse_mqa_noalloc");
}

size_t csa_sparse_mqa_noalloc_limit(void) { return kNoAllocScratchBytes; }

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
  IdxTopkPlan it;  // CSA: indexer + top-k
  size_t scores_off, idx_off, idx_bytes, attn_off, attn_bytes;
  size_t nq_off, nq_bytes, nw_off, nw_bytes;  // CSA_FLAG_QKV_NORM: normalized query / window copies
  size_t total;
};

// The indexer launch of a forward (device pointers are filled in by csa_forward)
IndexLaunch index_launch(const csa_layer_desc* L, int32_t qI_dtype) {
  IndexLaunch X{};
  X.qI.dtype = qI_dtype;
  X.kI.dtype = qI_dtype;
  X.B = L->B;
  X.Tq = L->Tq;
  X.N = (L->t0 + L->T) / L->ratio;
  X.kI_rows = L->cache_rows;
  X.HI = L->HI;
  X.DI = L->DI;
  X.ratio = L->ratio;
  X.score_bf16 = (L->flags & CSA_FLAG_BF16_SCORES) ? 1 : 0;
  return X;
}

// qI_dtype: the indexer's operand format (the plan depends on it); -1 for a size query
// without the operands, which covers either plan (and F32 query / window copies)
FwdPlan plan_forward(const csa_layer_desc* L, bool have_scores, bool have_idx, int32_t qI_dtype, int32_t q_dtype = -1,
                     int32_t win_dtype = -1) {
  FwdPlan p{};
  p.N = (L->t0 + L->T) / L->ratio;
  size_t off = 0;
  if (L->mode == CSA_MODE_CSA) {
    p.it = plan_index_topk(index_launch(L, qI_dtype < 0 ? CSA_BF16 : qI_dtype), L->topk, have_scores, qI_dtype >= 0);
    p.scores_off = off;
    off += p.it.bytes;
    p.idx_bytes = have_idx ? 0 : align256(static_cast<size_t>(L->B * L->Tq * L->topk) * sizeof(int32_t));
    p.idx_off = off;
    off += p.idx_bytes;
    p.attn_bytes = align256(attn_workspace_bytes(L->B, L->Tq, L->H, L->D, static_cast<int64_t>(L->topk) + L->n_win, true));
  } else {
    p.attn_bytes = align256(attn_workspace_bytes(L->B, L->Tq, L->H, L->D, p.N + L->n_win, false));
  }
  p.attn_off = off;
  off += p.attn_bytes;
  if (L->flags & CSA_FLAG_QKV_NORM) {
    const size_t qe = q_dtype == CSA_BF16 ? 2 : 4, we = win_dtype == CSA_BF16 ? 2 : 4;
    p.nq_bytes = align256(static_cast<size_t>(L->B * L->Tq * L->H) * L->D * qe);
    p.nq_off = off;
    off += p.nq_bytes;
    p.nw_bytes = align256(static_cast<size_t>(L->B * L->Tw) * L->D * we);
    p.nw_off = off;
    off += p.nw_bytes;
  }
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
  if (L->flags & ~(CSA_FLAG_BF16_SCORES | CSA_FLAG_QKV_NORM)) return fail(CSA_ERR_SHAPE, "unknown flags 0x%x", L->flags);
  if ((L->flags & CSA_FLAG_QKV_NORM) && (!(L->norm_eps >= 0.f) || !std::isfinite(L->norm_eps)))
    return fail(CSA_ERR_SHAPE, "norm_eps must be finite and >= 0");
  if (L->reserved != 0) return fail(CSA_ERR_SHAPE, "csa_layer_desc.reserved must be 0");
  return CSA_OK;
}

}  // namespace

size_t csa_forward_workspace_size(const csa_layer_desc* L) {
  if (validate_desc(L) != CSA_OK) return 0;
  return plan_forward(L, false, false, -1).total;
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
  const bool qkv_norm = (L->flags & CSA_FLAG_QKV_NORM) != 0;
  if (qkv_norm) {
    if (!io->q_norm || !io->kv_norm) return fail(CSA_ERR_NULL, "CSA_FLAG_QKV_NORM needs q_norm and kv_norm");
    if (!aligned16(io->q_norm) || !aligned16(io->kv_norm))
      return fail(CSA_ERR_SHAPE, "q_norm and kv_norm must be 16-byte aligned");
    if ((io->q.dtype != CSA_F32 && io->q.dtype != CSA_BF16) || (io->win.dtype != CSA_F32 && io->win.dtype != CSA_BF16))
      return fail(CSA_ERR_UNSUPPORTED, "CSA_FLAG_QKV_NORM takes F32 or BF16 queries and window rows");
    if (L->D % 8 || L->D > 2048) return fail(CSA_ERR_UNSUPPORTED, "CSA_FLAG_QKV_NORM needs D %% 8 == 0, D <= 2048");
  }
  const FwdPlan P = plan_forward(L, io->scores_out != nullptr, io->idx_out != nullptr,
                                 csa_mode ? io->qI.dtype : CSA_BF16, io->q.dtype, io->win.dtype);
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
    C.norm_w = qkv_norm ? io->kv_norm : nullptr;
    C.norm_eps = L->norm_eps;
    if (csa_mode) {
      CompressLaunch I = C;
      I.norm_w = nullptr;
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
  // the attention operands: the caller's query and window, or their normalized copies
  // (CSA: the normalization rides on the final top-k launch, whose few workgroups leave
  // most of the chip idle; HCA: its own launch)
  csa_buf q = io->q, win = io->win;
  AttnNormArgs norm{};
  if (qkv_norm) {
    q.data = w + P.nq_off;
    win.data = w + P.nw_off;
    norm = make_attn_norm(io->q, q, io->q_norm, io->win, win, io->kv_norm, io->q_pos, io->win_pos0, L->B, L->Tq, L->Tw,
                          L->H, L->D, L->n_win, L->norm_eps);
    if (!csa_mode) {
      const int rc = launch_attn_norm(norm, s);
      if (rc != 0) return launched(rc, "csa_forward/qkv_norm");
    }
  }
  if (csa_mode) {
    int32_t* idx = io->idx_out ? io->idx_out : reinterpret_cast<int32_t*>(w + P.idx_off);
    IndexLaunch X = index_launch(L, io->qI.dtype);
    X.qI = io->qI;
    X.wI = io->wI;
    X.kI = io->ik_cache;
    X.q_pos = io->q_pos;
    const char* stage = "";
    const int rc = run_index_topk(X, L->topk, P.it, idx, nullptr, io->scores_out, w + P.scores_off, s, &stage,
                                  qkv_norm ? &norm : nullptr);
    if (rc != 0) return launched(rc, stage);
    AttnLaunch A = make_attn(&q, io->q_pos, &io->kv_cache, L->cache_rows, 1, idx, L->topk, 1, &win, io->win_pos0,
                             L->Tw, io->sink, L->softmax_scale, L->rope_dims, L->rope_base, L->pos_offset, L->B, L->Tq,
                             L->H, L->D, N, L->n_win, &io->out);
    return launched(launch_attn(A, w + P.attn_off, P.attn_bytes, s), "csa_forward/sparse_mqa");
  }
  AttnLaunch A = make_attn(&q, io->q_pos, &io->kv_cache, L->cache_rows, 0, nullptr, 0, L->ratio, &win,
                           io->win_pos0, L->Tw, io->sink, L->softmax_scale, L->rope_dims, L->rope_base, L->pos_offset,
                           L->B, L->Tq, L->H, L->D, N, L->n_win, &io->out);
  return launched(launch_attn(A, w + P.attn_off, P.attn_bytes, s), "csa_forward/hca_dense_attn");
}


// ------------------------------------------------------------------ csa_decode_step

}  // extern "C"

namespace {

struct DecodePlan {
  int64_t P, N_cap;   // entries per page, indexer row length
  int shift;
  int K;              // attention slots from the cache (CSA: topk; HCA: N_cap)
  IdxTopkPlan it;
  size_t qpos_off, wp0b_off, wp0a_off, idx_off, idx_bytes, it_off, attn_off, attn_bytes;
  size_t nq_off, nq_bytes, nw_off, nw_bytes, total;
};

int log2_exact(int64_t x) {
  if (x < 1 || (x & (x - 1))) return -1;
  int s = 0;
  while ((int64_t{1} << s) < x) ++s;
  return s;
}

csa_status validate_decode_desc(const csa_decode_desc* L) {
  if (!L) return fail(CSA_ERR_NULL, "decode descriptor is NULL");
  if (L->struct_size != static_cast<int32_t>(sizeof(csa_decode_desc)))
    return fail(CSA_ERR_SHAPE, "csa_decode_desc.struct_size=%d, expected %zu", L->struct_size, sizeof(csa_decode_desc));
  if (L->mode != CSA_MODE_CSA && L->mode != CSA_MODE_HCA) return fail(CSA_ERR_SHAPE, "unknown mode %d", L->mode);
  if (L->reserved != 0) return fail(CSA_ERR_SHAPE, "csa_decode_desc.reserved must be 0");
  if (L->B < 0 || L->slots < 1 || L->pages < 1 || L->max_pages < 1 || L->B > L->slots)
    return fail(CSA_ERR_SHAPE, "need 0 <= B <= slots, pages >= 1, max_pages >= 1");
  if (L->ratio < 1 || L->ratio > 1024) return fail(CSA_ERR_SHAPE, "ratio out of [1, 1024]");
  if (L->page_tokens < L->ratio || L->page_tokens % L->ratio || log2_exact(L->page_tokens) < 0)
    return fail(CSA_ERR_SHAPE, "page_tokens=%d must be a power of two and a multiple of ratio", L->page_tokens);
  const int64_t P = L->page_tokens / L->ratio;
  if (log2_exact(P) < 0) return fail(CSA_ERR_SHAPE, "page_tokens / ratio must be a power of two");
  if (static_cast<int64_t>(L->max_pages) * P >= (int64_t{1} << 31) || L->pages * P >= (int64_t{1} << 31))
    return fail(CSA_ERR_SHAPE, "cache pools and rows must stay below 2^31 entries");
  if (L->D < 8 || L->D > 1024 || L->D % 8) return fail(CSA_ERR_SHAPE, "D=%d must be a multiple of 8 in [8, 1024]", L->D);
  if (L->n_win < 1) return fail(CSA_ERR_SHAPE, "n_win must be >= 1");
  if (L->stream_dtype != CSA_F32 && L->stream_dtype != CSA_BF16)
    return fail(CSA_ERR_DTYPE, "stream_dtype must be F32 or BF16");
  if (L->flags & ~(CSA_FLAG_BF16_SCORES | CSA_FLAG_QKV_NORM)) return fail(CSA_ERR_SHAPE, "unknown flags 0x%x", L->flags);
  if ((L->flags & CSA_FLAG_QKV_NORM) && (!(L->norm_eps >= 0.f) || !std::isfinite(L->norm_eps)))
    return fail(CSA_ERR_SHAPE, "norm_eps must be finite and >= 0");
  if (L->mode == CSA_MODE_CSA) {
    if (L->topk < 1 || L->topk > 4096) return fail(CSA_ERR_SHAPE, "topk out of [1, 4096]");
    if (P < index_min_page_entries)
      return fail(CSA_ERR_UNSUPPORTED, "CSA pages need at least %d entries (page_tokens >= %d)", index_min_page_entries,
                  index_min_page_entries * L->ratio);
    if (L->HI < 1 || L->HI > 128 || L->DI < 8 || L->DI > 512 || L->DI % 8)
      return fail(CSA_ERR_SHAPE, "indexer shape HI=%d DI=%d unsupported", L->HI, L->DI);
    if ((L->D / 8 + 63) / 64 * 64 + L->DI / 8 > 256)
      return fail(CSA_ERR_UNSUPPORTED, "D / 8 rounded up to a multiple of 64, plus DI / 8, must be <= 256");
  }
  return CSA_OK;
}

// elem: bytes per element of q and of the window (0: a size query, which takes 4)
DecodePlan plan_decode(const csa_decode_desc* L, bool have_idx, bool have_scores, int32_t qI_dtype, int q_elem,
                       int win_elem) {
  DecodePlan p{};
  p.P = L->page_tokens / L->ratio;
  p.shift = log2_exact(p.P);
  p.N_cap = static_cast<int64_t>(L->max_pages) * p.P;
  const bool csa_mode = L->mode == CSA_MODE_CSA;
  p.K = csa_mode ? L->topk : static_cast<int>(p.N_cap);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align256(bytes);
    return o;
  };
  p.qpos_off = take(static_cast<size_t>(L->B) * 8);
  p.wp0b_off = take(static_cast<size_t>(L->B) * 8);
  p.wp0a_off = take(static_cast<size_t>(L->B) * 8);
  p.idx_bytes = (csa_mode && have_idx) ? 0 : static_cast<size_t>(L->B) * p.K * sizeof(int32_t);
  p.idx_off = take(p.idx_bytes);
  if (csa_mode) {
    IndexLaunch X{};
    X.qI.dtype = qI_dtype < 0 ? CSA_BF16 : qI_dtype;
    X.kI.dtype = X.qI.dtype;
    X.B = L->B;
    X.Tq = 1;
    X.N = p.N_cap;
    X.HI = L->HI;
    X.DI = L->DI;
    X.ratio = L->ratio;
    X.score_bf16 = (L->flags & CSA_FLAG_BF16_SCORES) ? 1 : 0;
    p.it = plan_index_topk(X, L->topk, have_scores, qI_dtype >= 0);
    p.it_off = take(p.it.bytes);
  }
  p.attn_bytes = align256(attn_workspace_bytes(L->B, 1, L->H, L->D, static_cast<int64_t>(p.K) + L->n_win, true));
  p.attn_off = take(p.attn_bytes);
  if (L->flags & CSA_FLAG_QKV_NORM) {
    const size_t qe = q_elem > 0 ? q_elem : 4, we = win_elem > 0 ? win_elem : 4;
    p.nq_bytes = static_cast<size_t>(L->B) * L->H * L->D * qe;
    p.nq_off = take(p.nq_bytes);
    p.nw_bytes = static_cast<size_t>(L->B) * 2 * L->n_win * L->D * we;
    p.nw_off = take(p.nw_bytes);
  }
  p.total = off;
  return p;
}

int elem_bytes(int32_t dtype) { return dtype == CSA_F32 ? 4 : 2; }

}  // namespace

extern "C" {

size_t csa_decode_step_workspace_size(const csa_decode_desc* L) {
  if (validate_decode_desc(L) != CSA_OK) return 0;
  return plan_decode(L, false, false, -1, 0, 0).total;
}

csa_status csa_decode_step(const csa_decode_desc* L, const csa_decode_io* io, void* ws, size_t ws_bytes,
                           void* stream) {
  CSA_TRY(validate_decode_desc(L));
  if (!io) return fail(CSA_ERR_NULL, "io is NULL");
  const bool csa_mode = L->mode == CSA_MODE_CSA;
  const bool qkv_norm = (L->flags & CSA_FLAG_QKV_NORM) != 0;
  const int64_t Ws = 2 * static_cast<int64_t>(L->n_win);
  if (L->B == 0) return ok();
  if (!io->slot || !io->length || !io->ca || !io->za || !io->tail || !io->win_pos0 || !io->block_table)
    return fail(CSA_ERR_NULL, "slot, length, ca, za, tail, win_pos0 and block_table are required");
  if (csa_mode && (!io->cb || !io->zb || !io->ica || !io->icb || !io->iza || !io->izb || !io->itail))
    return fail(CSA_ERR_NULL, "CSA needs cb, zb, the indexer streams and itail");
  CSA_TRY(check_buf(&io->q, "q"));
  CSA_TRY(check_buf(&io->kv_pages, "kv_pages"));
  CSA_TRY(check_buf(&io->win, "win"));
  CSA_TRY(check_buf(&io->out, "out"));
  if (!io->sink) return fail(CSA_ERR_NULL, "sink is required");
  CSA_TRY(check_query(&io->q, io->kv_pages.dtype, &io->out, L->D, L->rope_dims, L->H));
  CSA_TRY(check_buf(&io->kv_raw, "kv_raw"));
  if (io->kv_pages.dtype == CSA_MXFP4) return fail(CSA_ERR_DTYPE, "the attention cache cannot be MXFP4");
  if (io->win.dtype != io->kv_pages.dtype || io->kv_raw.dtype != io->kv_pages.dtype)
    return fail(CSA_ERR_DTYPE, "win and kv_raw must have the dtype of kv_pages");
  if (io->kv_pages.dtype == CSA_FP8MIX) {
    if ((L->D - L->rope_dims) % 16 || L->rope_dims % 8)
      return fail(CSA_ERR_SHAPE, "FP8MIX needs (D - rope_dims) %% 16 == 0 and rope_dims %% 8 == 0");
    if (L->rope_dims > 0 && (!io->kv_pages.rope || !io->win.rope || !io->kv_raw.rope))
      return fail(CSA_ERR_NULL, "FP8MIX caches with rope_dims > 0 need rope pointers");
    if (!io->win.scale || !io->kv_raw.scale) return fail(CSA_ERR_NULL, "FP8MIX windows need scale pointers");
    if (qkv_norm) return fail(CSA_ERR_UNSUPPORTED, "CSA_FLAG_QKV_NORM takes F32 or BF16 windows");
  }
  if (L->H < 1 || L->H > 256) return fail(CSA_ERR_SHAPE, "H=%d out of [1, 256]", L->H);
  CSA_TRY(check_rope(L->D, L->rope_dims, L->rope_base));
  if (csa_mode) {
    CSA_TRY(check_buf(&io->qI, "qI"));
    CSA_TRY(check_buf(&io->ik_pages, "ik_pages"));
    if (!io->wI) return fail(CSA_ERR_NULL, "wI is required");
    if (io->qI.dtype != io->ik_pages.dtype) return fail(CSA_ERR_DTYPE, "qI and ik_pages must share a dtype");
    if (io->qI.dtype == CSA_FP8MIX) return fail(CSA_ERR_DTYPE, "the indexer takes F32, BF16 or MXFP4");
    if (io->qI.dtype == CSA_MXFP4 && L->DI % 32) return fail(CSA_ERR_SHAPE, "MXFP4 needs DI %% 32 == 0");
  }
  if (qkv_norm) {
    if (!io->q_norm || !io->kv_norm) return fail(CSA_ERR_NULL, "CSA_FLAG_QKV_NORM needs q_norm and kv_norm");
    if (!aligned16(io->q_norm) || !aligned16(io->kv_norm))
      return fail(CSA_ERR_SHAPE, "q_norm and kv_norm must be 16-byte aligned");
  }
  const DecodePlan P = plan_decode(L, io->idx_out != nullptr, io->scores_out != nullptr,
                                   csa_mode ? io->qI.dtype : -1, elem_bytes(io->q.dtype), elem_bytes(io->win.dtype));
  if (!ws || ws_bytes < P.total || !aligned16(ws))
    return fail(CSA_ERR_WORKSPACE, "csa_decode_step needs %zu workspace bytes (16-byte aligned), got %zu", P.total,
                ws_bytes);
  CSA_TRY(check_device());
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  int64_t* q_pos = reinterpret_cast<int64_t*>(w + P.qpos_off);
  int64_t* wp0_b = reinterpret_cast<int64_t*>(w + P.wp0b_off);
  int64_t* wp0_adj = reinterpret_cast<int64_t*>(w + P.wp0a_off);
  int32_t* idx = (csa_mode && io->idx_out) ? io->idx_out : reinterpret_cast<int32_t*>(w + P.idx_off);
  PageMap pm{io->block_table, io->slot, L->max_pages, P.shift};

  StateAppendLaunch A{};
  A.B = L->B;
  A.ca = io->ca; A.cb = io->cb; A.za = io->za; A.zb = io->zb;
  A.bias_a = io->bias_a; A.bias_b = csa_mode ? io->bias_b : nullptr;
  if (csa_mode) {
    A.ica = io->ica; A.icb = io->icb; A.iza = io->iza; A.izb = io->izb;
    A.ibias_a = io->ibias_a; A.ibias_b = io->ibias_b;
  }
  A.stream_dtype = L->stream_dtype;
  A.D = L->D;
  A.DI = L->DI;
  A.ratio = L->ratio;
  A.overlap = csa_mode ? 1 : 0;
  A.rope_dims = L->rope_dims;
  A.log2_base = L->rope_dims > 0 ? std::log2(static_cast<double>(L->rope_base)) : 0.0;
  A.pos_offset = L->pos_offset;
  A.norm_w = qkv_norm ? io->kv_norm : nullptr;
  A.norm_eps = L->norm_eps;
  A.kv_out = io->kv_pages;
  A.ik_out = io->ik_pages;
  A.pmap = pm;
  A.slot = io->slot;
  A.length = io->length;
  A.tail = io->tail;
  A.itail = io->itail;
  A.kv_raw = io->kv_raw;
  A.win = io->win;
  A.n_win = L->n_win;
  A.Ws = Ws;
  A.win_pos0 = io->win_pos0;
  A.q_pos = q_pos;
  A.wp0_b = wp0_b;
  A.wp0_adj = wp0_adj;
  A.vis_idx = csa_mode ? nullptr : idx;
  A.vis_K = P.K;
  int rc = launch_state_append(A, s);
  if (rc != 0) return launched(rc, "csa_decode_step/append");

  // the attention's query and window: the caller's and the slots' own, or normalized
  // copies (batch row b's window copy at rows b * Ws .., base wp0_b[b])
  csa_buf q = io->q, win = io->win;
  const int64_t* win_base = wp0_adj;
  AttnNormArgs norm{};
  if (qkv_norm) {
    q.data = w + P.nq_off;
    win.data = w + P.nw_off;
    norm = make_attn_norm(io->q, q, io->q_norm, io->win, win, io->kv_norm, q_pos, wp0_b, L->B, 1, Ws, L->H, L->D,
                          L->n_win, L->norm_eps);
    norm.win_slot = io->slot;
    win_base = wp0_b;
    if (!csa_mode) {
      rc = launch_attn_norm(norm, s);
      if (rc != 0) return launched(rc, "csa_decode_step/qkv_norm");
    }
  }
  if (csa_mode) {
    IndexLaunch X{};
    X.qI = io->qI;
    X.wI = io->wI;
    X.kI = io->ik_pages;
    X.q_pos = q_pos;
    X.B = L->B;
    X.Tq = 1;
    X.N = P.N_cap;
    X.kI_rows = 0;
    X.HI = L->HI;
    X.DI = L->DI;
    X.ratio = L->ratio;
    X.score_bf16 = (L->flags & CSA_FLAG_BF16_SCORES) ? 1 : 0;
    X.kmap = pm;
    const char* stage = "";
    rc = run_index_topk(X, L->topk, P.it, idx, nullptr, io->scores_out, w + P.it_off, s, &stage,
                        qkv_norm ? &norm : nullptr, &pm);
    if (rc != 0) return launched(rc, stage);
  }
  // the cache operand is addressed by pool rows: one row block for every sequence
  AttnLaunch AL = make_attn(&q, q_pos, &io->kv_pages, 0, 1, idx, P.K, 1, &win, win_base, Ws, io->sink,
                            L->softmax_scale, L->rope_dims, L->rope_base, L->pos_offset, L->B, 1, L->H, L->D, P.N_cap,
                            L->n_win, &io->out);
  return launched(launch_attn(AL, w + P.attn_off, P.attn_bytes, s), "csa_decode_step/attention");
}

}  // extern "C"
