// Internal (non-ABI) launch interface between the host API (api.hip) and the
// kernel translation units.  All arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa.h"
#include "rmsnorm.h"

namespace csa {

struct CompressLaunch {
  const void *ca, *cb, *za, *zb;
  const float *bias_a, *bias_b;
  const void *prev_cb, *prev_zb;
  int stream_dtype;
  int64_t B, T, t0;
  int D, ratio, overlap, rope_dims;
  double log2_base;
  int64_t pos_offset;
  csa_buf out;
  int64_t out_rows;
  const float* norm_w;  // RMSNorm weight [D] applied to each entry before RoPE, or NULL
  float norm_eps;
};
int launch_compress(const CompressLaunch& L, hipStream_t stream);
// two compressions sharing the stream dtype (KV and indexer keys) in one launch
int launch_compress2(const CompressLaunch& L0, const CompressLaunch& L1, hipStream_t stream);
int launch_quantize(const float* x, int64_t rows, int D, int rope_dims, const csa_buf& out,
                    hipStream_t stream);

// One decode token per sequence into its state-pool slot (compress.hip)
struct StateAppendLaunch {
  int64_t B;
  const void *ca, *cb, *za, *zb;      // [B, D] (no overlap: ca = C, za = Z)
  const float *bias_a, *bias_b;
  const void *ica, *icb, *iza, *izb;  // [B, DI] (overlap), or ica = NULL
  const float *ibias_a, *ibias_b;
  int stream_dtype;
  int D, DI, ratio, overlap, rope_dims;
  double log2_base;
  int64_t pos_offset;
  const float* norm_w;
  float norm_eps;
  csa_buf kv_out, ik_out;             // page pools
  PageMap pmap;
  const int32_t* slot;
  int64_t* length;
  void *tail, *itail;
  csa_buf kv_raw;                     // [B, D] in the window's format
  csa_buf win;                        // [slots, Ws, D] (F32, BF16 or FP8MIX planes)
  int n_win;
  int64_t Ws;
  int64_t* win_pos0;
  int64_t *q_pos, *wp0_b, *wp0_adj;   // [B] outputs
  int32_t* vis_idx;                   // [B, vis_K] (no overlap) or NULL
  int64_t vis_K;
};
int launch_state_append(const StateAppendLaunch& L, hipStream_t stream);

struct IndexLaunch {
  csa_buf qI;
  const float* wI;
  csa_buf kI;
  const int64_t* q_pos;
  int64_t B, Tq, N, kI_rows;
  int HI, DI, ratio;
  float* scores;         // [B, Tq, N] or NULL (selecting launch without a score copy)
  int score_bf16;        // round every score to bf16 before it is stored or selected
  // selecting launch (launch_index_select): each slice's top-k candidates
  int sel_k;
  float* sel_val;        // [B * Tq, slices, sel_k]
  int32_t* sel_idx;
  // paged keys (kmap.table != NULL; then kI_rows is unused): the MFMA kernels look a
  // page up once per key range, so a range must not cross a page (ranges are capped at
  // 2^kmap.shift entries, which must be at least index_min_page_entries)
  PageMap kmap;
};
int launch_index_scores(const IndexLaunch& L, hipStream_t stream);
constexpr int index_min_page_entries = 512;  // smallest page the indexer kernels take
// Decode-shaped bf16 lightning indexer that selects while it scores: every workgroup
// keeps its slice's top-k candidates (the score row is never stored unless L.scores is
// set); the candidates then go through topk_merge.  Returns 1 (nothing launched) when
// the shape is not covered.
int index_select_slices(const IndexLaunch& L);  // slices per row, 0 if not covered
int launch_index_select(const IndexLaunch& L, hipStream_t stream);
// side: a normalization job appended to the final selection launch, or NULL.
// out_map (table != NULL): the final indices are written as pool rows of a paged cache
// (row r of the selection belongs to batch row r / tq); -1 padding stays -1.
int launch_topk_merge(const float* cand_val, const int32_t* cand_idx, int64_t rows, int slices, int k,
                      int32_t* idx, int32_t* count, hipStream_t stream, const AttnNormArgs* side = nullptr,
                      const PageMap* out_map = nullptr, int64_t tq = 1);

size_t topk_workspace_bytes(int64_t rows, int64_t N, int k);
int launch_topk(const float* scores, int64_t rows, int64_t N, int k, int32_t* idx, int32_t* count,
                void* ws, hipStream_t stream, const AttnNormArgs* side = nullptr, const PageMap* out_map = nullptr,
                int64_t tq = 1);

struct GroupedProjLaunch {
  const void* o;        // bf16 [T, n_h, c]
  const void* w_group;  // bf16 [g, d_g, (n_h / g) c]
  const void* w_out;    // bf16 [d, g d_g]
  void* mid;            // workspace: bf16 [T, g d_g], then fp32 split partials
  void* out;            // [T, d], bf16 or f32
  int64_t T, n_h, c, g, d_g, d;
  int out_f32;
};
size_t grouped_out_proj_workspace_bytes(int64_t T, int64_t n_h, int64_t c, int64_t g, int64_t d_g, int64_t d);
int launch_grouped_out_proj(const GroupedProjLaunch& L, hipStream_t stream);

// Row-wise RMSNorm: y = x / sqrt(mean(x^2) + eps) * w, rows of D in F32 or BF16
int launch_rmsnorm(const csa_buf& x, int64_t rows, int D, const float* w, float eps, const csa_buf& y,
                   hipStream_t stream);
// The normalization job of a forward's attention operands (rmsnorm.h): query heads
// [B*Tq*H, D] into q_out and, per sequence, the window rows its queries see into the
// same rows of win_out ([B, Tw, D]); other rows of win_out are not written.  It runs as
// its own launch, or rides as extra workgroups on the last top-k launch.
AttnNormArgs make_attn_norm(const csa_buf& q, const csa_buf& q_out, const float* q_w, const csa_buf& win,
                            const csa_buf& win_out, const float* kv_w, const int64_t* q_pos, const int64_t* win_pos0,
                            int64_t B, int64_t Tq, int64_t Tw, int H, int D, int n_win, float eps);
int launch_attn_norm(AttnNormArgs a, hipStream_t stream);

struct AttnLaunch {
  csa_buf q;
  const int64_t* q_pos;
  csa_buf kv;
  int64_t kv_rows;
  int sparse;          // 1: keys come from idx; 0: every visible entry (dense)
  const int32_t* idx;  // sparse: [B, Tq, K] (may be NULL when K == 0)
  int K;               // sparse slots per query
  int ratio;           // dense visibility ratio
  csa_buf win;
  const int64_t* win_pos0;
  int64_t Tw;
  const float* sink;
  float scale;
  int rope_dims;
  double log2_base;
  int64_t pos_offset;
  int64_t B, Tq, N;
  int H, D, n_win;
  csa_buf out;
};
size_t attn_workspace_bytes(int64_t B, int64_t Tq, int H, int D, int64_t max_keys, bool sparse);
bool attn_uses_mfma(const AttnLaunch& L);
int launch_attn(const AttnLaunch& L, void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace csa
