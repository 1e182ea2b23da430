// Internal (non-ABI) launch interface between the host API (api.hip) and the
// kernel translation units.  All arguments are validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/csa.h"

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
};
int launch_compress(const CompressLaunch& L, hipStream_t stream);
// two compressions sharing the stream dtype (KV and indexer keys) in one launch
int launch_compress2(const CompressLaunch& L0, const CompressLaunch& L1, hipStream_t stream);
int launch_quantize(const float* x, int64_t rows, int D, int rope_dims, const csa_buf& out,
                    hipStream_t stream);

struct IndexLaunch {
  csa_buf qI;
  const float* wI;
  csa_buf kI;
  const int64_t* q_pos;
  int64_t B, Tq, N, kI_rows;
  int HI, DI, ratio;
  float* scores;
};
int launch_index_scores(const IndexLaunch& L, hipStream_t stream);

size_t topk_workspace_bytes(int64_t rows, int64_t N, int k);
int launch_topk(const float* scores, int64_t rows, int64_t N, int k, int32_t* idx, int32_t* count,
                void* ws, hipStream_t stream);

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
