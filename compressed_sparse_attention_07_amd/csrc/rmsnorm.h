// Row-wise RMSNorm on the device ([V4-CN] "DeepSeek-V4中文翻译" §2.3.3: the query heads
// and the KV entries are RMS-normalized before core attention):
//     y[d] = x[d] / sqrt(mean_j x[j]^2 + eps) * w[d]          (fp32 arithmetic)
// One wave per row; lane l owns dims 8 (l + 64 i), and the sum of squares is reduced
// across the wave in a fixed order (DPP), so results are bitwise repeatable.
//
// The attention operands of a forward are normalized by one job (attn_norm_block):
// every query head row, and for each sequence only the window rows its queries can see
// (positions max(0, min q_pos - n_win + 1) .. max q_pos, clipped to the buffer), each
// written to the same row of a copy (the source window of a batch row may be another
// row block of the buffer: a state-pool slot).  The job runs as its own launch or as extra
// workgroups appended to another launch (any whole number of waves per workgroup).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"
#include "device_common.h"

namespace csa {

struct NormArgs {
  const void* x;
  void* y;
  const float* w;
  int64_t rows;
  int D, dtype;  // D % 8 == 0, D <= 2048; dtype CSA_F32 or CSA_BF16
  float eps;
};

__device__ __forceinline__ void norm_load8(const void* x, int dtype, int64_t off, float v[8]) {
  if (dtype == CSA_F32) {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(x) + off + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
    v[0] = bf16lo(a.x); v[1] = bf16hi(a.x); v[2] = bf16lo(a.y); v[3] = bf16hi(a.y);
    v[4] = bf16lo(a.z); v[5] = bf16hi(a.z); v[6] = bf16lo(a.w); v[7] = bf16hi(a.w);
  }
}

// one row (called by a whole wave): the sum of squares, then a second pass over the
// row (now in cache) that scales and stores, so few registers stay live
__device__ __forceinline__ void norm_row(const void* x, int64_t xrow, void* y, int64_t row, const float* w, int D,
                                         int dtype, float eps, int lane) {
  float ss = 0.f;
  for (int d0 = 8 * lane; d0 < D; d0 += 8 * WAVE) {
    float v[8];
    norm_load8(x, dtype, xrow * D + d0, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
  }
  const float inv = 1.0f / sqrtf(wave_sum_dpp(ss) / static_cast<float>(D) + eps);
  for (int d0 = 8 * lane; d0 < D; d0 += 8 * WAVE) {
    float v[8];
    norm_load8(x, dtype, xrow * D + d0, v);
    const float4 w0 = *reinterpret_cast<const float4*>(w + d0);
    const float4 w1 = *reinterpret_cast<const float4*>(w + d0 + 4);
    const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = v[i] * inv * wv[i];
    if (dtype == CSA_F32) {
      float4* p = reinterpret_cast<float4*>(static_cast<float*>(y) + row * D + d0);
      p[0] = make_float4(o[0], o[1], o[2], o[3]);
      p[1] = make_float4(o[4], o[5], o[6], o[7]);
    } else {
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(y) + row * D + d0) =
          make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                     pack_bf16x2(o[6], o[7]));
    }
  }
}

struct AttnNormArgs {
  NormArgs q;            // query head rows [B * Tq * H, D]
  const void* win;       // window rows [B, Tw, D]
  void* win_out;
  const float* kv_w;
  const int64_t* q_pos;  // [B, Tq]
  const int64_t* win_pos0;  // [B] position of row 0 of each batch row's window
  const int32_t* win_slot;  // [B] or NULL: batch row b's source window is row block win_slot[b] of win
  int64_t B, Tq, Tw;
  int win_dtype, n_win;
  uint32_t q_blocks;     // workgroups of the query part (NW rows each)
  uint32_t w_blocks;     // workgroups per sequence of the window part
  uint32_t blocks;       // q_blocks + B * w_blocks (0: no job)
};

// the job's workgroup count for NW waves per workgroup
inline void attn_norm_shape(AttnNormArgs& a, int NW) {
  const int64_t B = a.B;
  const int64_t rows = a.q.rows;
  a.q_blocks = static_cast<uint32_t>((rows + NW - 1) / NW);
  // enough waves for the rows a contiguous run of queries sees, a few rows per wave
  const int64_t seen = a.Tq + a.n_win - 1;
  int64_t wb = (seen + 2 * NW - 1) / (2 * NW);
  wb = wb < 1 ? 1 : (wb > 1024 ? 1024 : wb);
  a.w_blocks = static_cast<uint32_t>(wb);
  a.blocks = rows == 0 ? 0u : a.q_blocks + ((a.Tw > 0 && a.n_win > 0) ? static_cast<uint32_t>(B) * a.w_blocks : 0u);
}

// workgroup `blk` (< a.blocks) of the job, NW waves
template <int NW>
__device__ __forceinline__ void attn_norm_block(const AttnNormArgs& a, uint32_t blk) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (blk < a.q_blocks) {
    const int64_t row = static_cast<int64_t>(blk) * NW + wid;
    if (row < a.q.rows) norm_row(a.q.x, row, a.q.y, row, a.q.w, a.q.D, a.q.dtype, a.q.eps, lane);
    return;
  }
  const uint32_t wb = blk - a.q_blocks;
  const int64_t b = wb / a.w_blocks;
  const uint32_t part = wb % a.w_blocks;
  __shared__ int64_t s_lo[NW], s_hi[NW];
  int64_t lo = INT64_MAX, hi = INT64_MIN;
  for (int64_t t = threadIdx.x; t < a.Tq; t += NW * WAVE) {
    const int64_t p = a.q_pos[b * a.Tq + t];
    lo = p < lo ? p : lo;
    hi = p > hi ? p : hi;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int64_t l2 = static_cast<int64_t>(__shfl_xor(static_cast<long long>(lo), o));
    const int64_t h2 = static_cast<int64_t>(__shfl_xor(static_cast<long long>(hi), o));
    lo = l2 < lo ? l2 : lo;
    hi = h2 > hi ? h2 : hi;
  }
  if (lane == 0) {
    s_lo[wid] = lo;
    s_hi[wid] = hi;
  }
  __syncthreads();
  lo = s_lo[0];
  hi = s_hi[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    lo = s_lo[i] < lo ? s_lo[i] : lo;
    hi = s_hi[i] > hi ? s_hi[i] : hi;
  }
  if (lo > hi) return;
  const int64_t wp0 = a.win_pos0[b];
  int64_t first = lo - a.n_win + 1;
  first = first < 0 ? 0 : first;
  first = first < wp0 ? wp0 : first;
  const int64_t last = hi < wp0 + a.Tw - 1 ? hi : wp0 + a.Tw - 1;
  const int64_t src_b = a.win_slot ? static_cast<int64_t>(a.win_slot[b]) : b;
  for (int64_t p = first + static_cast<int64_t>(part) * NW + wid; p <= last; p += static_cast<int64_t>(a.w_blocks) * NW)
    norm_row(a.win, src_b * a.Tw + (p - wp0), a.win_out, b * a.Tw + (p - wp0), a.kv_w, a.q.D, a.win_dtype, a.q.eps,
             lane);
}

}  // namespace csa
