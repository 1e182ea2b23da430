// K2: lightning-indexer scores
//     I[t, s] = sum_h w[t, h] * ReLU(q[t, h, :] . K[s, :])   for s < floor(pos_t / m),
// -inf for the other entries.  [V4-CN] "DeepSeek-V4中文翻译" §2.3.1 (index-score
// equation), §2.3.3 (a query only sees earlier compressed blocks).
//
// bf16 path: one wave owns one query token and a contiguous range of entries.  The
// token's indexer queries [HI, DI] stay in registers as the MFMA A operand (heads =
// rows); each 16-entry tile of keys is loaded straight from HBM into the B operand
// (16 lanes x 64 contiguous bytes per load), multiplied with
// v_mfma_f32_16x16x32_bf16, and reduced in the epilogue: every lane applies ReLU
// and the head weights to the 4 heads x 1 entry it holds per head block, two
// cross-lane adds finish the sum over heads, and each lane stores one score of a
// 64-entry run (one coalesced 256-byte store per iteration).
//
// The SIMT kernel (fp32, or shapes the MFMA tiling does not cover) computes one
// score per thread with the token's queries staged in LDS.
#include "device_common.h"
#include "launch.h"

namespace csa {

namespace {

// ------------------------------------------------------------------ SIMT path

constexpr int kSimtThreads = 256;
constexpr int kSimtQ = 8192;  // floats of queries staged in LDS per pass

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

template <typename T>
__global__ __launch_bounds__(kSimtThreads) void index_simt_kernel(IndexLaunch a) {
  __shared__ float qs[kSimtQ];
  __shared__ float ws[128];
  const int64_t bt = blockIdx.y;            // b * Tq + t
  const int64_t b = bt / a.Tq;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kSimtThreads + threadIdx.x;
  const int64_t pos = a.q_pos[bt];
  int64_t vis = pos / a.ratio;
  if (vis > a.N) vis = a.N;
  if (vis < 0) vis = 0;
  const T* q = static_cast<const T*>(a.qI.data) + bt * a.HI * a.DI;
  const T* k = static_cast<const T*>(a.kI.data) + (b * a.kI_rows + (s < vis ? s : 0)) * a.DI;
  for (int h = threadIdx.x; h < a.HI; h += kSimtThreads) ws[h] = a.wI[bt * a.HI + h];
  const int hc = kSimtQ / a.DI;             // heads per LDS pass
  float score = 0.f;
  for (int h0 = 0; h0 < a.HI; h0 += hc) {
    const int nh = min(hc, a.HI - h0);
    __syncthreads();
    for (int i = threadIdx.x; i < nh * a.DI; i += kSimtThreads) qs[i] = ld<T>(q, h0 * a.DI + i);
    __syncthreads();
    if (s < vis) {
      for (int h = 0; h < nh; ++h) {
        float dot = 0.f;
        for (int d = 0; d < a.DI; ++d) dot = fmaf(qs[h * a.DI + d], ld<T>(k, d), dot);
        score = fmaf(ws[h0 + h], fmaxf(dot, 0.f), score);
      }
    }
  }
  if (s < a.N) a.scores[bt * a.N + s] = s < vis ? score : -INFINITY;
}

// ------------------------------------------------------------------ MFMA path

constexpr int kWavesPerWG = 4;
constexpr int kTiles = 4;  // 16-entry tiles per iteration (64 entries)

template <int HB, int KS>
__global__ __launch_bounds__(kWavesPerWG * WAVE) void index_mfma_kernel(IndexLaunch a, int keys_per_wave,
                                                                        int64_t waves_per_token) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWavesPerWG + (threadIdx.x >> 6);
  const int64_t total = a.B * a.Tq * waves_per_token;
  if (wave >= total) return;
  const int64_t bt = wave / waves_per_token;
  const int64_t b = bt / a.Tq;
  const int64_t s_begin = (wave % waves_per_token) * keys_per_wave;
  const int64_t s_end = min(s_begin + keys_per_wave, a.N);
  const int64_t pos = a.q_pos[bt];
  int64_t vis = pos / a.ratio;
  vis = vis > a.N ? a.N : (vis < 0 ? 0 : vis);

  const int col = lane & 15;   // entry within a tile / head row within a head block
  const int grp = lane >> 4;   // k-group of the operands, row group of the result

  float* out = a.scores + bt * a.N;
  const int64_t vis_end = min(s_end, vis);

  // queries: A operand, rows = heads, k = DI (8 bf16 per lane per k-step)
  bf16x8 qa[HB][KS];
  float w[HB][4];
  if (s_begin < vis_end) {
    const uint16_t* q = static_cast<const uint16_t*>(a.qI.data) + bt * a.HI * a.DI;
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qa[hb][ks] = *reinterpret_cast<const bf16x8*>(q + (hb * 16 + col) * a.DI + ks * 32 + grp * 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) w[hb][r] = a.wI[bt * a.HI + hb * 16 + grp * 4 + r];
    }
  }

  const uint16_t* kbase = static_cast<const uint16_t*>(a.kI.data) + b * a.kI_rows * a.DI;
  // keys of 64 entries starting at s0 (B operand: entry = col, k = 32ks + 8grp .. +8)
  auto load = [&](bf16x8 (&kb)[kTiles][KS], int64_t s0) {
#pragma unroll
    for (int tI = 0; tI < kTiles; ++tI) {
      int64_t s = s0 + tI * 16 + col;
      if (s >= vis_end) s = vis_end - 1;   // clamp: in bounds, masked below
      const uint16_t* kp = kbase + s * a.DI + grp * 8;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kb[tI][ks] = *reinterpret_cast<const bf16x8*>(kp + ks * 32);
    }
  };
  // scores of the 64 entries at s0: lane (grp, col) stores entry s0 + 16*grp + col
  auto score = [&](const bf16x8 (&kb)[kTiles][KS], int64_t s0) {
    float res = -INFINITY;
    if (s0 < vis_end) {
      float part[kTiles];
#pragma unroll
      for (int tI = 0; tI < kTiles; ++tI) {
        float sc = 0.f;
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[hb][ks], kb[tI][ks], acc, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) sc = fmaf(w[hb][r], fmaxf(acc[r], 0.f), sc);
        }
        // sum the four row groups (heads) holding the same entry
        sc += __shfl_xor(sc, 16, WAVE);
        sc += __shfl_xor(sc, 32, WAVE);
        part[tI] = sc;
      }
#pragma unroll
      for (int tI = 0; tI < kTiles; ++tI)
        if (grp == tI) res = part[tI];
      if (s0 + lane >= vis_end) res = -INFINITY;
    }
    const int64_t s = s0 + lane;
    if (s < s_end) out[s] = res;
  };

  // two register buffers: the next 64 entries are in flight while the current ones
  // go through the MFMAs and the epilogue
  constexpr int64_t kStep = 16 * kTiles;
  bf16x8 kA[kTiles][KS], kB[kTiles][KS];
  int64_t s0 = s_begin;
  if (s0 < vis_end) load(kA, s0);
  for (; s0 < s_end; s0 += 2 * kStep) {
    if (s0 + kStep < vis_end) load(kB, s0 + kStep);
    score(kA, s0);
    if (s0 + kStep >= s_end) break;
    if (s0 + 2 * kStep < vis_end) load(kA, s0 + 2 * kStep);
    score(kB, s0 + kStep);
  }
}

typedef void (*MfmaKern)(IndexLaunch, int, int64_t);

template <int HB>
MfmaKern pick_ks(int KS) {
  switch (KS) {
    case 1: return index_mfma_kernel<HB, 1>;
    case 2: return index_mfma_kernel<HB, 2>;
    case 4: return index_mfma_kernel<HB, 4>;
    case 8:
      if constexpr (HB * 8 <= 32) return index_mfma_kernel<HB, 8>;  // larger tiles would spill
      return nullptr;
  }
  return nullptr;
}

MfmaKern pick_mfma(int HB, int KS) {
  switch (HB) {
    case 1: return pick_ks<1>(KS);
    case 2: return pick_ks<2>(KS);
    case 4: return pick_ks<4>(KS);
    case 8: return pick_ks<8>(KS);
  }
  return nullptr;
}

}  // namespace

int launch_index_scores(const IndexLaunch& L, hipStream_t stream) {
  if (L.B == 0 || L.Tq == 0 || L.N == 0) return 0;
  if (L.qI.dtype == CSA_BF16 && L.HI % 16 == 0 && L.DI % 32 == 0) {
    MfmaKern k = pick_mfma(L.HI / 16, L.DI / 32);
    if (k) {
      // entries per wave: small ranges when there are few tokens (decode) so that the
      // whole chip streams the keys; longer ranges amortise the query load otherwise
      const int64_t tokens = L.B * L.Tq;
      int kpw = 256;
      while (kpw < 4096 && tokens * ((L.N + kpw - 1) / kpw) > 8192) kpw *= 2;
      const int64_t wpt = (L.N + kpw - 1) / kpw;
      const int64_t waves = tokens * wpt;
      const int64_t grid = (waves + kWavesPerWG - 1) / kWavesPerWG;
      hipLaunchKernelGGL(k, dim3(static_cast<uint32_t>(grid)), dim3(kWavesPerWG * WAVE), 0, stream, L, kpw, wpt);
      return hipGetLastError() == hipSuccess ? 0 : -1;
    }
  }
  if (L.qI.dtype == CSA_F32 || L.qI.dtype == CSA_BF16) {
    dim3 grid(static_cast<uint32_t>((L.N + kSimtThreads - 1) / kSimtThreads), static_cast<uint32_t>(L.B * L.Tq));
    if (L.qI.dtype == CSA_F32)
      hipLaunchKernelGGL(index_simt_kernel<float>, grid, dim3(kSimtThreads), 0, stream, L);
    else
      hipLaunchKernelGGL(index_simt_kernel<uint16_t>, grid, dim3(kSimtThreads), 0, stream, L);
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  return -2;  // unsupported dtype
}

}  // namespace csa
