// K3: top-k selector over index-score rows.  [V4-CN] "DeepSeek-V4中文翻译" §2.3.1
// (the top-k selector keeps k compressed entries per query); [NOTES] C_t = TopK_k(I_t,:).
//
// Exact radix select, one workgroup of 16 waves per row:
//   1. scores become order-preserving uint32 keys (non-finite -> 0, never chosen);
//   2. four MSB-first 8-bit passes build LDS histograms of the keys that still
//      match the prefix; one wave finds the bin holding the k-th largest key with
//      a suffix scan, giving the exact threshold key theta and the number r of
//      theta-valued entries to take (lowest indices first);
//   3. an order-preserving compaction pass writes every key > theta and the first r
//      keys == theta in ascending index order: each thread owns 8 consecutive
//      entries, and wave prefix sums plus a 16-wave LDS scan give every entry its
//      output slot, so no sort is needed.  Unused slots get -1.
#include "device_common.h"
#include "launch.h"

namespace csa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / WAVE;
constexpr int kPer = 8;                 // consecutive entries per thread
constexpr int kTile = kThreads * kPer;  // entries per compaction tile

__device__ __forceinline__ void load_keys(const float* row, int64_t N, int64_t base, bool vec_ok,
                                          uint32_t key[kPer]) {
  if (vec_ok && base + kPer <= N) {
    float4 a = *reinterpret_cast<const float4*>(row + base);
    float4 b = *reinterpret_cast<const float4*>(row + base + 4);
    key[0] = score_key(a.x); key[1] = score_key(a.y); key[2] = score_key(a.z); key[3] = score_key(a.w);
    key[4] = score_key(b.x); key[5] = score_key(b.y); key[6] = score_key(b.z); key[7] = score_key(b.w);
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) key[j] = (base + j < N) ? score_key(row[base + j]) : 0u;
  }
}

// inclusive scan of a 32-bit value across the wave
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t u = __shfl_up(v, o, WAVE);
    if (lane >= o) v += u;
  }
  return v;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores, int64_t N, int k,
                                                        int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_tot[kWaves];
  __shared__ uint32_t sel_info[4];  // [0] chosen digit, [1] count above it, [2] finite count

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t r = blockIdx.x;
  const float* row = scores + r * N;
  int32_t* out = idx + r * static_cast<int64_t>(k);
  const bool vec_ok = (N & 3) == 0;

  uint32_t prefix = 0;       // fixed high bits of theta
  uint32_t pmask = 0;        // which bits of prefix are fixed
  uint32_t remaining = 0;    // how many keys >= theta (within prefix) still to take
  uint32_t finite = 0;

  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kThreads) hist[i] = 0u;
    __syncthreads();
    uint32_t my_finite = 0;
    for (int64_t base = static_cast<int64_t>(tid) * kPer; base < N; base += static_cast<int64_t>(kTile)) {
      uint32_t key[kPer];
      load_keys(row, N, base, vec_ok, key);
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (key[j] != 0u && (key[j] & pmask) == prefix) {
          atomicAdd(&hist[(key[j] >> shift) & 0xffu], 1u);
          ++my_finite;
        }
      }
    }
    if (pass == 0) {
      // number of finite scores (all keys match the empty prefix)
      uint32_t t = my_finite;
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) t += __shfl_xor(t, o, WAVE);
      if (lane == 0) wave_tot[wid] = t;
    }
    __syncthreads();
    if (pass == 0) {
      uint32_t tot = 0;
      for (int w = 0; w < kWaves; ++w) tot += wave_tot[w];
      finite = tot;
      remaining = finite < static_cast<uint32_t>(k) ? finite : static_cast<uint32_t>(k);
      if (finite <= static_cast<uint32_t>(k)) break;  // every finite score is selected
    }
    // wave 0 locates the bin holding the remaining-th largest key
    if (wid == 0) {
      uint32_t c[4];
      uint32_t local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = hist[4 * lane + j]; local += c[j]; }
      // suffix sum over lanes > lane
      uint32_t incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        uint32_t u = __shfl_down(incl, o, WAVE);
        if (lane + o < 64) incl += u;
      }
      uint32_t above = incl - local;  // keys in bins of higher lanes
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < remaining && remaining <= above + c[j]) {
          sel_info[0] = static_cast<uint32_t>(4 * lane + j);
          sel_info[1] = above;
        }
        above += c[j];
      }
    }
    __syncthreads();
    const uint32_t digit = sel_info[0];
    remaining -= sel_info[1];
    prefix |= digit << shift;
    pmask |= 0xffu << shift;
    __syncthreads();
  }

  // selection rule: key > theta, or key == theta among the first `ties` such keys
  uint32_t theta, ties;
  if (finite <= static_cast<uint32_t>(k)) {
    theta = 0u;   // key > 0 <=> finite score
    ties = 0u;
  } else {
    theta = prefix;
    ties = remaining;
  }
  const uint32_t total_sel = finite < static_cast<uint32_t>(k) ? finite : static_cast<uint32_t>(k);

  uint32_t run_gt = 0, run_tie = 0;  // totals of earlier tiles (uniform across the WG)
  for (int64_t tile = 0; tile < N; tile += kTile) {
    const int64_t base = tile + static_cast<int64_t>(tid) * kPer;
    uint32_t key[kPer];
    if (base < N) load_keys(row, N, base, vec_ok, key);
    else {
#pragma unroll
      for (int j = 0; j < kPer; ++j) key[j] = 0u;
    }
    uint32_t ngt = 0, ntie = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      ngt += key[j] > theta ? 1u : 0u;
      ntie += (key[j] == theta && key[j] != 0u) ? 1u : 0u;
    }
    const uint32_t packed = ngt | (ntie << 16);
    const uint32_t incl = wave_incl_scan(packed);
    if (lane == 63) wave_tot[wid] = incl;
    __syncthreads();
    uint32_t before = incl - packed;
    uint32_t tile_tot = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t t = wave_tot[w];
      if (w < wid) before += t;
      tile_tot += t;
    }
    __syncthreads();
    uint32_t gt_before = run_gt + (before & 0xffffu);
    uint32_t tie_before = run_tie + (before >> 16);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const bool gt = key[j] > theta;
      const bool tie = key[j] == theta && key[j] != 0u;
      if (gt || (tie && tie_before < ties)) {
        const uint32_t slot = gt_before + (tie_before < ties ? tie_before : ties);
        out[slot] = static_cast<int32_t>(base + j);
      }
      gt_before += gt ? 1u : 0u;
      tie_before += tie ? 1u : 0u;
    }
    run_gt += tile_tot & 0xffffu;
    run_tie += tile_tot >> 16;
  }
  for (int i = static_cast<int>(total_sel) + tid; i < k; i += kThreads) out[i] = -1;
  if (count && tid == 0) count[r] = static_cast<int32_t>(total_sel);
}

}  // namespace

size_t topk_workspace_bytes(int64_t, int64_t, int) { return 0; }

int launch_topk(const float* scores, int64_t rows, int64_t N, int k, int32_t* idx, int32_t* count, void*,
                hipStream_t stream) {
  if (rows == 0) return 0;
  hipLaunchKernelGGL(topk_kernel, dim3(static_cast<uint32_t>(rows)), dim3(kThreads), 0, stream, scores, N, k,
                     idx, count);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
