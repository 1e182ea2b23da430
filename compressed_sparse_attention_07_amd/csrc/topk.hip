// K3: top-k selector over index-score rows.  [V4-CN] "DeepSeek-V4中文翻译" §2.3.1
// (the top-k selector keeps k compressed entries per query); [NOTES] C_t = TopK_k(I_t,:).
//
// One workgroup of 16 waves per row.  Every score becomes an order-preserving uint32
// key once (non-finite -> 0, never chosen; -0 and +0 share a key), and all passes
// work on keys.  Each thread owns 32 consecutive keys of a 32768-key tile: rows up to
// that size stay in registers across every pass (read from memory once); longer rows
// stream tile by tile.  The exact threshold key theta (the k-th largest) and the
// number r of theta-valued entries to keep (lowest indices first) come from:
//   A. the finite count and the smallest / largest finite key;
//   B. a 2048-bin histogram of (key - min) >> shift, a monotone map spread over the
//      row's actual key range, so LDS atomic collisions stay rare even though index
//      scores share their leading bits; a suffix scan finds the bin holding the k-th
//      largest key;
//   C. the keys of that bin (typically a few dozen) are gathered in LDS and ranked.
// If the threshold bin is crowded (heavy ties), an exact MSB-first 8-bit radix
// select over the row takes over.  Finally an order-preserving compaction writes
// every key > theta and the first r keys == theta in ascending index order: wave
// prefix sums plus a 16-wave LDS scan give every entry its output slot, so no sort
// is needed.  Unused slots get -1.
#include "device_common.h"
#include "launch.h"

namespace csa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / WAVE;
constexpr int kPer = 32;                // consecutive entries per thread
constexpr int kTile = kThreads * kPer;  // entries per tile (32768)
constexpr int kBinBits = 11;
constexpr int kBins = 1 << kBinBits;
constexpr int kRankCap = 1024;          // candidates ranked directly in LDS

__device__ __forceinline__ void load_keys(const float* row, int64_t N, int64_t base, bool vec_ok,
                                          uint32_t (&key)[kPer]) {
  if (vec_ok && base + kPer <= N) {
#pragma unroll
    for (int q = 0; q < kPer / 4; ++q) {
      const float4 a = *reinterpret_cast<const float4*>(row + base + 4 * q);
      key[4 * q] = score_key(a.x);
      key[4 * q + 1] = score_key(a.y);
      key[4 * q + 2] = score_key(a.z);
      key[4 * q + 3] = score_key(a.w);
    }
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
    const uint32_t u = __shfl_up(v, o, WAVE);
    if (lane >= o) v += u;
  }
  return v;
}

struct Shared {
  uint32_t hist[kBins];
  uint32_t cand[kRankCap];
  uint32_t wave_a[kWaves], wave_b[kWaves], wave_c[kWaves];
  uint32_t info[4];
  uint32_t theta, ties, ncand;
};

// Exact MSB-first radix select of the k-th largest key (k < number of finite keys).
template <bool RES>
__device__ __forceinline__ void radix_select(const float* row, int64_t N, bool vec_ok, uint32_t k, Shared& sh,
                                             uint32_t (&key)[kPer], uint32_t* theta, uint32_t* ties) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  uint32_t prefix = 0, pmask = 0, remaining = k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kThreads) sh.hist[i] = 0u;
    __syncthreads();
    for (int64_t tb = 0; tb < N; tb += kTile) {
      if (!RES) load_keys(row, N, tb + static_cast<int64_t>(tid) * kPer, vec_ok, key);
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (key[j] != 0u && (key[j] & pmask) == prefix) atomicAdd(&sh.hist[(key[j] >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    if (wid == 0) {
      uint32_t c[4], local = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) { c[j] = sh.hist[4 * lane + j]; local += c[j]; }
      uint32_t incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_down(incl, o, WAVE);
        if (lane + o < 64) incl += u;
      }
      uint32_t above = incl - local;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < remaining && remaining <= above + c[j]) {
          sh.info[0] = static_cast<uint32_t>(4 * lane + j);
          sh.info[1] = above;
        }
        above += c[j];
      }
    }
    __syncthreads();
    remaining -= sh.info[1];
    prefix |= sh.info[0] << shift;
    pmask |= 0xffu << shift;
    __syncthreads();
  }
  *theta = prefix;
  *ties = remaining;
}

template <bool RES>
__global__ __launch_bounds__(kThreads) void topk_kernel(const float* __restrict__ scores, int64_t N, int k,
                                                        int32_t* __restrict__ idx, int32_t* __restrict__ count) {
  __shared__ Shared sh;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t r = blockIdx.x;
  const float* row = scores + r * N;
  int32_t* out = idx + r * static_cast<int64_t>(k);
  const bool vec_ok = (N & 3) == 0;
  const uint32_t K = static_cast<uint32_t>(k);
  uint32_t key[kPer];  // this thread's 32 keys of the current tile
  if (RES) load_keys(row, N, static_cast<int64_t>(tid) * kPer, vec_ok, key);

  // ---- A: finite count, smallest and largest finite key
  uint32_t nfin = 0, kmax = 0, kmin1 = 0xffffffffu;  // kmin1 = min(key - 1): 0 wraps to the top
  for (int64_t tb = 0; tb < N; tb += kTile) {
    if (!RES) load_keys(row, N, tb + static_cast<int64_t>(tid) * kPer, vec_ok, key);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      nfin += key[j] != 0u ? 1u : 0u;
      kmax = max(kmax, key[j]);
      kmin1 = min(kmin1, key[j] - 1u);
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    nfin += __shfl_xor(nfin, o, WAVE);
    kmax = max(kmax, static_cast<uint32_t>(__shfl_xor(kmax, o, WAVE)));
    kmin1 = min(kmin1, static_cast<uint32_t>(__shfl_xor(kmin1, o, WAVE)));
  }
  if (lane == 0) {
    sh.wave_a[wid] = nfin;
    sh.wave_b[wid] = kmax;
    sh.wave_c[wid] = kmin1;
  }
  __syncthreads();
  nfin = 0;
  kmax = 0;
  kmin1 = 0xffffffffu;
  for (int w = 0; w < kWaves; ++w) {
    nfin += sh.wave_a[w];
    kmax = max(kmax, sh.wave_b[w]);
    kmin1 = min(kmin1, sh.wave_c[w]);
  }
  const uint32_t kmin = kmin1 + 1u;

  uint32_t theta, ties;
  const uint32_t total_sel = nfin < K ? nfin : K;
  if (nfin <= K) {
    theta = 0u;  // key > 0 <=> finite score: take them all
    ties = 0u;
  } else if (kmin == kmax) {
    theta = kmax;  // every finite score is equal: the first k by index
    ties = K;
  } else {
    // ---- B: histogram of (key - kmin) >> shift over the row's key range
    const uint32_t span = kmax - kmin;
    const int bits = 32 - __clz(span);
    const int shift = bits > kBinBits ? bits - kBinBits : 0;
    for (int i = tid; i < kBins; i += kThreads) sh.hist[i] = 0u;
    if (tid == 0) sh.ncand = 0u;
    __syncthreads();
    for (int64_t tb = 0; tb < N; tb += kTile) {
      if (!RES) load_keys(row, N, tb + static_cast<int64_t>(tid) * kPer, vec_ok, key);
#pragma unroll
      for (int j = 0; j < kPer; ++j)
        if (key[j] != 0u) atomicAdd(&sh.hist[(key[j] - kmin) >> shift], 1u);
    }
    __syncthreads();
    if (wid == 0) {
      constexpr int PB = kBins / WAVE;  // bins per lane
      uint32_t local = 0;
      for (int j = 0; j < PB; ++j) local += sh.hist[PB * lane + j];
      uint32_t incl = local;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t u = __shfl_down(incl, o, WAVE);
        if (lane + o < 64) incl += u;
      }
      uint32_t above = incl - local;
      for (int j = PB - 1; j >= 0; --j) {
        const uint32_t c = sh.hist[PB * lane + j];
        if (above < K && K <= above + c) {
          sh.info[0] = static_cast<uint32_t>(PB * lane + j);
          sh.info[1] = above;
          sh.info[2] = c;
        }
        above += c;
      }
    }
    __syncthreads();
    const uint32_t bstar = sh.info[0];
    const uint32_t above = sh.info[1];
    const uint32_t ncand = sh.info[2];
    const uint32_t need = K - above;  // entries to take from the threshold bin (>= 1)
    if (ncand <= static_cast<uint32_t>(kRankCap)) {
      // ---- C: gather the threshold bin and rank it exactly
      for (int64_t tb = 0; tb < N; tb += kTile) {
        if (!RES) load_keys(row, N, tb + static_cast<int64_t>(tid) * kPer, vec_ok, key);
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          if (key[j] != 0u && ((key[j] - kmin) >> shift) == bstar) {
            const uint32_t slot = atomicAdd(&sh.ncand, 1u);
            sh.cand[slot] = key[j];
          }
        }
      }
      __syncthreads();
      for (uint32_t i = tid; i < ncand; i += kThreads) {
        const uint32_t ki = sh.cand[i];
        uint32_t gt = 0, eq = 0;
        for (uint32_t j = 0; j < ncand; ++j) {
          const uint32_t kj = sh.cand[j];
          gt += kj > ki ? 1u : 0u;
          eq += kj == ki ? 1u : 0u;
        }
        if (gt < need && need <= gt + eq) {
          sh.theta = ki;          // every writer stores the same pair
          sh.ties = need - gt;
        }
      }
      __syncthreads();
      theta = sh.theta;
      ties = sh.ties;
    } else {
      radix_select<RES>(row, N, vec_ok, K, sh, key, &theta, &ties);
    }
  }

  // ---- D: ordered compaction of key > theta, and the first `ties` keys == theta
  uint32_t run_gt = 0, run_tie = 0;  // totals of earlier tiles (uniform across the WG)
  for (int64_t tile = 0; tile < N; tile += kTile) {
    const int64_t base = tile + static_cast<int64_t>(tid) * kPer;
    if (!RES) load_keys(row, N, base, vec_ok, key);
    uint32_t ngt = 0, ntie = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      ngt += key[j] > theta ? 1u : 0u;
      ntie += (key[j] == theta && key[j] != 0u) ? 1u : 0u;
    }
    const uint32_t packed = ngt | (ntie << 16);
    const uint32_t incl = wave_incl_scan(packed);
    __syncthreads();
    if (lane == 63) sh.wave_a[wid] = incl;
    __syncthreads();
    uint32_t before = incl - packed;
    uint32_t tile_tot = 0;
    for (int w = 0; w < kWaves; ++w) {
      const uint32_t t = sh.wave_a[w];
      if (w < wid) before += t;
      tile_tot += t;
    }
    uint32_t gt_before = run_gt + (before & 0xffffu);
    uint32_t tie_before = run_tie + (before >> 16);
    if (ngt + ntie > 0) {
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
  if (N <= kTile)
    hipLaunchKernelGGL(topk_kernel<true>, dim3(static_cast<uint32_t>(rows)), dim3(kThreads), 0, stream, scores, N, k,
                       idx, count);
  else
    hipLaunchKernelGGL(topk_kernel<false>, dim3(static_cast<uint32_t>(rows)), dim3(kThreads), 0, stream, scores, N,
                       k, idx, count);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
