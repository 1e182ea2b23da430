// K3: top-k selector over index-score rows.  [V4-CN] "DeepSeek-V4中文翻译" §2.3.1
// (the top-k selector keeps k compressed entries per query); [NOTES] C_t = TopK_k(I_t,:).
//
// Result per row: the indices of the min(k, #finite) largest scores, ties broken
// towards the lower index, in ascending index order, padded with -1 (and the count).
//
// Scores are kept as floats (NaN and +-inf become -inf, which is never chosen; -0 and
// +0 compare equal).  A few rows of at most 32768 scores take one workgroup each;
// otherwise a row is cut into slices of at most 16384 scores and selection runs in
// (at most a few) levels:
//   level 1: one workgroup per (row, slice) keeps its slice's top-k as (value, index)
//            pairs in index order;
//   level n: the same selection over the concatenated candidate lists of a row
//            (which stay in index order); the last level writes the indices.
// An entry of the row's top-k is also in its slice's top-k (fewer than k entries of
// the slice beat it; a tie it wins by index it also wins inside the slice), so the
// levels are exact.  Short rows with many rows per launch take one level.
//
// Inside a workgroup every value stays in registers, thread t holding entries
// t, t + NT, t + 2 NT, ... (so each round of a wave covers 64 consecutive entries):
//   A. count of finite values (ballots) and their smallest / largest value;
//   B. the threshold value theta (the k-th largest) and the number of theta-valued
//      entries to keep: a histogram of the values on a linear scale between the
//      extremes (monotone bins); when the threshold bin holds at most 64 entries one
//      wave ranks them exactly.  Otherwise an MSB-first radix select with 11-bit
//      digits over order-preserving integer keys (at most three levels);
//   C. an order-preserving compaction: every value > theta and the first `ties`
//      values == theta, in index order.  Per (round, wave) counts from ballots go
//      through one workgroup prefix scan; inside a round a lane's slot is the
//      round's base plus the ballot bits below it.
#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace csa {

namespace {

constexpr int kBinBits = 11;
constexpr int kBins = 1 << kBinBits;
constexpr int kMaxSlice = 16384;  // keys per workgroup

struct TopkArgs {
  const float* scores;      // level 1 input: [rows, n_in]
  const float* in_val;      // later levels: [rows, n_in] candidate values (-inf = none)
  const int32_t* in_idx;    //               and their row indices
  int64_t n_in;             // input entries per row
  int64_t slice;            // entries per slice (workgroup)
  int slices;               // slices per row
  int k;
  float* out_val;           // candidate output: [rows, slices, k]
  int32_t* out_idx;         // candidate output [rows, slices, k], or the final [rows, k]
  int32_t* count;           // final level: [rows] or NULL
  // Pre-thresholded selection (many long rows): row_tau[r] is an estimate from below of
  // row r's k-th largest score.  A first-level slice whose entries >= tau fit in k keeps
  // just those.  The last level (of two) flags a row whose candidates turned out to miss
  // part of its top-k (redo[r] = 1, else 0), and a repair kernel recomputes such rows
  // one workgroup each, through the spare candidate buffer.
  const float* row_tau;     // first and last level: [rows] or NULL
  // ... whose first level then writes each slice's candidate count instead of padding
  // its k slots, and whose last level reads only the counted candidates (k a multiple
  // of the last level's thread count, so a thread's j-th slot lies in a uniform slice)
  int32_t* out_cnt;         // first level: [rows, slices] or NULL
  const int32_t* in_cnt;    // last level: [rows, n_in / k] or NULL
  int32_t* redo;            // last level and repair: [rows]
  int64_t n_row;            // repair: scores per row
  float* spare_val;         // repair: [rows, ceil(n_row / capacity), k] scratch
  int32_t* spare_idx;
};

constexpr int kFewCand = 64;  // a threshold bin this small is resolved by one wave

template <int NT>
struct Shared {
  // radix levels alternate between the two
  alignas(16) uint32_t hist[2][kBins + 4];
  alignas(16) uint4 wave_abc[NT / WAVE];
  uint32_t wave_a[NT / WAVE];
  uint32_t info[3];
  uint32_t ncand;
  uint32_t cand[kFewCand];
};

// the float a finite key encodes (inverse of score_key)
__device__ __forceinline__ float key_value(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Wave 0's step of a selection level: lane l owns bins [PB l, PB l + PB) of hc; finds
// the bin holding the remaining-th largest counted entry and writes (bin, entries in
// higher bins, entries in the bin) to info.  The bins are read twice from LDS rather
// than held in registers, which would cost PB registers in every thread.
__device__ __forceinline__ void find_bin(const uint32_t* hc, uint32_t remaining, uint32_t* info) {
  constexpr int PB = kBins / WAVE;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const uint4* hb = reinterpret_cast<const uint4*>(&hc[PB * lane]);
  uint32_t local = 0;
#pragma unroll 2
  for (int j = 0; j < PB / 4; ++j) {
    const uint4 v = hb[j];
    local += v.x + v.y + v.z + v.w;
  }
  const uint32_t pre = wave_prefix_sum(local);
  const uint32_t incl = __builtin_amdgcn_readlane(pre, 63) - pre + local;  // this lane and those above
  uint32_t above = incl - local;
  asm volatile("" ::: "memory");  // re-read the bins below instead of keeping them
  if (above < remaining && remaining <= incl) {  // the threshold bin is one of this lane's
    uint32_t bin = 0, abv = 0, cnt = 0;
#pragma unroll 1
    for (int q = PB / 4 - 1; q >= 0; --q) {
      const uint4 v = hb[q];
      const uint32_t cq[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < remaining && remaining <= above + cq[j]) {
          bin = static_cast<uint32_t>(PB * lane + 4 * q + j);
          abv = above;
          cnt = cq[j];
        }
        above += cq[j];
      }
    }
    info[0] = bin;
    info[1] = abv;
    info[2] = cnt;
  }
}

// The same step by the whole workgroup: thread t owns bins [BPT t, BPT t + BPT); the
// entries in higher bins come from a wave prefix sum and the per-wave totals.  Ends
// with a barrier after which info holds the result.
template <int NT>
__device__ __forceinline__ void find_bin_block(const uint32_t* hc, uint32_t remaining, Shared<NT>& sh) {
  constexpr int BPT = kBins / NT;
  constexpr int NW = NT / WAVE;
  static_assert(BPT >= 2 && BPT * NT == kBins, "bins per thread");
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int wid = tid >> 6;
  uint32_t c[BPT];
#pragma unroll
  for (int j = 0; j < BPT; j += 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(&hc[BPT * tid + j]);
    c[j] = v.x;
    c[j + 1] = v.y;
  }
  uint32_t local = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) local += c[j];
  const uint32_t incl = wave_prefix_sum(local);
  const uint32_t wtot = __builtin_amdgcn_readlane(incl, 63);
  if (lane == 63) sh.wave_a[wid] = wtot;
  __syncthreads();
  uint32_t above = wtot - incl;  // later lanes of this wave
#pragma unroll
  for (int w = 0; w < NW; ++w)
    if (w > wid) above += sh.wave_a[w];
  if (above < remaining && remaining <= above + local) {  // exactly one thread
    uint32_t bin = 0, abv = 0, cnt = 0;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (above < remaining && remaining <= above + c[j]) {
        bin = static_cast<uint32_t>(BPT * tid + j);
        abv = above;
        cnt = c[j];
      }
      above += c[j];
    }
    sh.info[0] = bin;
    sh.info[1] = abv;
    sh.info[2] = cnt;
  }
  __syncthreads();
}

__device__ __forceinline__ bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Raw buffer view of [p, p + bytes): dword loads past the end return 0 (hardware range
// check), so a partly filled thread range needs no per-element address or guard.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_view(const void* p, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(n), 0x00020000);
}

// Load slice blk's values: thread t holds entries t + NT j of the slice.
template <int NT, int PER, bool PAIRS>
__device__ __forceinline__ void load_slice(const TopkArgs& a, int64_t blk, float (&v)[PER]) {
  const int tid = static_cast<int>(threadIdx.x);
  const int64_t r = static_cast<uint32_t>(blk) / static_cast<uint32_t>(a.slices);
  const int sl = static_cast<int>(static_cast<uint32_t>(blk) % static_cast<uint32_t>(a.slices));
  const int64_t lo = static_cast<int64_t>(sl) * a.slice;
  const int n = static_cast<int>(min(a.n_in, lo + a.slice) - lo);  // <= NT * PER
  const float* src = (PAIRS ? a.in_val : a.scores) + r * a.n_in + lo;
  if (PAIRS && a.in_cnt) {
    // slot j NT + t lies in candidate list (j NT) / k (one slice per row here, lo = 0):
    // slots past that list's count read nothing (out of the buffer's range) and are -inf
    const __amdgpu_buffer_rsrc_t bs = buffer_view(src, static_cast<int64_t>(n) * 4);
    const int32_t* cnt = a.in_cnt + r * (a.n_in / a.k);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = j * NT;
      const int c = e < n ? cnt[e / a.k] : 0;  // wave-uniform
      const bool ok = (e % a.k) + tid < c;
      const float x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(bs, ok ? 4 * (e + tid) : 0x7ffffff0, 0, 0));
      v[j] = ok ? x : -INFINITY;
    }
    return;
  }
  if (n == NT * PER) {
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = src[j * NT + tid];
  } else {
    // loads past the slice return 0 (hardware range check) and are replaced by -inf
    const __amdgpu_buffer_rsrc_t bs = buffer_view(src, static_cast<int64_t>(n) * 4);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const float x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(bs, 4 * (j * NT + tid), 0, 0));
      v[j] = j * NT + tid < n ? x : -INFINITY;
    }
  }
  if (!PAIRS) {
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = __builtin_isfinite(v[j]) ? v[j] : -INFINITY;
  }
}

// lane J of `mine` gets f(J) (a wave-uniform value), for J = J0 .. PER-1
template <int J, int PER, typename F>
__device__ __forceinline__ void count_rounds(uint32_t& mine, const F& f) {
  if constexpr (J < PER) {
    const uint32_t c = f(J);
    asm volatile("v_writelane_b32 %0, %1, %2" : "+v"(mine) : "s"(c), "i"(J));
    count_rounds<J + 1, PER>(mine, f);
  }
}

__device__ __forceinline__ uint32_t lane_prefix(uint64_t m) {  // set bits of m below this lane
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
}

// Select slice blk's top-k from its values (every thread of the workgroup calls this;
// it holds barriers).  Returns true, having written nothing but the flag, when the row
// must be recomputed (last level of a pre-thresholded selection).
template <int NT, int PER, bool PAIRS, bool FINAL>
__device__ __forceinline__ bool select_slice(const TopkArgs& a, Shared<NT>& sh, int64_t blk, float (&v)[PER]) {
  constexpr int NW = NT / WAVE;
  static_assert(PER % 2 == 0 && PER <= 64, "rounds per thread");
  const int tid = static_cast<int>(threadIdx.x);
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t r = static_cast<uint32_t>(blk) / static_cast<uint32_t>(a.slices);
  const int sl = static_cast<int>(static_cast<uint32_t>(blk) % static_cast<uint32_t>(a.slices));
  const int64_t lo = static_cast<int64_t>(sl) * a.slice;
  const int n = static_cast<int>(min(a.n_in, lo + a.slice) - lo);
  const uint32_t K = static_cast<uint32_t>(a.k);

  // ---- A: finite count, smallest and largest finite value
  uint32_t nfin = 0;
  float vmax = -INFINITY, vmin = INFINITY;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const bool fin = v[j] > -INFINITY;
    nfin += fin ? 1u : 0u;
    vmax = fmaxf(vmax, v[j]);
    vmin = fminf(vmin, fin ? v[j] : INFINITY);
  }
  nfin = wave_sum_u32(nfin);
  // entries >= the row's estimated threshold (pre-thresholded first level)
  const float tau = (!PAIRS && a.row_tau) ? a.row_tau[r] : -INFINITY;
  uint32_t nge = 0;
  if (tau > -INFINITY) {
#pragma unroll
    for (int j = 0; j < PER; ++j) nge += v[j] >= tau ? 1u : 0u;
    nge = wave_sum_u32(nge);
  }
  {
    // extremes through order-preserving integer images (DPP reductions); +-inf map to
    // the ends of the order, and the values here are never NaN
    auto okey = [](float x) {
      const uint32_t u = __float_as_uint(x);
      return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    };
    vmax = key_value(wave_max_u32(okey(vmax)));
    vmin = key_value(wave_min_u32(okey(vmin)));
  }
  if (lane == 0) sh.wave_abc[wid] = make_uint4(nfin, __float_as_uint(vmax), __float_as_uint(vmin), nge);
  for (int i = tid; i < 2 * (kBins + 4); i += NT) (&sh.hist[0][0])[i] = 0u;
  if (tid == 0) sh.ncand = 0u;
  __syncthreads();
  nfin = 0;
  vmax = -INFINITY;
  vmin = INFINITY;
  nge = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint4 x = sh.wave_abc[w];
    nfin += x.x;
    vmax = fmaxf(vmax, __uint_as_float(x.y));
    vmin = fminf(vmin, __uint_as_float(x.z));
    nge += x.w;
  }
  // last level: fewer than k candidates while a finite threshold was applied, so
  // entries below it may belong to the row's top-k; the row is flagged for the repair
  if (FINAL && a.row_tau) {
    const bool shortfall = nfin < K && a.row_tau[r] > -INFINITY;
    if (tid == 0) a.redo[r] = shortfall ? 1 : 0;
    if (shortfall) return true;
  }

  // ---- B: threshold value theta and the number of theta-valued entries kept
  float theta;
  uint32_t ties, total_eq = 0;  // total_eq: entries == theta (needed when 0 < ties)
  uint32_t total_sel = nfin < K ? nfin : K;
  if (nfin <= K) {
    theta = -INFINITY;  // keep every finite value
    ties = 0u;
  } else if (tau > -INFINITY && nge <= K) {
    // every entry >= tau (all finite), in index order: one >= test
    theta = tau;
    ties = 1u;
    total_eq = 1u;
    total_sel = nge;
  } else if (vmin == vmax) {
    theta = vmax;  // every finite value is equal: the first k by index
    ties = K;
    total_eq = nfin;
  } else {
    bool found = false;
    const float scale = static_cast<float>(kBins) / (vmax - vmin);
    if (scale > 0.f && scale < INFINITY) {
      // bin = floor((v - vmin) * kBins / (vmax - vmin)), monotone in v, so each bin is
      // a contiguous value range; non-finite values (bin kBins) are not counted.  Scores
      // spread over many bins, so the atomics rarely meet and the threshold bin
      // usually holds a few entries, which one wave then ranks exactly.  Each value's
      // bin is kept (two 16-bit bins per register) for the gather.
      auto vbin = [&](float x) {
        const uint32_t b = static_cast<uint32_t>((x - vmin) * scale);
        return x > -INFINITY ? (b < static_cast<uint32_t>(kBins) ? b : static_cast<uint32_t>(kBins - 1))
                             : static_cast<uint32_t>(kBins);
      };
      uint32_t* h1 = sh.hist[1];
      uint32_t binp[PER / 2];
#pragma unroll
      for (int j = 0; j < PER; j += 2) {
        const uint32_t b0 = vbin(v[j]), b1 = vbin(v[j + 1]);
        if (b0 < static_cast<uint32_t>(kBins)) atomicAdd(&h1[b0], 1u);
        if (b1 < static_cast<uint32_t>(kBins)) atomicAdd(&h1[b1], 1u);
        binp[j / 2] = b0 | (b1 << 16);
      }
      __syncthreads();
      find_bin_block<NT>(h1, K, sh);
      const uint32_t tb = sh.info[0], rem = K - sh.info[1], cnt = sh.info[2];
      if (cnt <= kFewCand) {
        // gather the threshold bin's values (any order) and rank them in wave 0
#pragma unroll
        for (int j = 0; j < PER; ++j)
          if (((binp[j / 2] >> (16 * (j & 1))) & 0xffffu) == tb) sh.cand[atomicAdd(&sh.ncand, 1u)] = __float_as_uint(v[j]);
        __syncthreads();
        if (wid == 0) {
          const float c = lane < static_cast<int>(cnt) ? __uint_as_float(sh.cand[lane]) : 0.f;
          uint32_t gt = 0, eq = 0;
          for (int i = 0; i < static_cast<int>(cnt); ++i) {
            const float o = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__float_as_int(c), i));
            gt += o > c ? 1u : 0u;
            eq += o == c ? 1u : 0u;
          }
          // lanes holding the threshold value all write the same triple (every
          // theta-valued entry of the slice is in this bin)
          if (lane < static_cast<int>(cnt) && gt < rem && rem <= gt + eq) {
            sh.info[0] = __float_as_uint(c);
            sh.info[1] = rem - gt;
            sh.info[2] = eq;
          }
        }
        __syncthreads();
        theta = __uint_as_float(sh.info[0]);
        ties = sh.info[1];
        total_eq = sh.info[2];
        found = true;
      }
    }
    if (!found) {
      // radix levels over w = key - kmin + 1 of the order-preserving integer keys
      // (finite values give 1 .. span + 1, 0 = not finite), held in v's registers as
      // bit patterns and turned back into values afterwards
      const uint32_t kmin = score_key(vmin), kmax = score_key(vmax);
      const uint32_t koff = kmin - 1u;
#pragma unroll
      for (int j = 0; j < PER; ++j) v[j] = __uint_as_float(v[j] > -INFINITY ? score_key(v[j]) - koff : 0u);
      const uint32_t span = kmax - kmin;
      int shift = 32 - __clz(span);  // low bits of w - 1 still to decide
      uint32_t pval = 0, pmask = 0, remaining = K;
      uint32_t theta_w;
      // one level: histogram of the matching keys' next digit (hist[cur], cleared before),
      // barrier; wave 0 finds the threshold digit while the other waves clear the other
      // histogram for the next level; barrier; everyone reads the result
      for (int cur = 0;; cur ^= 1) {
        const int nsh = shift > kBinBits ? shift - kBinBits : 0;
        const uint32_t dmask = (1u << (shift - nsh)) - 1u;
        uint32_t* hc = sh.hist[cur];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          const uint32_t w = __float_as_uint(v[j]);
          const uint32_t x = w - 1u;
          if (w != 0u && (x & pmask) == pval) atomicAdd(&hc[(x >> nsh) & dmask], 1u);
          if ((j & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bound the addresses computed ahead
        }
        __syncthreads();
        if (wid == 0) {
          find_bin(hc, remaining, sh.info);
        } else if (nsh > 0) {
          uint32_t* hn = sh.hist[cur ^ 1];
          for (int i = tid - WAVE; i < kBins; i += NT - WAVE) hn[i] = 0u;
        }
        __syncthreads();
        remaining -= sh.info[1];
        pval |= sh.info[0] << nsh;
        pmask |= dmask << nsh;
        if (sh.info[2] == remaining) {
          // the threshold bin holds exactly the entries still needed: take all of it,
          // i.e. every key above w = pval (the bin's lowest is pval + 1)
          theta_w = pval;
          ties = 0u;
          break;
        }
        if (nsh == 0) {
          theta_w = pval + 1u;  // the exact threshold key
          ties = remaining;
          total_eq = sh.info[2];  // the last level's bin holds exactly that key
          break;
        }
        shift = nsh;
      }
      theta = key_value(theta_w + koff);  // w = 0 + koff >= the key below every finite value
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const uint32_t w = __float_as_uint(v[j]);
        v[j] = w != 0u ? key_value(w + koff) : -INFINITY;
      }
    }
  }

  // ---- C: per (round, wave) counts, then one prefix scan in index order (round-major,
  // then wave); the histograms are free now.  When every theta-valued entry or none is
  // kept one comparison selects (count in the low half); otherwise the counts of
  // v > theta and v == theta are packed in the two halves.
  const bool one_test = ties == 0u || ties == total_eq;
  const bool with_eq = ties != 0u;
  uint32_t* tab = sh.hist[0];  // [NW][PER]
  uint32_t mine = 0;           // lane j < PER: this wave's count(s) of round j
  // the (wave-uniform) count of round j goes straight into lane j
  if (one_test && with_eq) {
    count_rounds<0, PER>(mine, [&](int j) { return static_cast<uint32_t>(__popcll(__ballot(v[j] >= theta))); });
  } else if (one_test) {
    count_rounds<0, PER>(mine, [&](int j) { return static_cast<uint32_t>(__popcll(__ballot(v[j] > theta))); });
  } else {
    count_rounds<0, PER>(mine, [&](int j) {
      return static_cast<uint32_t>(__popcll(__ballot(v[j] > theta))) |
             (static_cast<uint32_t>(__popcll(__ballot(v[j] == theta))) << 16);
    });
  }
  if (lane < PER) tab[wid * PER + lane] = mine;
  __syncthreads();
  // lane j < PER of wave w: the entries before round j of wave w in index order are
  // all of rounds < j plus round j of waves < w; every wave reads the whole table
  // instead of a separate scan pass (two barriers fewer)
  uint32_t row = 0, before_w = 0;
  if (lane < PER) {
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const uint32_t c = tab[w * PER + lane];
      row += c;
      before_w += w < wid ? c : 0u;
    }
  }
  const uint32_t base = wave_prefix_sum(row) - row + before_w;  // lane j: round j's prefix
  // candidate indices, loaded now that the selection registers are free
  int32_t ix[PAIRS ? PER : 1];
  if (PAIRS) {
    const __amdgpu_buffer_rsrc_t bi = buffer_view(a.in_idx + r * a.n_in + lo, static_cast<int64_t>(n) * 4);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      // slots holding no candidate (-inf) are never selected: their index is not read
      const uint32_t off = (a.in_cnt && !(v[j] > -INFINITY)) ? 0x7ffffff0u : 4u * (j * NT + tid);
      ix[j] = static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(bi, off, 0, 0));
    }
  }
  int32_t* oi;
  float* ov = nullptr;
  if (FINAL) {
    oi = a.out_idx + r * static_cast<int64_t>(a.k);
  } else {
    const int64_t o = (r * a.slices + sl) * static_cast<int64_t>(a.k);
    oi = a.out_idx + o;
    ov = a.out_val + o;
  }
  auto put = [&](int j, uint32_t slot) {
    oi[slot] = PAIRS ? ix[PAIRS ? j : 0] : static_cast<int32_t>(lo + j * NT + tid);
    if (!FINAL) ov[slot] = v[j];
  };
  if (one_test && with_eq) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t bj = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(base), j));
      const bool sel = v[j] >= theta;
      if (sel) put(j, bj + lane_prefix(__ballot(sel)));
    }
  } else if (one_test) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t bj = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(base), j));
      const bool sel = v[j] > theta;
      if (sel) put(j, bj + lane_prefix(__ballot(sel)));
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const uint32_t bj = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(base), j));
      const bool gt = v[j] > theta, eq = v[j] == theta;
      const uint32_t gb = (bj & 0xffffu) + lane_prefix(__ballot(gt));
      const uint32_t tbf = (bj >> 16) + lane_prefix(__ballot(eq));
      if (gt || (eq && tbf < ties)) put(j, gb + (tbf < ties ? tbf : ties));
    }
  }
  if (!FINAL && a.out_cnt) {
    if (tid == 0) a.out_cnt[r * a.slices + sl] = static_cast<int32_t>(total_sel);
  } else {
    for (int i = static_cast<int>(total_sel) + tid; i < a.k; i += NT) {
      oi[i] = -1;
      if (!FINAL) ov[i] = -INFINITY;
    }
  }
  if (FINAL && a.count && tid == 0) a.count[r] = static_cast<int32_t>(total_sel);
  return false;
}

// Exact selection of row r inside one workgroup, for a row whose pre-thresholded
// candidates fell short: the row's slices of NT * PER scores one after another, each
// slice's top-k into the row's part of the spare buffer, then the top-k of those.
template <int NT, int PER>
__device__ __forceinline__ void redo_row(const TopkArgs& a, Shared<NT>& sh, int64_t r) {
  constexpr int64_t cap = static_cast<int64_t>(NT) * PER;
  float v[PER];
  TopkArgs b{};
  b.scores = a.scores;
  b.n_in = a.n_row;
  b.slice = cap;
  b.slices = static_cast<int>((a.n_row + cap - 1) / cap);
  b.k = a.k;
  b.out_val = a.spare_val;
  b.out_idx = a.spare_idx;
  for (int j = 0; j < b.slices; ++j) {
    const int64_t blk = r * b.slices + j;
    __syncthreads();  // the shared state is reused
    load_slice<NT, PER, false>(b, blk, v);
    select_slice<NT, PER, false, false>(b, sh, blk, v);
  }
  __threadfence();  // the candidates are read back by other waves of this workgroup
  __syncthreads();
  TopkArgs c{};
  c.in_val = a.spare_val;
  c.in_idx = a.spare_idx;
  c.n_in = static_cast<int64_t>(b.slices) * a.k;  // <= cap (checked by the host)
  c.slice = c.n_in;
  c.slices = 1;
  c.k = a.k;
  c.out_idx = a.out_idx;
  c.count = a.count;
  load_slice<NT, PER, true>(c, r, v);
  select_slice<NT, PER, true, true>(c, sh, r, v);
}

// PAIRS: input is (value, index) candidates; FINAL: write indices (and count) only.
template <int NT, int PER, bool PAIRS, bool FINAL>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  __shared__ Shared<NT> sh;
  float v[PER];
  load_slice<NT, PER, PAIRS>(a, blockIdx.x, v);
  select_slice<NT, PER, PAIRS, FINAL>(a, sh, blockIdx.x, v);
}

// Rows flagged by the last level, each recomputed by one workgroup (most launches find
// none: every workgroup reads its rows' flags and ends)
template <int NT, int PER>
__global__ __launch_bounds__(NT) void topk_repair_kernel(TopkArgs a, int64_t rows) {
  __shared__ Shared<NT> sh;
  __shared__ int32_t flag[NT];
  const int tid = static_cast<int>(threadIdx.x);
  // rows blockIdx.x + gridDim.x * i; one flag per thread and chunk, all read at once
  for (int64_t c0 = 0; c0 * gridDim.x + blockIdx.x < rows; c0 += NT) {
    const int64_t rr = (c0 + tid) * gridDim.x + blockIdx.x;
    const int32_t f = rr < rows ? a.redo[rr] : 0;
    flag[tid] = f;
    if (!__syncthreads_or(f)) continue;
    for (int i = 0; i < NT; ++i) {
      if (flag[i] == 0) continue;  // the same for the whole workgroup
      redo_row<NT, PER>(a, sh, (c0 + i) * gridDim.x + blockIdx.x);
      __syncthreads();
    }
    __syncthreads();  // flag[] is rewritten by the next chunk
  }
}

// The rank-th largest of a spread sample of the row (kTauRuns runs of kTauRun
// consecutive scores, evenly spaced; few runs, so few pages per row; shifted by a
// row-dependent multiple of 64 scores, so rows with a power-of-two length do not all
// start their runs on the same memory channels) estimates the row's k-th largest from below when rank is a
// few times k * sample / N: the fraction of the row at or above the sample's rank-th
// largest has mean rank / sample and relative spread 1 / sqrt(rank).  One wave per
// row finds it, to 16 bits, by a bitwise search over order-preserving keys (non-finite
// = 0, below everything); -inf when fewer than rank sampled scores are finite.
constexpr int kTauThreads = 256;
constexpr int kTauRuns = 4;
constexpr int kTauRun = 1024;
constexpr int kTauSample = kTauRuns * kTauRun;
constexpr int kTauJitter = 64 * 64;  // largest run shift
__global__ __launch_bounds__(kTauThreads) void topk_tau_kernel(const float* scores, int64_t rows, int64_t N,
                                                               uint32_t rank, float* tau) {
  constexpr int PER = kTauSample / WAVE;
  const int lane = static_cast<int>(threadIdx.x) & 63;
  const int64_t r = static_cast<int64_t>(blockIdx.x) * (kTauThreads / WAVE) + (threadIdx.x >> 6);
  if (r >= rows) return;  // no barriers below
  const int64_t step = ((N - kTauRun - kTauJitter) / (kTauRuns - 1)) & ~static_cast<int64_t>(63);
  const float* row = scores + r * N + ((static_cast<uint32_t>(r) * 2654435761u) >> 26) * 64;
  uint32_t key[PER];
  if ((N & 3) == 0 && (reinterpret_cast<uintptr_t>(scores) & 15) == 0) {
    // 16-byte loads: lane l holds scores 4 l .. 4 l + 3 of each 256-score piece
#pragma unroll
    for (int j = 0; j < PER; j += 4) {
      const int piece = j / 4;  // kTauRun / 256 pieces per run
      const float4 x = *reinterpret_cast<const float4*>(
          row + (piece / (kTauRun / 256)) * step + (piece % (kTauRun / 256)) * 256 + 4 * lane);
      key[j] = score_key(x.x);
      key[j + 1] = score_key(x.y);
      key[j + 2] = score_key(x.z);
      key[j + 3] = score_key(x.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j)
      key[j] = score_key(row[(j / (kTauRun / WAVE)) * step + (j % (kTauRun / WAVE)) * WAVE + lane]);
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    // a plain register value: otherwise the compiler keeps each key's finiteness as a
    // lane mask and re-tests it in every step of the search
    asm volatile("" : "+v"(key[j]));
  }
  // the top 16 key bits suffice (the low ones cleared, T stays a lower bound of the
  // rank-th largest key); counts come from ballots, so the sums are scalar
  uint32_t T = 0;
  for (int b = 31; b >= 16; --b) {
    const uint32_t cand = T | (1u << b);
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      c += static_cast<uint32_t>(__popcll(__ballot(key[j] >= cand)));
      if ((j & 7) == 7) __builtin_amdgcn_sched_barrier(0);  // bound the masks held at once
    }
    if (c >= rank) T = cand;
  }
  if (lane == 0) tau[r] = T != 0u ? key_value(T) : -INFINITY;
}

// workgroup shapes: (threads, keys per thread), slice capacity = threads * keys
struct Shape {
  int nt, per;
  int64_t cap() const { return static_cast<int64_t>(nt) * per; }
};
// 16384-entry slices take 512 threads of 32 entries: two workgroups share a CU, so the
// barrier-separated phases of one overlap the other's.  The 32768-entry shape serves
// only single-level selections of a few rows.
constexpr Shape kShapes[] = {{256, 16}, {512, 16}, {512, 32}, {1024, 32}};
constexpr int64_t kOneLevelMax = 32768;  // a row this long may take one workgroup

Shape shape_for(int64_t n) {
  for (const Shape& s : kShapes)
    if (s.cap() >= n) return s;
  return kShapes[3];
}

template <int NT, int PER, bool PAIRS, bool FINAL>
void launch_nt(int64_t blocks, const TopkArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((topk_kernel<NT, PER, PAIRS, FINAL>), dim3(static_cast<uint32_t>(blocks)), dim3(NT), 0, stream, a);
}

template <bool PAIRS, bool FINAL>
void launch_shape(const Shape& s, int64_t blocks, const TopkArgs& a, hipStream_t stream) {
  if (s.nt == 256) launch_nt<256, 16, PAIRS, FINAL>(blocks, a, stream);
  else if (s.per == 16) launch_nt<512, 16, PAIRS, FINAL>(blocks, a, stream);
  else if (s.nt == 512) launch_nt<512, 32, PAIRS, FINAL>(blocks, a, stream);
  else launch_nt<1024, 32, PAIRS, FINAL>(blocks, a, stream);
}

void launch_repair(const Shape& s, int64_t rows, const TopkArgs& a, hipStream_t stream) {
  const dim3 g(static_cast<uint32_t>(std::min<int64_t>(rows, 32)));
  if (s.nt == 256) hipLaunchKernelGGL((topk_repair_kernel<256, 16>), g, dim3(256), 0, stream, a, rows);
  else if (s.per == 16) hipLaunchKernelGGL((topk_repair_kernel<512, 16>), g, dim3(512), 0, stream, a, rows);
  else if (s.nt == 512) hipLaunchKernelGGL((topk_repair_kernel<512, 32>), g, dim3(512), 0, stream, a, rows);
  else hipLaunchKernelGGL((topk_repair_kernel<1024, 32>), g, dim3(1024), 0, stream, a, rows);
}

// Selection levels: input entries per row, slice length and slices per row of each.
struct Levels {
  int n;
  int64_t len[16], slice[16];
  int slices[16];
};

Levels plan_levels(int64_t rows, int64_t N, int k) {
  Levels L{};
  // a few rows of at most 32768 entries: one workgroup per row and one level, which
  // ends sooner than two levels of many workgroups each
  if (N <= kOneLevelMax && rows <= 64) {
    L.n = 1;
    L.len[0] = N;
    L.slice[0] = N;
    L.slices[0] = 1;
    return L;
  }
  // level-1 slices: halved from 32768 (not below 4096 or 2k) while the launch has fewer
  // workgroups than compute units and one further level still covers the candidates
  int64_t sl = kMaxSlice;
  while (sl > 4096 && sl / 2 >= 2 * static_cast<int64_t>(k) && rows * ((N + sl - 1) / sl) < 256 &&
         ((N + sl / 2 - 1) / (sl / 2)) * k <= kMaxSlice)
    sl /= 2;
  int64_t len = N;
  int i = 0;
  // k <= kMaxSlice / 4, so every level shrinks a row at least 2.5x: 16 levels cover N < 2^31
  while (i < 15 && (len > kMaxSlice || (i == 0 && len > sl))) {
    const int64_t s = i == 0 ? sl : kMaxSlice;
    L.len[i] = len;
    L.slice[i] = s;
    L.slices[i] = static_cast<int>((len + s - 1) / s);
    len = static_cast<int64_t>(L.slices[i]) * k;
    ++i;
  }
  L.len[i] = len;
  L.slice[i] = len;
  L.slices[i] = 1;
  L.n = i + 1;
  return L;
}

size_t level_buffer_bytes(int64_t rows, const Levels& L, int k) {
  int64_t mx = 0;
  for (int i = 0; i + 1 < L.n; ++i) mx = std::max<int64_t>(mx, static_cast<int64_t>(L.slices[i]) * k);
  return (static_cast<size_t>(rows * mx) * (sizeof(uint32_t) + sizeof(int32_t)) + 255) / 256 * 256;
}

// Pre-thresholding pays off for many long rows: the sample rank aims at 4k entries per
// row at or above the estimate, and a first-level slice's expected share of those must
// stay well under k (so slices nearly always take the cheap path).
uint32_t tau_rank(int64_t rows, int64_t N, int k, const Levels& L) {
  if (L.n != 2 || rows < 256 || N < 8 * L.slice[0] || N < 4 * static_cast<int64_t>(kTauSample)) return 0;
  // a row recomputed by the last level's workgroup: slices of its capacity, whose
  // candidates fit it (and the spare buffer)
  const int64_t cap = shape_for(L.slice[1]).cap();
  const int64_t sl = (N + cap - 1) / cap;
  if (sl * k > cap || sl > L.slices[0]) return 0;
  const int64_t rank = (4 * static_cast<int64_t>(k) * kTauSample + N - 1) / N;
  return rank >= 1 && rank <= kTauSample / 8 ? static_cast<uint32_t>(rank) : 0u;
}

// thresholds and repair flags, then the first level's per-slice candidate counts
size_t tau_bytes(int64_t rows, const Levels& L) {
  return (static_cast<size_t>(rows) * (8 + 4 * static_cast<size_t>(L.slices[0])) + 255) / 256 * 256;
}

}  // namespace

// Workspace: two candidate buffers (keys + indices), sized for the largest level
// output, then (pre-thresholded selection) the row thresholds and repair flags.
size_t topk_workspace_bytes(int64_t rows, int64_t N, int k) {
  if (rows <= 0 || N <= 0) return 0;
  const Levels L = plan_levels(rows, N, k);
  if (L.n == 1) return 0;
  return 2 * level_buffer_bytes(rows, L, k) + (tau_rank(rows, N, k, L) ? tau_bytes(rows, L) : 0);
}

namespace {

int run_levels(const float* scores, int64_t rows, int64_t N, int k, int32_t* idx, int32_t* count, char* w,
               size_t one, const Levels& L, const float* row_tau, int32_t* redo, int32_t* cnt, hipStream_t stream) {
  const float* in_val = nullptr;
  const int32_t* in_idx = nullptr;
  for (int i = 0; i < L.n; ++i) {
    const bool final_level = i + 1 == L.n;
    TopkArgs a{};
    a.scores = scores;
    a.in_val = in_val;
    a.in_idx = in_idx;
    a.n_in = L.len[i];
    a.slice = L.slice[i] > 0 ? L.slice[i] : 1;
    a.slices = L.slices[i];
    a.k = k;
    a.count = count;
    if (i == 0 || final_level) a.row_tau = row_tau;
    // ragged candidate lists (pre-thresholded, two levels): see TopkArgs
    const bool ragged = row_tau && k % shape_for(L.slice[L.n - 1]).nt == 0;
    if (ragged && i == 0) a.out_cnt = cnt;
    if (ragged && final_level) a.in_cnt = cnt;
    if (final_level) {
      a.out_idx = idx;
      a.redo = redo;
    } else {
      char* buf = w + (i & 1) * one;
      const int64_t n_out = rows * static_cast<int64_t>(L.slices[i]) * k;
      a.out_val = reinterpret_cast<float*>(buf);
      a.out_idx = reinterpret_cast<int32_t*>(buf + n_out * sizeof(uint32_t));
    }
    const Shape s = shape_for(a.slice);
    const int64_t blocks = rows * L.slices[i];
    if (i == 0) {
      if (final_level) launch_shape<false, true>(s, blocks, a, stream);
      else launch_shape<false, false>(s, blocks, a, stream);
    } else {
      if (final_level) launch_shape<true, true>(s, blocks, a, stream);
      else launch_shape<true, false>(s, blocks, a, stream);
    }
    if (hipGetLastError() != hipSuccess) return -1;
    if (final_level && row_tau) {
      // flagged rows again, exactly, through the spare buffer (not the one holding
      // this level's input, which level 0 wrote)
      const int64_t cap = s.cap();
      const int64_t n_spare = rows * ((N + cap - 1) / cap) * k;
      char* spare = w + (i & 1) * one;
      a.n_row = N;
      a.spare_val = reinterpret_cast<float*>(spare);
      a.spare_idx = reinterpret_cast<int32_t*>(spare + n_spare * sizeof(uint32_t));
      launch_repair(s, rows, a, stream);
      if (hipGetLastError() != hipSuccess) return -1;
    }
    in_val = a.out_val;
    in_idx = a.out_idx;
  }
  return 0;
}

}  // namespace

int launch_topk(const float* scores, int64_t rows, int64_t N, int k, int32_t* idx, int32_t* count, void* ws,
                hipStream_t stream) {
  if (rows == 0) return 0;
  const Levels L = N > 0 ? plan_levels(rows, N, k) : Levels{1, {0}, {1}, {1}};
  const size_t one = level_buffer_bytes(rows, L, k);
  char* w = static_cast<char*>(ws);
  const uint32_t rank = N > 0 ? tau_rank(rows, N, k, L) : 0u;
  if (rank == 0) return run_levels(scores, rows, N, k, idx, count, w, one, L, nullptr, nullptr, nullptr, stream);
  float* tau = reinterpret_cast<float*>(w + 2 * one);
  int32_t* redo = reinterpret_cast<int32_t*>(w + 2 * one + static_cast<size_t>(rows) * 4);
  int32_t* cnt = reinterpret_cast<int32_t*>(w + 2 * one + static_cast<size_t>(rows) * 8);
  constexpr int64_t rows_per_wg = kTauThreads / WAVE;
  hipLaunchKernelGGL(topk_tau_kernel, dim3(static_cast<uint32_t>((rows + rows_per_wg - 1) / rows_per_wg)),
                     dim3(kTauThreads), 0, stream, scores, rows, N, rank, tau);
  if (hipGetLastError() != hipSuccess) return -1;
  return run_levels(scores, rows, N, k, idx, count, w, one, L, tau, redo, cnt, stream);
}

}  // namespace csa
