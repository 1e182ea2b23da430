// Exact top-k selection inside one workgroup: the building blocks of the top-k
// selector (topk.hip) and of the lightning indexer's fused decode selection
// (indexer.hip).  [V4-CN] "DeepSeek-V4中文翻译" §2.3.1 (the top-k selector keeps k
// compressed entries per query).
//
// Result of a selection: the min(k, #finite) largest values of a slice, ties broken
// towards the lower position, written in position order (candidate lists keep
// (value, index) pairs in index order), padded with -inf / -1.
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
#pragma once

#include "device_common.h"
#include "rmsnorm.h"

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
  // final level: workgroups main_blocks .. main_blocks + side.blocks - 1 run an
  // independent normalization job instead (side.blocks = 0: none)
  uint32_t main_blocks;
  AttnNormArgs side;
  // final level: omap.table != NULL writes each selected entry as its pool row in a
  // paged cache (selection row r belongs to batch row r / tq)
  PageMap omap;
  int64_t tq;
};

constexpr int kFewCand = 64;  // a threshold bin this small is resolved by one wave
constexpr int kPageLds = 1024;  // block-table entries a final level stages in LDS
constexpr int kMaxTopK = 4096;  // largest k (the entry points reject more)

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

// cache-policy bits of a buffer load: the nontemporal hint
constexpr int kCachePolicyNT = 2;

// Load slice blk's values: thread t holds entries t + NT j of the slice.  FINAL: the
// slice is the whole row of a one-level selection.
template <int NT, int PER, bool PAIRS, bool FINAL = false>
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
  // a row cut into slices is read once and is too long to stay in the caches:
  // nontemporal loads (measured a few per cent faster there); a row selected whole
  // comes straight from the indexer and is read through the caches that still hold it
  constexpr bool kStream = !PAIRS && !FINAL;
  if (n == NT * PER) {
#pragma unroll
    for (int j = 0; j < PER; ++j) v[j] = kStream ? __builtin_nontemporal_load(src + j * NT + tid) : src[j * NT + tid];
  } else {
    // loads past the slice return 0 (hardware range check) and are replaced by -inf
    const __amdgpu_buffer_rsrc_t bs = buffer_view(src, static_cast<int64_t>(n) * 4);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const float x = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(bs, 4 * (j * NT + tid), 0, kStream ? kCachePolicyNT : 0));
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
  // paged output: the row's block-table row, fetched now and read after the selection
  // (the selection's barriers order the LDS stores before those reads)
  __shared__ int32_t pg_lds[FINAL ? kPageLds : 1];
  const bool pg_in_lds = FINAL && a.omap.table && a.omap.max_pages <= kPageLds;
  if (pg_in_lds) {
    const int32_t* row = a.omap.table + static_cast<int64_t>(a.omap.slot[r / a.tq]) * a.omap.max_pages;
    for (int i = tid; i < a.omap.max_pages; i += NT) pg_lds[i] = row[i];
  }

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
  if (tid == 0) {
    sh.ncand = 0u;
    sh.cand[0] = 0xffffffffu;  // the threshold bin's smallest and largest key (crowded bins)
    sh.cand[1] = 0u;
  }
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
      } else {
        // a crowded threshold bin: when all its entries hold one value (scores rounded
        // to few distinct values, as BF16 scores are) that value is the threshold
#pragma unroll
        for (int j = 0; j < PER; ++j) {
          if (((binp[j / 2] >> (16 * (j & 1))) & 0xffffu) == tb) {
            const uint32_t key = score_key(v[j]);
            atomicMin(&sh.cand[0], key);
            atomicMax(&sh.cand[1], key);
          }
        }
        __syncthreads();
        if (sh.cand[0] == sh.cand[1]) {
          theta = key_value(sh.cand[0]);
          ties = rem;
          total_eq = cnt;
          found = true;
        }
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
  // The last level stages the selected entries in LDS at their output slots and writes
  // them (as pool rows for a paged cache) in one coalesced pass afterwards: each of the
  // unrolled rounds below is then a few instructions, where translating in place put a
  // page lookup into every round (the rounds run once per launch, from a cold
  // instruction cache, so their code size is their cost).
  __shared__ int32_t stg[FINAL ? kMaxTopK : 1];
  auto put = [&](int j, uint32_t slot) {
    const int32_t e = PAIRS ? ix[PAIRS ? j : 0] : static_cast<int32_t>(lo + j * NT + tid);
    if (FINAL) {
      stg[slot] = e;
    } else {
      oi[slot] = e;
      ov[slot] = v[j];
    }
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
  if (FINAL) {
    __syncthreads();
    const int n_sel = static_cast<int>(total_sel);
    const int psh = a.omap.shift;
    const int32_t pmask = (1 << psh) - 1;
    if (pg_in_lds) {
      for (int i = tid; i < a.k; i += NT) {
        const int32_t e = i < n_sel ? stg[i] : 0;
        oi[i] = i < n_sel ? ((pg_lds[e >> psh] << psh) | (e & pmask)) : -1;
      }
    } else if (a.omap.table) {
      const int32_t* trow = a.omap.table + static_cast<int64_t>(a.omap.slot[r / a.tq]) * a.omap.max_pages;
      for (int i = tid; i < a.k; i += NT) {
        const int32_t e = i < n_sel ? stg[i] : 0;
        oi[i] = i < n_sel ? ((trow[e >> psh] << psh) | (e & pmask)) : -1;
      }
    } else {
      for (int i = tid; i < a.k; i += NT) oi[i] = i < n_sel ? stg[i] : -1;
    }
  } else if (a.out_cnt) {
    if (tid == 0) a.out_cnt[r * a.slices + sl] = static_cast<int32_t>(total_sel);
  } else {
    for (int i = static_cast<int>(total_sel) + tid; i < a.k; i += NT) {
      oi[i] = -1;
      ov[i] = -INFINITY;
    }
  }
  if (FINAL && a.count && tid == 0) a.count[r] = static_cast<int32_t>(total_sel);
  return false;
}

}  // namespace

}  // namespace csa
