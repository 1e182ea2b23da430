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
#include "topk_select.h"

namespace csa {

namespace {

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
  c.omap = a.omap;
  c.tq = a.tq;
  load_slice<NT, PER, true>(c, r, v);
  select_slice<NT, PER, true, true>(c, sh, r, v);
}

// PAIRS: input is (value, index) candidates; FINAL: write indices (and count) only.
template <int NT, int PER, bool PAIRS, bool FINAL>
__global__ __launch_bounds__(NT) void topk_kernel(TopkArgs a) {
  if constexpr (FINAL) {
    // workgroups past the rows' own run the appended normalization job (uniform per
    // workgroup; the selection below never waits on them)
    if (a.side.blocks > 0 && blockIdx.x >= a.main_blocks) {
      attn_norm_block<NT / WAVE>(a.side, blockIdx.x - a.main_blocks);
      return;
    }
  }
  __shared__ Shared<NT> sh;
  float v[PER];
  load_slice<NT, PER, PAIRS, FINAL>(a, blockIdx.x, v);
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
// only the selections of a few rows (decode): one level, or the first of two.
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
  // ... of at most twice that: two halves a row, then the 2k candidates in one small
  // workgroup (a decode row just past 32768 entries)
  if (N <= 2 * kOneLevelMax && rows <= 64 && 2 * static_cast<int64_t>(k) <= kMaxSlice) {
    L.n = 2;
    L.len[0] = N;
    L.slice[0] = (N + 1) / 2;
    L.slices[0] = 2;
    L.len[1] = 2 * static_cast<int64_t>(k);
    L.slice[1] = L.len[1];
    L.slices[1] = 1;
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

// the final launch's block count with a side job shaped for its workgroups (and its
// output translation to pool rows)
int64_t with_side(TopkArgs& a, int64_t blocks, const Shape& s, const AttnNormArgs* side, const PageMap* out_map,
                  int64_t tq) {
  a.main_blocks = static_cast<uint32_t>(blocks);
  if (out_map) a.omap = *out_map;
  a.tq = tq > 0 ? tq : 1;
  if (!side) return blocks;
  a.side = *side;
  attn_norm_shape(a.side, s.nt / WAVE);
  return blocks + a.side.blocks;
}

int run_levels(const float* scores, int64_t rows, int64_t N, int k, int32_t* idx, int32_t* count, char* w,
               size_t one, const Levels& L, const float* row_tau, int32_t* redo, int32_t* cnt, hipStream_t stream,
               const AttnNormArgs* side, const PageMap* out_map, int64_t tq) {
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
    const int64_t blocks =
        final_level ? with_side(a, rows * L.slices[i], s, side, out_map, tq) : rows * L.slices[i];
    if (blocks >= (int64_t(1) << 32)) return -4;
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

// The last selection level over per-slice candidate lists ([rows, slices, k] values and
// entry indices in entry order, -inf / -1 padded): the lists of a row are concatenated
// (still in entry order) and selected once, exactly as the last level of run_levels.
int launch_topk_merge(const float* cand_val, const int32_t* cand_idx, int64_t rows, int slices, int k,
                      int32_t* idx, int32_t* count, hipStream_t stream, const AttnNormArgs* side,
                      const PageMap* out_map, int64_t tq) {
  if (rows == 0) return 0;
  TopkArgs a{};
  a.in_val = cand_val;
  a.in_idx = cand_idx;
  a.n_in = static_cast<int64_t>(slices) * k;
  a.slice = a.n_in;
  a.slices = 1;
  a.k = k;
  a.out_idx = idx;
  a.count = count;
  if (a.n_in > kShapes[3].cap()) return -2;
  const Shape s = shape_for(a.n_in);
  const int64_t blocks = with_side(a, rows, s, side, out_map, tq);
  if (blocks >= (int64_t(1) << 32)) return -4;
  launch_shape<true, true>(s, blocks, a, stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_topk(const float* scores, int64_t rows, int64_t N, int k, int32_t* idx, int32_t* count, void* ws,
                hipStream_t stream, const AttnNormArgs* side, const PageMap* out_map, int64_t tq) {
  if (rows == 0) return 0;
  const Levels L = N > 0 ? plan_levels(rows, N, k) : Levels{1, {0}, {1}, {1}};
  const size_t one = level_buffer_bytes(rows, L, k);
  char* w = static_cast<char*>(ws);
  const uint32_t rank = N > 0 ? tau_rank(rows, N, k, L) : 0u;
  if (rank == 0) return run_levels(scores, rows, N, k, idx, count, w, one, L, nullptr, nullptr, nullptr, stream, side, out_map, tq);
  float* tau = reinterpret_cast<float*>(w + 2 * one);
  int32_t* redo = reinterpret_cast<int32_t*>(w + 2 * one + static_cast<size_t>(rows) * 4);
  int32_t* cnt = reinterpret_cast<int32_t*>(w + 2 * one + static_cast<size_t>(rows) * 8);
  constexpr int64_t rows_per_wg = kTauThreads / WAVE;
  hipLaunchKernelGGL(topk_tau_kernel, dim3(static_cast<uint32_t>((rows + rows_per_wg - 1) / rows_per_wg)),
                     dim3(kTauThreads), 0, stream, scores, rows, N, rank, tau);
  if (hipGetLastError() != hipSuccess) return -1;
  return run_levels(scores, rows, N, k, idx, count, w, one, L, tau, redo, cnt, stream, side, out_map, tq);
}

}  // namespace csa
