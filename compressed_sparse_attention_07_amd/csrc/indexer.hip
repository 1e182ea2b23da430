// K2: lightning-indexer scores
//     I[t, s] = sum_h w[t, h] * ReLU(q[t, h, :] . K[s, :])   for s < floor(pos_t / m),
// -inf for the other entries.  [V4-CN] "DeepSeek-V4中文翻译" §2.3.1 (index-score
// equation), §2.3.3 (a query only sees earlier compressed blocks).
//
// bf16 path: one wave owns one query token and a contiguous range of entries.  The
// token's indexer queries [HI, DI] stay in registers as the MFMA A operand (heads =
// rows); the wave streams its keys through a private LDS ring (whole contiguous KiBs
// per direct global->LDS load, 16-byte chunks XOR-swizzled by entry), reads each
// 16-entry tile back as the B operand, multiplies with v_mfma_f32_16x16x32_bf16, and
// reduces in the epilogue: every lane applies ReLU and the head weights to the 4
// heads x 1 entry it holds per head block, two cross-lane adds finish the sum over
// heads, and each lane stores one score of a 64-entry run (one coalesced 256-byte
// store per four tiles).  Rows longer than 256 bytes load the B operand straight from
// HBM instead (16 lanes x 64 contiguous bytes per load).
//
// Prefill path (bf16, many queries per sequence): a workgroup of 8 waves owns 16
// queries of one sequence and a range of keys.  Key tiles (128 keys) are brought into
// a 4-stage LDS ring by direct global->LDS loads and shared by all 16 queries; each
// wave keeps two queries' q^I in registers, so every key fragment read from LDS feeds
// 2 x HB MFMA chains.  The 16-byte chunks of each key row are XOR-swizzled by the key
// index (applied through the load addresses), so the 16 keys of an operand read hit
// distinct banks.
//
// MXFP4 path ([V4-CN] §3.4: the indexer QK in FP4): both operands are e2m1 codes with
// an e8m0 scale per 32 elements, fed to v_mfma_scale_f32_16x16x128_f8f6f4.  Its operand
// layout is the storage layout: lane (col, grp) holds 32 consecutive codes of row col
// (16 bytes, element 2i in the low nibble of byte i) for elements 32 grp .. 32 grp + 31
// of a 128-element step, plus that block's scale byte.  The products of the dequantized
// values are exact in fp32; accumulation is fp32.
//
// The SIMT kernels (fp32, or shapes the MFMA tilings do not cover) compute one score
// per thread with the token's queries staged (dequantized) in LDS.
#include "device_common.h"
#include "launch.h"

#include <algorithm>
#include "topk_select.h"

namespace csa {

namespace {

// max(x, 0) as one integer max of the bit pattern: a float with the sign bit set is a
// negative integer and becomes +0, any other value is unchanged.  fmaxf on an MFMA
// result costs two instructions, the first quieting a possible signalling NaN.
__device__ __forceinline__ float relu_bits(float x) { return __int_as_float(max(__float_as_int(x), 0)); }


// A score as stored: fp32, or rounded to bf16 (nearest-even) for the BF16-score
// variant ([V4-CN] §3.4 stores the index scores in BF16 for a faster selection).
__device__ __forceinline__ float stored_score(const IndexLaunch& a, float v) {
  return a.score_bf16 ? __uint_as_float(static_cast<uint32_t>(f32_to_bf16(v)) << 16) : v;
}

// ------------------------------------------------------------------ SIMT path

constexpr int kSimtThreads = 256;
constexpr int kSimtQ = 8192;  // floats of queries staged in LDS per pass

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// Row of key 0 of the range holding key s0 of batch row b, so that key s of the range
// sits at row base + s: the sequence's rows, or (paged keys) the page holding s0, whose
// table entry is read only when the range has keys (pages past the sequence may be
// unassigned).  Ranges never cross a page (the launches cap them at the page size).
__device__ __forceinline__ int64_t key_range_base(const IndexLaunch& a, int64_t b, int64_t s0, bool has_keys) {
  if (!a.kmap.table) return b * a.kI_rows;
  if (!has_keys) return 0;
  return paged_row(a.kmap, b, s0) - s0;
}

// row of key s (per key; the SIMT kernels)
__device__ __forceinline__ int64_t key_row(const IndexLaunch& a, int64_t b, int64_t s) {
  return a.kmap.table ? paged_row(a.kmap, b, s) : b * a.kI_rows + s;
}

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
  const T* k = static_cast<const T*>(a.kI.data) + key_row(a, b, s < vis ? s : 0) * a.DI;
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
  if (s < a.N) a.scores[bt * a.N + s] = s < vis ? stored_score(a, score) : -INFINITY;
}

// MXFP4 keys and queries: dequantized element d of row r (codes [., DI/2], scales [., DI/32])
__device__ __forceinline__ float mx_elem(const uint8_t* codes, const uint8_t* scales, int64_t r, int DI, int d) {
  const uint8_t c = codes[r * (DI / 2) + d / 2];
  const int code = (d & 1) ? (c >> 4) : (c & 15);
  return ldexpf(e2m1_to_f32(code), static_cast<int>(scales[r * (DI / 32) + d / 32]) - 127);
}

__global__ __launch_bounds__(kSimtThreads) void index_simt_mxfp4_kernel(IndexLaunch a) {
  __shared__ float qs[kSimtQ];
  __shared__ float ws[128];
  const int64_t bt = blockIdx.y;
  const int64_t b = bt / a.Tq;
  const int64_t s = static_cast<int64_t>(blockIdx.x) * kSimtThreads + threadIdx.x;
  const int64_t pos = a.q_pos[bt];
  int64_t vis = pos / a.ratio;
  if (vis > a.N) vis = a.N;
  if (vis < 0) vis = 0;
  const uint8_t* qc = static_cast<const uint8_t*>(a.qI.data);
  const uint8_t* qsc = static_cast<const uint8_t*>(a.qI.scale);
  const uint8_t* kc = static_cast<const uint8_t*>(a.kI.data);
  const uint8_t* ksc = static_cast<const uint8_t*>(a.kI.scale);
  const int64_t krow = vis > 0 ? key_row(a, b, s < vis ? s : 0) : 0;
  for (int h = threadIdx.x; h < a.HI; h += kSimtThreads) ws[h] = a.wI[bt * a.HI + h];
  const int hc = kSimtQ / a.DI;
  float score = 0.f;
  for (int h0 = 0; h0 < a.HI; h0 += hc) {
    const int nh = min(hc, a.HI - h0);
    __syncthreads();
    for (int i = threadIdx.x; i < nh * a.DI; i += kSimtThreads)
      qs[i] = mx_elem(qc, qsc, bt * a.HI + h0 + i / a.DI, a.DI, i % a.DI);
    __syncthreads();
    if (s < vis) {
      for (int h = 0; h < nh; ++h) {
        float dot = 0.f;
        for (int d = 0; d < a.DI; ++d) dot = fmaf(qs[h * a.DI + d], mx_elem(kc, ksc, krow, a.DI, d), dot);
        score = fmaf(ws[h0 + h], fmaxf(dot, 0.f), score);
      }
    }
  }
  if (s < a.N) a.scores[bt * a.N + s] = s < vis ? stored_score(a, score) : -INFINITY;
}

// ------------------------------------------------------------------ MFMA path

constexpr int kWavesPerWG = 4;
constexpr int kSelKeysPerWave = 256;  // entries per wave of the selecting stream kernel
constexpr int kSelWaves = 8;          // waves per workgroup of the selecting stream kernel
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

  const uint16_t* kbase =
      static_cast<const uint16_t*>(a.kI.data) + key_range_base(a, b, s_begin, s_begin < vis_end) * a.DI;
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
          for (int r = 0; r < 4; ++r) sc = fmaf(w[hb][r], relu_bits(acc[r]), sc);
        }
        // sum the four row groups (heads) holding the same entry
        sc = rows4_sum(sc);
        part[tI] = sc;
      }
#pragma unroll
      for (int tI = 0; tI < kTiles; ++tI)
        if (grp == tI) res = part[tI];
      if (s0 + lane >= vis_end) res = -INFINITY;
    }
    const int64_t s = s0 + lane;
    if (s < s_end) out[s] = stored_score(a, res);
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


// Streaming variant of the same work split (one wave per token and entry range, no
// key sharing between waves): loading a 16-entry B operand straight from HBM reads
// 64 bytes from each of 16 rows per instruction, which streams measurably slower than
// whole contiguous KiBs.  Here each wave instead copies its rows into a private LDS
// ring of NST stages (16 TPS entries each) with direct global->LDS loads: every
// instruction fetches one contiguous KiB (RB-byte rows, the 16-byte chunks of a row
// XOR-swizzled by the entry index through the per-lane addresses), and the operand is
// read back from LDS with conflict-free 16-byte reads.  A wave only ever reads the
// stages it filled itself, so the loop has no barrier: the wave's own vmcnt orders
// its loads.  The four waves of a workgroup serve one token (the host rounds the
// waves per token up to a multiple of four), so its queries (swizzled like the keys)
// and head weights come into LDS once per workgroup, also by direct loads, ahead of
// the first key stages.
template <int STEP, int MAXL>
__device__ __forceinline__ void wait_stage(int later) {
  if constexpr (MAXL == 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= MAXL) wait_vmcnt<STEP * MAXL>();
    else wait_stage<STEP, MAXL - 1>(later);
  }
}

template <int HB, int KS, int TPS, int NST, int NWV = kWavesPerWG, bool SEL = false>
__global__ __launch_bounds__(NWV * WAVE) void index_stream_kernel(IndexLaunch a, int keys_per_wave,
                                                                  int64_t waves_per_token) {
  constexpr int DI = 32 * KS;
  constexpr int RB = 2 * DI;             // bytes per key row
  constexpr int CPR = RB / 16;           // 16-byte chunks per row
  constexpr int KPS = 16 * TPS;          // entries per stage
  constexpr int STAGE_B = KPS * RB;
  constexpr int DPS = STAGE_B / 1024;    // direct loads per stage
  static_assert(DPS >= 1 && DPS * 1024 == STAGE_B, "a stage is whole KiBs");
  static_assert(NST >= 2 && DPS * (NST - 1) < 64, "vmcnt range");
  constexpr int QOPS = HB * KS;          // KiBs of queries: HI x DI bf16
  constexpr int WOPS = (16 * HB + 63) / 64;  // head weights: 64 floats per dword load
  __shared__ __attribute__((aligned(16))) uint8_t ring[NWV][NST * STAGE_B];
  // SEL: the workgroup's slice of the score row stays in LDS and is selected there
  constexpr int SLICE = SEL ? NWV * kSelKeysPerWave : 1;
  __shared__ __attribute__((aligned(16))) float sel_sc[SLICE];
  __shared__ Shared<SEL ? NWV * WAVE : 64> sel_sh;
  __shared__ __attribute__((aligned(16))) uint8_t qsh[QOPS * 1024];
  __shared__ __attribute__((aligned(16))) float wsh[WOPS * 64];

  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // fewer than 2^32 waves and tokens (the grid is 32-bit): 32-bit index arithmetic
  const uint32_t wpt = static_cast<uint32_t>(waves_per_token);
  const uint32_t wave = blockIdx.x * NWV + static_cast<uint32_t>(wid);
  const uint32_t bt32 = __builtin_amdgcn_readfirstlane(blockIdx.x * NWV / wpt);  // the workgroup's token
  const int64_t bt = bt32;
  const int64_t b = bt32 / static_cast<uint32_t>(a.Tq);
  const int64_t s_begin = static_cast<int64_t>(wave - bt32 * wpt) * keys_per_wave;
  const int64_t s_end = min(s_begin + keys_per_wave, a.N);
  const int64_t pos = a.q_pos[bt];  // a scalar load, waited for only where vis is needed
  const int col = lane & 15;
  const int grp = lane >> 4;
  // the token's queries and head weights, split over the waves (load i by wave i % 4)
  {
    const uint8_t* q = static_cast<const uint8_t*>(a.qI.data) + uni64(bt * a.HI) * RB;
    const uint32_t q_b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(qsh));
#pragma unroll
    for (int j = 0; j < (QOPS + NWV - 1) / NWV; ++j) {
      const int i = wid + NWV * j;
      if (i >= QOPS) break;
      const int off = i * 1024 + 16 * lane;
      const int row = off / RB;
      const int lc = ((off % RB) / 16) ^ (row & (CPR - 1));
      lds_dma16(q + row * RB + lc * 16, q_b + i * 1024);
    }
    const float* wr = a.wI + uni64(bt * a.HI);
    const uint32_t w_b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(wsh));
#pragma unroll
    for (int i = 0; i < WOPS; ++i)
      if ((QOPS + i) % NWV == wid) {  // wave-uniform
        const int e = 64 * i + lane;
        lds_dma4(wr + (e < 16 * HB ? e : 0), w_b + i * 256);  // lanes past HI re-read weight 0
      }
  }
  int64_t vis = (pos >= 0 && pos <= 0xffffffffll) ? static_cast<int64_t>(static_cast<uint32_t>(pos) / static_cast<uint32_t>(a.ratio))
                                                 : pos / a.ratio;
  vis = vis > a.N ? a.N : (vis < 0 ? 0 : vis);
  const int64_t vis_end = uni64(min(s_end, vis));
  const int nst = vis_end > s_begin ? static_cast<int>((vis_end - s_begin + KPS - 1) / KPS) : 0;
  const uint8_t* kbase =
      static_cast<const uint8_t*>(a.kI.data) + uni64(key_range_base(a, b, s_begin, vis_end > s_begin)) * RB;
  const uint32_t ring_b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&ring[wid][0]));
  // stage u: entries s_begin + KPS u ..; load i covers stage bytes [1024 i, +1024)
  auto issue = [&](int u) {
    const int st = u % NST;
#pragma unroll
    for (int i = 0; i < DPS; ++i) {
      const int off = i * 1024 + 16 * lane;
      const int kk = off / RB;                // entry within the stage
      const int lc = ((off % RB) / 16) ^ (kk & (CPR - 1));  // logical chunk stored at this slot
      int64_t s = s_begin + static_cast<int64_t>(u) * KPS + kk;
      if (s >= vis_end) s = vis_end - 1;      // in bounds; masked when stored
      lds_dma16_nt(kbase + s * RB + lc * 16, ring_b + st * STAGE_B + i * 1024);
    }
  };
#pragma unroll
  for (int u = 0; u < NST - 1; ++u)
    if (u < nst) issue(u);
  // the query loads were issued before every key stage: wait for them alone
  wait_stage<DPS, NST - 1>(min(nst, NST - 1));
  __syncthreads();

  bf16x8 qa[HB][KS];
  float w[HB][4];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int row = hb * 16 + col;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qa[hb][ks] = *reinterpret_cast<const bf16x8*>(qsh + row * RB + (((4 * ks + grp) ^ (row & (CPR - 1))) * 16));
    const float4 wv = *reinterpret_cast<const float4*>(&wsh[hb * 16 + grp * 4]);
    w[hb][0] = wv.x;
    w[hb][1] = wv.y;
    w[hb][2] = wv.z;
    w[hb][3] = wv.w;
  }

  float* out = a.scores ? a.scores + bt * a.N : nullptr;
  // SEL: entry s of the row lands at sel_sc[s - s_slice] (the workgroup's first entry)
  const int64_t s_slice = SEL ? s_begin - static_cast<int64_t>(wid) * keys_per_wave : 0;
  auto put = [&](int64_t s, float v) {
    v = stored_score(a, v);
    if (SEL) sel_sc[s - s_slice] = v;
    if (out) out[s] = v;
  };
  float res = -INFINITY;
  for (int t = 0; t < nst; ++t) {
    wait_stage<DPS, NST - 2>(min(nst - 1 - t, NST - 2));
    if (t + NST - 1 < nst) issue(t + NST - 1);  // into the stage read in iteration t-1
    const uint8_t* T = &ring[wid][(t % NST) * STAGE_B];
#pragma unroll
    for (int tI = 0; tI < TPS; ++tI) {
      const int kk = tI * 16 + col;
      bf16x8 kb[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kb[ks] = *reinterpret_cast<const bf16x8*>(T + kk * RB + (((4 * ks + grp) ^ (kk & (CPR - 1))) * 16));
      float sc = 0.f;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[hb][ks], kb[ks], acc, 0, 0, 0);
#pragma unroll
        for (int r = 0; r < 4; ++r) sc = fmaf(w[hb][r], relu_bits(acc[r]), sc);
      }
      sc = rows4_sum(sc);
      // tiles are stored in runs of four: lane (col, grp) holds entry 16 grp + col of the run
      const int tile = t * TPS + tI;
      const int g = tile & 3;
      if (grp == g) res = sc;
      if (g == 3 || (t == nst - 1 && tI == TPS - 1)) {
        const int64_t s = s_begin + static_cast<int64_t>(tile - g) * 16 + lane;
        if (s < s_end) put(s, s < vis_end ? res : -INFINITY);
        res = -INFINITY;
      }
    }
  }
  // entries past the visible prefix that no run covered
  const int64_t covered = s_begin + static_cast<int64_t>((nst * TPS + 3) / 4) * 64;
  for (int64_t s = covered + lane; s < s_end; s += WAVE) put(s, -INFINITY);
  if constexpr (SEL) {
    // ---- the slice's top-k as (score, entry) candidates in entry order: thread t holds
    // entries t, t + NT, ... of the slice (entries past the row are -inf)
    constexpr int NT = NWV * WAVE;
    constexpr int PER = SLICE / NT;
    __syncthreads();
    const int64_t n_here = a.N - s_slice;
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int e = j * NT + static_cast<int>(threadIdx.x);
      const float x = e < n_here ? sel_sc[e] : -INFINITY;
      v[j] = __builtin_isfinite(x) ? x : -INFINITY;
    }
    TopkArgs t{};
    t.n_in = a.N;
    t.slice = SLICE;
    t.slices = static_cast<int>((a.N + SLICE - 1) / SLICE);
    t.k = a.sel_k;
    t.out_val = a.sel_val;
    t.out_idx = a.sel_idx;
    select_slice<NT, PER, false, false>(t, sel_sh, bt * t.slices + s_slice / SLICE, v);
  }
}

// ------------------------------------------------------------------ prefill (LDS-shared keys)

constexpr int kPfWaves = 8;
constexpr int kPfTokPerWave = 2;
constexpr int kPfTok = kPfWaves * kPfTokPerWave;  // queries per workgroup
constexpr int kPfKeys = 128;                  // keys per ring stage
constexpr int kPfStages = 4;

// HB head blocks of 16, KS k-steps of 32 (DI = 32 KS).  Grid: (sequence, query group,
// key range of keys_per_wg) flattened.
template <int HB, int KS>
__global__ __launch_bounds__(kPfWaves * WAVE) void index_prefill_kernel(IndexLaunch a, int64_t keys_per_wg,
                                                                         int64_t ranges, int64_t groups) {
  constexpr int DI = 32 * KS;
  constexpr int RB = 2 * DI;                 // bytes per key row
  constexpr int CPR = RB / 16;               // 16-byte chunks per row
  constexpr int STAGE_B = kPfKeys * RB;      // bytes per stage
  constexpr int DMA_PER_WAVE = STAGE_B / 1024 / kPfWaves;
  static_assert(DMA_PER_WAVE >= 1 && DMA_PER_WAVE * kPfWaves * 1024 == STAGE_B, "stage must split into waves");
  static_assert(DMA_PER_WAVE * (kPfStages - 2) < 64, "vmcnt range");
  constexpr int NSUB = kPfKeys / 64;         // 64-key groups per stage
  __shared__ __attribute__((aligned(16))) uint8_t ring[kPfStages * STAGE_B];
  __shared__ int64_t vis_w[kPfWaves];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t kr = blockIdx.x % ranges;
  const int64_t tg = blockIdx.x / ranges;
  const int64_t b = tg / groups;
  const int64_t tq0 = (tg % groups) * kPfTok;
  const int64_t s_begin = kr * keys_per_wg;
  const int64_t s_end = min(s_begin + keys_per_wg, a.N);

  // this wave's two queries: q^I (A operand, rows = heads) and head weights
  bf16x8 qa[kPfTokPerWave][HB][KS];
  float w[kPfTokPerWave][HB][4];
  int64_t vis[kPfTokPerWave];
  int64_t vmax = 0;
#pragma unroll
  for (int u = 0; u < kPfTokPerWave; ++u) {
    const int64_t tq = tq0 + wid * kPfTokPerWave + u;
    vis[u] = 0;
    if (tq < a.Tq) {
      const int64_t bt = b * a.Tq + tq;
      int64_t v = a.q_pos[bt] / a.ratio;
      vis[u] = v > a.N ? a.N : (v < 0 ? 0 : v);
      const uint16_t* q = static_cast<const uint16_t*>(a.qI.data) + bt * a.HI * DI;
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          qa[u][hb][ks] = *reinterpret_cast<const bf16x8*>(q + (hb * 16 + col) * DI + ks * 32 + grp * 8);
#pragma unroll
        for (int r = 0; r < 4; ++r) w[u][hb][r] = a.wI[bt * a.HI + hb * 16 + grp * 4 + r];
      }
    } else {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qa[u][hb][ks] = bf16x8{};
#pragma unroll
        for (int r = 0; r < 4; ++r) w[u][hb][r] = 0.f;
      }
    }
    vmax = max(vmax, vis[u]);
  }
  if (lane == 0) vis_w[wid] = vmax;
  // every load the compiler tracks completes before the first row load it cannot see
#pragma unroll
  for (int u = 0; u < kPfTokPerWave; ++u)
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 t = __builtin_bit_cast(uint4, qa[u][hb][ks]);
        asm volatile("" ::"v"(t.x), "v"(t.y), "v"(t.z), "v"(t.w));
      }
  wait_vmcnt<0>();
  __syncthreads();
  int64_t wg_vis = 0;
#pragma unroll
  for (int i = 0; i < kPfWaves; ++i) wg_vis = max(wg_vis, vis_w[i]);
  // keys the workgroup has to score: [s_begin, s_stop); the rest of the range is -inf
  const int64_t s_stop = uni64(min(s_end, max(s_begin, wg_vis)));
  const int ntiles = static_cast<int>((s_stop - s_begin + kPfKeys - 1) / kPfKeys);
  const uint8_t* kbase = static_cast<const uint8_t*>(a.kI.data) + uni64(b * a.kI_rows) * RB;
  const uint32_t ring_b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));

  // stage u: keys s_begin + kPfKeys u ..; instruction m covers stage bytes [1024 m, +1024)
  auto issue = [&](int u) {
    const int st = u % kPfStages;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
      const int m = wid * DMA_PER_WAVE + i;
      const int off = m * 1024 + 16 * lane;     // byte within the stage
      const int kk = off / RB;                  // key within the stage
      const int pc = (off % RB) / 16;           // physical chunk
      const int lc = pc ^ (kk & (CPR - 1));     // logical chunk stored there
      int64_t s = s_begin + static_cast<int64_t>(u) * kPfKeys + kk;
      if (s >= s_stop) s = s_stop - 1;          // in bounds; masked when scored
      lds_dma16(kbase + s * RB + lc * 16, ring_b + st * STAGE_B + m * 1024);
    }
  };

  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  if (ntiles > 2) issue(2);

  float* out[kPfTokPerWave];
#pragma unroll
  for (int u = 0; u < kPfTokPerWave; ++u) {
    const int64_t tq = tq0 + wid * kPfTokPerWave + u;
    out[u] = tq < a.Tq ? a.scores + (b * a.Tq + tq) * a.N : nullptr;
  }

  for (int t = 0; t < ntiles; ++t) {
    const int st = t % kPfStages;
    const int later = min(ntiles - 1 - t, kPfStages - 2);
    if (later >= 2) wait_vmcnt<2 * DMA_PER_WAVE>();
    else if (later == 1) wait_vmcnt<DMA_PER_WAVE>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (t + kPfStages - 1 < ntiles) issue(t + kPfStages - 1);  // into the stage freed by tile t-1

#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const uint8_t* T = ring + st * STAGE_B + sub * 64 * RB;
      const int64_t s0 = s_begin + static_cast<int64_t>(t) * kPfKeys + sub * 64;
      float part[kPfTokPerWave][4];
#pragma unroll
      for (int tI = 0; tI < 4; ++tI) {
        const int kk = tI * 16 + col;  // key within the 64-key group (swizzle uses kk mod CPR)
        bf16x8 kb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kb[ks] = *reinterpret_cast<const bf16x8*>(T + kk * RB + (((4 * ks + grp) ^ (kk & (CPR - 1))) * 16));
#pragma unroll
        for (int u = 0; u < kPfTokPerWave; ++u) {
          float sc = 0.f;
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[u][hb][ks], kb[ks], acc, 0, 0, 0);
#pragma unroll
            for (int r = 0; r < 4; ++r) sc = fmaf(w[u][hb][r], relu_bits(acc[r]), sc);
          }
          sc = rows4_sum(sc);
          part[u][tI] = sc;
        }
      }
      // lane (col, grp) stores entry s0 + 16 grp + col of each query
#pragma unroll
      for (int u = 0; u < kPfTokPerWave; ++u) {
        float res = part[u][0];
#pragma unroll
        for (int tI = 1; tI < 4; ++tI)
          if (grp == tI) res = part[u][tI];
        const int64_t s = s0 + lane;
        if (out[u] && s < s_end) out[u][s] = s < vis[u] ? stored_score(a, res) : -INFINITY;
      }
    }
  }
  // entries of the range past every query's visible prefix
  for (int64_t s = s_begin + static_cast<int64_t>(ntiles) * kPfKeys + lane; s < s_end; s += WAVE) {
#pragma unroll
    for (int u = 0; u < kPfTokPerWave; ++u)
      if (out[u]) out[u][s] = -INFINITY;
  }
}

typedef void (*PrefillKern)(IndexLaunch, int64_t, int64_t, int64_t);

PrefillKern pick_prefill(int HB, int KS) {
  if (KS == 4 && HB == 4) return index_prefill_kernel<4, 4>;
  if (KS == 4 && HB == 2) return index_prefill_kernel<2, 4>;
  if (KS == 4 && HB == 1) return index_prefill_kernel<1, 4>;
  if (KS == 2 && HB == 4) return index_prefill_kernel<4, 2>;
  if (KS == 2 && HB == 2) return index_prefill_kernel<2, 2>;
  if (KS == 2 && HB == 1) return index_prefill_kernel<1, 2>;
  return nullptr;
}

// MXFP4 scores: HB head blocks of 16, KS4 steps of 128 elements (DI = 128 KS4).  One
// wave per token and key range, as index_mfma_kernel.
template <int HB, int KS4>
__global__ __launch_bounds__(kWavesPerWG * WAVE) void index_mxfp4_kernel(IndexLaunch a, int keys_per_wave,
                                                                          int64_t waves_per_token) {
  constexpr int DI = 128 * KS4;
  const int lane = threadIdx.x & 63;
  // fewer than 2^32 waves and tokens (the grid is 32-bit): 32-bit index arithmetic
  const uint32_t wpt = static_cast<uint32_t>(waves_per_token);
  const uint32_t wave = __builtin_amdgcn_readfirstlane(blockIdx.x * kWavesPerWG + (threadIdx.x >> 6));
  if (wave >= static_cast<uint64_t>(a.B * a.Tq) * wpt) return;
  const uint32_t bt32 = wave / wpt;
  const int64_t bt = bt32;
  const int64_t b = bt32 / static_cast<uint32_t>(a.Tq);
  const int64_t s_begin = static_cast<int64_t>(wave - bt32 * wpt) * keys_per_wave;
  const int64_t s_end = min(s_begin + keys_per_wave, a.N);
  const int64_t pos = a.q_pos[bt];
  int64_t vis = (pos >= 0 && pos <= 0xffffffffll) ? static_cast<int64_t>(static_cast<uint32_t>(pos) / static_cast<uint32_t>(a.ratio))
                                                 : pos / a.ratio;
  vis = vis > a.N ? a.N : (vis < 0 ? 0 : vis);
  const int col = lane & 15;
  const int grp = lane >> 4;
  float* out = a.scores + bt * a.N;
  const int64_t vis_end = min(s_end, vis);

  // queries: A operand (rows = heads), codes and block scale per lane
  v8i32 qa[HB][KS4];
  int qsc[HB][KS4];
  float w[HB][4];
  if (s_begin < vis_end) {
    const uint8_t* qc = static_cast<const uint8_t*>(a.qI.data) + bt * a.HI * (DI / 2);
    const uint8_t* qs = static_cast<const uint8_t*>(a.qI.scale) + bt * a.HI * (DI / 32);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int h = hb * 16 + col;
#pragma unroll
      for (int ks = 0; ks < KS4; ++ks) {
        const uint4 v = *reinterpret_cast<const uint4*>(qc + h * (DI / 2) + ks * 64 + grp * 16);
        qa[hb][ks] = v8i32{static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z),
                           static_cast<int>(v.w), 0, 0, 0, 0};
        qsc[hb][ks] = qs[h * (DI / 32) + ks * 4 + grp];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) w[hb][r] = a.wI[bt * a.HI + hb * 16 + grp * 4 + r];
    }
  }

  const int64_t krow0 = key_range_base(a, b, s_begin, s_begin < vis_end);
  const uint8_t* kc = static_cast<const uint8_t*>(a.kI.data) + krow0 * (DI / 2);
  const uint8_t* ksp = static_cast<const uint8_t*>(a.kI.scale) + krow0 * (DI / 32);
  // keys of 64 entries starting at s0: codes (B operand) and the 4 block scales per step
  auto load = [&](uint4 (&kb)[kTiles][KS4], uint32_t (&ks4)[kTiles][KS4], int64_t s0) {
#pragma unroll
    for (int tI = 0; tI < kTiles; ++tI) {
      int64_t s = s0 + tI * 16 + col;
      if (s >= vis_end) s = vis_end - 1;  // clamp: in bounds, masked below
#pragma unroll
      for (int ks = 0; ks < KS4; ++ks) {
        kb[tI][ks] = load_stream16(kc + s * (DI / 2) + ks * 64 + grp * 16);
        ks4[tI][ks] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(ksp + s * (DI / 32) + ks * 4));
      }
    }
  };
  auto score = [&](const uint4 (&kb)[kTiles][KS4], const uint32_t (&ks4)[kTiles][KS4], int64_t s0) {
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
          for (int ks = 0; ks < KS4; ++ks) {
            const uint4 v = kb[tI][ks];
            const v8i32 bop = {static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z),
                               static_cast<int>(v.w), 0, 0, 0, 0};
            const int kscale = static_cast<int>((ks4[tI][ks] >> (8 * grp)) & 0xffu);
            acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[hb][ks], bop, acc, 4, 4, 0, qsc[hb][ks], 0,
                                                                    kscale);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) sc = fmaf(w[hb][r], relu_bits(acc[r]), sc);
        }
        sc = rows4_sum(sc);
        part[tI] = sc;
      }
#pragma unroll
      for (int tI = 0; tI < kTiles; ++tI)
        if (grp == tI) res = part[tI];
      if (s0 + lane >= vis_end) res = -INFINITY;
    }
    const int64_t s = s0 + lane;
    if (s < s_end) out[s] = stored_score(a, res);
  };

  constexpr int64_t kStep = 16 * kTiles;
  uint4 kA[kTiles][KS4], kB[kTiles][KS4];
  uint32_t sA[kTiles][KS4], sB[kTiles][KS4];
  int64_t s0 = s_begin;
  if (s0 < vis_end) load(kA, sA, s0);
  for (; s0 < s_end; s0 += 2 * kStep) {
    if (s0 + kStep < vis_end) load(kB, sB, s0 + kStep);
    score(kA, sA, s0);
    if (s0 + kStep >= s_end) break;
    if (s0 + 2 * kStep < vis_end) load(kA, sA, s0 + 2 * kStep);
    score(kB, sB, s0 + kStep);
  }
}

typedef void (*MfmaKern)(IndexLaunch, int, int64_t);

constexpr int kMxfp4Kpw = 512;  // smallest key range per wave of the MXFP4 kernel

MfmaKern pick_mxfp4(int HB, int KS4) {
#define CSA_MX(H_, K_) \
  if (HB == H_ && KS4 == K_) return index_mxfp4_kernel<H_, K_>;
  CSA_MX(1, 1) CSA_MX(2, 1) CSA_MX(4, 1) CSA_MX(8, 1) CSA_MX(1, 2) CSA_MX(2, 2) CSA_MX(4, 2)
#undef CSA_MX
  return nullptr;
}

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

constexpr int kStreamTPS = 1;  // 16-entry tiles per ring stage
constexpr int kStreamNST = 3;  // ring stages per wave (two workgroups of 64 KiB share a CU)

template <int HB>
MfmaKern pick_stream_ks(int KS) {
  switch (KS) {
    case 1: return index_stream_kernel<HB, 1, kStreamTPS, kStreamNST>;
    case 2: return index_stream_kernel<HB, 2, kStreamTPS, kStreamNST>;
    case 4: return index_stream_kernel<HB, 4, kStreamTPS, kStreamNST>;
  }
  return nullptr;  // longer rows: the direct-load kernel
}

MfmaKern pick_stream(int HB, int KS) {
  switch (HB) {
    case 1: return pick_stream_ks<1>(KS);
    case 2: return pick_stream_ks<2>(KS);
    case 4: return pick_stream_ks<4>(KS);
    case 8: return pick_stream_ks<8>(KS);
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

// The selecting stream kernel: bf16 queries and keys with 16-head blocks and DI of 32,
// 64 or 128, few queries per sequence (the decode shape), and every row's candidates
// (slices x k) within one final workgroup's capacity.
int index_select_slices(const IndexLaunch& L) {
  if (L.qI.dtype != CSA_BF16 || L.HI % 16 != 0 || L.HI > 128 || L.Tq >= kPfTok || L.N <= 0) return 0;
  if (L.DI != 32 && L.DI != 64 && L.DI != 128) return 0;
  if (L.sel_k < 1 || L.sel_k > 4096) return 0;
  constexpr int64_t slice = static_cast<int64_t>(kSelWaves) * kSelKeysPerWave;
  const int64_t slices = (L.N + slice - 1) / slice;
  if (slices * L.sel_k > 32768) return 0;
  // Selecting while scoring pays only when the slices shed most of the row: the fused
  // kernel runs one 8-wave workgroup per CU (its prologue and selection are not hidden
  // behind other workgroups' streaming) and the merge of the candidate lists costs about
  // as much as a one-level selection of the whole row.  Measured on the 128K decode
  // shape (k = 1024: half of every slice kept) the two-kernel path is faster.
  if (slices * L.sel_k * 8 > L.N) return 0;
  if (L.B * L.Tq * slices * kSelWaves >= (int64_t{1} << 32)) return 0;
  return static_cast<int>(slices);
}

int launch_index_select(const IndexLaunch& L, hipStream_t stream) {
  if (L.B * L.Tq == 0) return 0;
  const int slices = index_select_slices(L);
  if (slices == 0) return 1;
  const int64_t grid = L.B * L.Tq * slices;
  const int64_t wpt = static_cast<int64_t>(slices) * kSelWaves;
  const dim3 g(static_cast<uint32_t>(grid)), blk(kSelWaves * WAVE);
#define CSA_SEL(HB_, KS_)                                                                                          \
  if (L.HI / 16 == HB_ && L.DI / 32 == KS_) {                                                                       \
    hipLaunchKernelGGL((index_stream_kernel<HB_, KS_, kStreamTPS, kStreamNST, kSelWaves, true>), g, blk, 0, stream, \
                       L, kSelKeysPerWave, wpt);                                                                   \
    return hipGetLastError() == hipSuccess ? 0 : -1;                                                               \
  }
  CSA_SEL(1, 1) CSA_SEL(1, 2) CSA_SEL(1, 4) CSA_SEL(2, 1) CSA_SEL(2, 2) CSA_SEL(2, 4)
  CSA_SEL(4, 1) CSA_SEL(4, 2) CSA_SEL(4, 4) CSA_SEL(8, 1) CSA_SEL(8, 2) CSA_SEL(8, 4)
#undef CSA_SEL
  return 1;
}

int launch_index_scores(const IndexLaunch& L, hipStream_t stream) {
  if (L.B == 0 || L.Tq == 0 || L.N == 0) return 0;
  if (L.qI.dtype == CSA_MXFP4) {
    MfmaKern k = (L.HI % 16 == 0 && L.DI % 128 == 0) ? pick_mxfp4(L.HI / 16, L.DI / 128) : nullptr;
    if (k) {
      // MXFP4 keys are 68 bytes (DI = 128): longer ranges per wave for the same bytes
      const int64_t tokens = L.B * L.Tq;
      int kpw = kMxfp4Kpw;
      while (kpw < 8192 && tokens * ((L.N + kpw - 1) / kpw) > 8192) kpw *= 2;
      if (L.kmap.table) {
        if ((1 << L.kmap.shift) < kMxfp4Kpw) return -2;
        kpw = std::min(kpw, 1 << L.kmap.shift);  // a range stays inside one page
      }
      const int64_t wpt = (L.N + kpw - 1) / kpw;
      const int64_t grid = (tokens * wpt + kWavesPerWG - 1) / kWavesPerWG;
      if (tokens * wpt >= (int64_t{1} << 32)) return -1;  // beyond the kernel's 32-bit wave index
      hipLaunchKernelGGL(k, dim3(static_cast<uint32_t>(grid)), dim3(kWavesPerWG * WAVE), 0, stream, L, kpw, wpt);
    } else {
      dim3 grid(static_cast<uint32_t>((L.N + kSimtThreads - 1) / kSimtThreads), static_cast<uint32_t>(L.B * L.Tq));
      hipLaunchKernelGGL(index_simt_mxfp4_kernel, grid, dim3(kSimtThreads), 0, stream, L);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  if (L.kmap.table && (L.kmap.shift < 0 || (1 << L.kmap.shift) < index_min_page_entries)) return -2;
  if (L.qI.dtype == CSA_BF16 && L.HI % 16 == 0 && L.DI % 32 == 0 && L.Tq >= kPfTok) {
    if (L.kmap.table) return -2;  // the prefill kernel reads contiguous keys only
    // many queries per sequence: keys staged once in LDS for kPfTok queries at a time
    PrefillKern k = pick_prefill(L.HI / 16, L.DI / 32);
    if (k) {
      const int64_t groups = (L.Tq + kPfTok - 1) / kPfTok;
      int64_t kpw = 8192;
      while (kpw > kPfKeys && L.B * groups * ((L.N + kpw - 1) / kpw) < 1024) kpw /= 2;
      const int64_t ranges = (L.N + kpw - 1) / kpw;
      const int64_t grid = L.B * groups * ranges;
      hipLaunchKernelGGL(k, dim3(static_cast<uint32_t>(grid)), dim3(kPfWaves * WAVE), 0, stream, L, kpw, ranges,
                         groups);
      return hipGetLastError() == hipSuccess ? 0 : -1;
    }
  }
  if (L.qI.dtype == CSA_BF16 && L.HI % 16 == 0 && L.DI % 32 == 0) {
    MfmaKern k = pick_stream(L.HI / 16, L.DI / 32);
    const bool streamed = k != nullptr;
    if (!k) k = pick_mfma(L.HI / 16, L.DI / 32);
    if (k) {
      // entries per wave: small ranges when there are few tokens (decode) so that the
      // whole chip streams the keys; longer ranges amortise the query load otherwise
      const int64_t tokens = L.B * L.Tq;
      int kpw = 128;
      while (kpw < 4096 && tokens * ((L.N + kpw - 1) / kpw) > 8192) kpw *= 2;
      if (L.kmap.table) kpw = std::min(kpw, 1 << L.kmap.shift);  // a range stays inside one page
      int64_t wpt = (L.N + kpw - 1) / kpw;
      if (streamed) {
        wpt = (wpt + kWavesPerWG - 1) / kWavesPerWG * kWavesPerWG;  // one token per workgroup
        if (tokens * wpt >= (int64_t{1} << 32)) {  // its index arithmetic is 32-bit
          k = pick_mfma(L.HI / 16, L.DI / 32);
          wpt = (L.N + kpw - 1) / kpw;
          if (!k) return -1;
        }
      }
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
