// K1: softmax-weighted KV compression (CSA overlap / HCA block) and the fp32 ->
// storage-format quantizer.
//
// Method: [V4-CN] "DeepSeek-V4中文翻译" §2.3.1 (CSA compression equations: the
// current block's a-branch and the previous block's b-branch, soft-maxed per
// channel across the 2m positions) and §2.3.2 (HCA: one block of m' positions, no
// overlap); partial RoPE of the entry, §2.3.3; storage formats §2.3.4 / §3.4.
//
// Design (HBM stream-and-reduce): every input row is read exactly once, a thread owns
// 8 consecutive channels of one entry, and consecutive lanes own consecutive channel
// chunks, so every wave load is a contiguous row segment.  Loaded rows stay in the
// input format in registers until the math needs them, which keeps the register count
// low enough for four or five waves per SIMD: the loads of some waves then overlap the
// arithmetic of others.  Three paths, chosen per launch:
//   - at most 8 rows per entry (CSA with ratio 4): all of a thread's rows are loaded
//     at once and each channel is reduced in one pass (max, then exp-weighted sums);
//   - long non-overlapping blocks (HCA): row groups of consecutive rows, each walked
//     in batches of 8 with a running (max, sum, weighted sum), merged in LDS in group
//     order;
//   - anything else: the general online softmax with row groups merged through LDS.
// The epilogue applies RoPE and the output format (fp32, bf16, FP8-mixed with a
// per-entry scale, MXFP4 with a per-32 scale), reducing the scale maxima with LDS
// atomics.
#include "device_common.h"
#include "launch.h"

#include <algorithm>

namespace csa {

namespace {

constexpr int kThreads = 256;
constexpr int kVec = 8;      // channels per thread
constexpr int kBatch = 8;    // rows per online-softmax batch

// The input streams are read once: nontemporal 16-byte loads (load_stream16; measured
// 2-10 % more bandwidth than plain loads for the bulk compression).

// Eight consecutive input channels as loaded: kept in the input format until the
// math needs them, so a batch of rows in flight costs 4 (bf16) or 8 (f32) registers
// per row and stream rather than 8 unpacked floats.
template <typename TIn>
struct Raw8;

template <>
struct Raw8<uint16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = load_stream16(p); }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t x = i < 2 ? w.x : (i < 4 ? w.y : (i < 6 ? w.z : w.w));
    return (i & 1) ? bf16hi(x) : bf16lo(x);
  }
};

template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    const uint4 x = load_stream16(p), y = load_stream16(p + 4);
    a = make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w));
    b = make_float4(__uint_as_float(y.x), __uint_as_float(y.y), __uint_as_float(y.z), __uint_as_float(y.w));
  }
  __device__ __forceinline__ float get(int i) const {
    switch (i) {
      case 0: return a.x;
      case 1: return a.y;
      case 2: return a.z;
      case 3: return a.w;
      case 4: return b.x;
      case 5: return b.y;
      case 6: return b.z;
      default: return b.w;
    }
  }
};

template <typename TIn>
__device__ __forceinline__ void load8(const TIn* p, float v[kVec]);

template <>
__device__ __forceinline__ void load8<float>(const float* p, float v[kVec]) {
  const uint4 a = load_stream16(p), b = load_stream16(p + 4);
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
  v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float v[kVec]) {
  const uint4 a = load_stream16(p);
  v[0] = bf16lo(a.x); v[1] = bf16hi(a.x);
  v[2] = bf16lo(a.y); v[3] = bf16hi(a.y);
  v[4] = bf16lo(a.z); v[5] = bf16hi(a.z);
  v[6] = bf16lo(a.w); v[7] = bf16hi(a.w);
}

struct OutDesc {
  void* data;
  void* rope;
  void* scale;
  int dtype;
  int D;
  int R;
};

// Store 8 channels (chunk c) of the entry at global row `row`.  `amax_slot` is an
// LDS word per entry (FP8MIX) or per 32-block (MXFP4) already holding the reduced
// maximum magnitude.  Must be called after the LDS maxima are final.
// Compressed entries are written once and not read back here: nontemporal stores
// (measured: a few percent less time than plain stores next to the 16x larger read
// stream).
__device__ __forceinline__ void store_stream16(void* p, uint4 v) {
  __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(p));
}

__device__ __forceinline__ void store_chunk(const OutDesc& o, int64_t row, int c, const float v[kVec],
                                            const uint32_t* amax_lds_entry) {
  const int d0 = c * kVec;
  switch (o.dtype) {
    case CSA_F32: {
      float* p = static_cast<float*>(o.data) + row * o.D + d0;
      store_stream16(p, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])));
      store_stream16(p + 4, make_uint4(__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]), __float_as_uint(v[7])));
      break;
    }
    case CSA_BF16: {
      uint16_t* p = static_cast<uint16_t*>(o.data) + row * o.D + d0;
      store_stream16(p, make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                                   pack_bf16x2(v[6], v[7])));
      break;
    }
    case CSA_FP8MIX: {
      const int nope = o.D - o.R;
      if (d0 >= nope) {
        uint16_t* p = static_cast<uint16_t*>(o.rope) + row * o.R + (d0 - nope);
        *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                  pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
      } else {
        float amax = __uint_as_float(amax_lds_entry[0]);
        float s = amax > 0.f ? amax / 448.0f : 1.0f;
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) lo |= f32_to_e4m3(v[i] / s) << (8 * i);
#pragma unroll
        for (int i = 0; i < 4; ++i) hi |= f32_to_e4m3(v[4 + i] / s) << (8 * i);
        uint8_t* p = static_cast<uint8_t*>(o.data) + row * nope + d0;
        *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
        if (c == 0) static_cast<float*>(o.scale)[row] = s;
      }
      break;
    }
    case CSA_MXFP4: {
      const int blk = d0 / 32;
      float amax = __uint_as_float(amax_lds_entry[blk]);
      int X = -127;
      if (amax > 0.f) X = ilogbf(amax) - 2;
      X = X < -127 ? -127 : (X > 127 ? 127 : X);
      uint32_t packed = 0;
#pragma unroll
      for (int i = 0; i < kVec; ++i) packed |= f32_to_e2m1(ldexpf(v[i], -X)) << (4 * i);
      uint8_t* p = static_cast<uint8_t*>(o.data) + row * (o.D / 2) + d0 / 2;
      *reinterpret_cast<uint32_t*>(p) = packed;
      if ((d0 & 31) == 0) static_cast<uint8_t*>(o.scale)[row * (o.D / 32) + blk] = static_cast<uint8_t>(X + 127);
      break;
    }
  }
}

// Contribute this chunk's magnitudes to the LDS maxima used by the quantized formats.
__device__ __forceinline__ void amax_chunk(const OutDesc& o, int c, const float v[kVec],
                                           uint32_t* amax_lds_entry) {
  const int d0 = c * kVec;
  if (o.dtype == CSA_FP8MIX) {
    if (d0 >= o.D - o.R) return;
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < kVec; ++i) m = fmaxf(m, fabsf(v[i]));
    atomicMax(&amax_lds_entry[0], __float_as_uint(m));
  } else if (o.dtype == CSA_MXFP4) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < kVec; ++i) m = fmaxf(m, fabsf(v[i]));
    atomicMax(&amax_lds_entry[d0 / 32], __float_as_uint(m));
  }
}

__device__ __forceinline__ int amax_words(int dtype, int D) {
  return dtype == CSA_MXFP4 ? D / 32 : 1;
}

// Kept small: the short-lived workgroups of the compression paths each read their
// arguments, and a larger argument block measurably slows the bulk launches.
struct CompressArgs {
  const void* ca;
  const void* cb;
  const void* za;
  const void* zb;
  const float* bias_a;
  const float* bias_b;
  const void* prev_cb;
  const void* prev_zb;
  int64_t B, T, t0, out_rows, pos_offset;
  int D, ratio, overlap, R;
  int chunks, G, entries_per_wg;
  int mode;  // kModeGeneral, kModeSmall or kModeGroups
  double log2_base;
  OutDesc out;
  const float* norm_w;  // RMSNorm weight [D] of the entries, or NULL
  float norm_eps;
};

constexpr int kModeGeneral = 0;  // online softmax in batches of kBatch rows, 256 threads
constexpr int kModeSmall = 1;    // at most kBatch rows per entry, 256 threads
constexpr int kModeGroups = 2;   // no overlap, ratio a multiple of kBatch, row groups

// Entry epilogue, shared by both compression paths: the entry's RMSNorm when a weight
// is given ([V4-CN] §2.3.3: the KV entries are normalized before core attention; the
// owners' partial sums of squares meet in LDS and each owner adds them in chunk order,
// so the result does not depend on scheduling), partial RoPE of the owner's chunk at
// position pos_offset + ratio * I (angles per revolution from theta_tab when the caller
// staged them, else computed here), the scale maxima of the quantized formats, then
// the store.  Every thread of the workgroup calls it (it holds barriers).
__device__ __forceinline__ void finish_entry(const CompressArgs& a, bool owner, int64_t b, int64_t I, int c,
                                             float val[kVec], uint32_t* amax_entry, float* ss_entry,
                                             const double* theta_tab = nullptr, int64_t out_row = -1) {
  if (a.norm_w) {  // uniform in the workgroup (one job per workgroup)
    if (owner) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < kVec; ++i) ss = fmaf(val[i], val[i], ss);
      ss_entry[c] = ss;
    }
    __syncthreads();
    if (owner) {
      float tot = 0.f;
      for (int j = 0; j < a.chunks; ++j) tot += ss_entry[j];
      const float inv = 1.0f / sqrtf(tot / static_cast<float>(a.D) + a.norm_eps);
      const float4 w0 = reinterpret_cast<const float4*>(a.norm_w + c * kVec)[0];
      const float4 w1 = reinterpret_cast<const float4*>(a.norm_w + c * kVec)[1];
      const float w[kVec] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < kVec; ++i) val[i] = val[i] * inv * w[i];
    }
  }
  if (owner) {
    const int d0 = c * kVec;
    const int nope = a.D - a.R;
    if (a.R > 0 && d0 + kVec > nope) {
      const double pos = static_cast<double>(a.pos_offset + I * a.ratio);
#pragma unroll
      for (int ch = 0; ch < kVec; ch += 2) {
        const int d = d0 + ch;
        if (d >= nope) {
          float cs, sn;
          if (theta_tab) rope_cs_rev(pos, theta_tab[(d - nope) / 2], &cs, &sn);
          else rope_cs(pos, (d - nope) / 2, a.R, a.log2_base, &cs, &sn);
          const float x0 = val[ch], x1 = val[ch + 1];
          val[ch] = x0 * cs - x1 * sn;
          val[ch + 1] = x0 * sn + x1 * cs;
        }
      }
    }
  }
  if (a.out.dtype == CSA_FP8MIX || a.out.dtype == CSA_MXFP4) {  // scales need the entry's maxima
    __syncthreads();
    if (owner) amax_chunk(a.out, c, val, amax_entry);
    __syncthreads();
  }
  if (owner) store_chunk(a.out, out_row >= 0 ? out_row : b * a.out_rows + I, c, val, amax_entry);
}

// Entries of at most kBatch rows (CSA with ratio <= 4, HCA with ratio <= 8): one thread
// per 8 channels of an entry loads all the entry's rows at once, kept in the input
// format, then reduces each channel in one pass (max, then exp-weighted sums).  No
// online rescaling and no row groups, so few registers stay live and more waves fit.
template <typename TIn>
__device__ __forceinline__ void compress_small(const CompressArgs& a, int64_t block, uint32_t* amax_lds,
                                               double* theta_lds, float* ss_lds) {
  const int tid = threadIdx.x;
  const int e_local = tid / a.chunks;
  const int c = tid % a.chunks;
  const int64_t n_entries = a.T / a.ratio;
  const int64_t e_glob = block * a.entries_per_wg + e_local;
  const bool active = e_local < a.entries_per_wg && e_glob < a.B * n_entries;
  const int aw = amax_words(a.out.dtype, a.D);
  for (int i = tid; i < a.entries_per_wg * aw && i < kThreads; i += kThreads) amax_lds[i] = 0u;

  float val[kVec];
  int64_t b = 0, I = 0;
  const int r = a.ratio;
  int nrows = 0;
  Raw8<TIn> z[kBatch], v[kBatch];
  if (active) {
    // entry counts below 2^32 take 32-bit division
    int64_t il;
    if (e_glob <= 0xffffffffll && n_entries <= 0xffffffffll) {
      const uint32_t e32 = static_cast<uint32_t>(e_glob), n32 = static_cast<uint32_t>(n_entries);
      b = e32 / n32;
      il = e32 - static_cast<uint32_t>(b) * n32;
    } else {
      b = e_glob / n_entries;
      il = e_glob % n_entries;
    }
    I = a.t0 / a.ratio + il;
    nrows = (a.overlap && I >= 1) ? 2 * r : r;  // <= kBatch
    const int d0 = c * kVec;
    const int64_t D = a.D;
    const TIn* cA = static_cast<const TIn*>(a.ca) + (b * a.T + il * r) * D + d0;
    const TIn* zA = static_cast<const TIn*>(a.za) + (b * a.T + il * r) * D + d0;
    const TIn* cB = cA;
    const TIn* zB = zA;
    if (a.overlap) {
      cB = il >= 1 ? static_cast<const TIn*>(a.cb) + (b * a.T + (il - 1) * r) * D + d0
                   : static_cast<const TIn*>(a.prev_cb) + b * r * D + d0;
      zB = il >= 1 ? static_cast<const TIn*>(a.zb) + (b * a.T + (il - 1) * r) * D + d0
                   : static_cast<const TIn*>(a.prev_zb) + b * r * D + d0;
    }
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (q < nrows) {
        const bool in_a = q < r;
        const int64_t off = static_cast<int64_t>(in_a ? q : q - r) * D;
        v[q].load((in_a ? cA : cB) + off);
        z[q].load((in_a ? zA : zB) + off);
      }
    }
  }
  // the RoPE angles (revolutions per position) once per workgroup, computed while the
  // rows are in flight
  if (a.R > 0) {
    if (tid < a.R / 2) theta_lds[tid] = rope_theta_rev(tid, a.R, a.log2_base);
    __syncthreads();
  }
  if (active) {
    constexpr float kLog2e = 1.4426950408889634f;
#pragma unroll
    for (int ch = 0; ch < kVec; ++ch) {
      float zc[kBatch];
      float bm = -INFINITY;
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        if (q < nrows) {
          zc[q] = z[q].get(ch);
          const float* bp = q < r ? a.bias_a : a.bias_b;  // bias rows: [ratio, D] per branch
          if (bp) zc[q] += bp[(q < r ? q : q - r) * a.D + c * kVec + ch];
          bm = fmaxf(bm, zc[q]);
        }
      }
      float ss = 0.f, aa = 0.f;
      if (bm != -INFINITY) {
        const float mb = -bm * kLog2e;
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          if (q < nrows) {
            const float p = __builtin_amdgcn_exp2f(fmaf(zc[q], kLog2e, mb));  // e^(z - max)
            ss += p;
            aa = fmaf(p, v[q].get(ch), aa);
          }
        }
      }
      val[ch] = __fdividef(aa, ss);
    }
  }
  finish_entry(a, active, b, I, c, val, amax_lds + e_local * aw, ss_lds + e_local * a.chunks,
               a.R > 0 ? theta_lds : nullptr);
}

// Long non-overlapping blocks (HCA, ratio a multiple of kBatch): G row groups of
// ratio / G consecutive rows.  A thread walks its group's rows of 8 channels in
// batches of kBatch (the batch's loads kept in the input format and issued together),
// reducing each batch in one pass and folding it into a running (max, sum, weighted
// sum).  The G partials of every channel meet in LDS and one thread per channel merges
// them in group order.  Small workgroups with few live registers let several
// workgroups share a CU, so one's loads overlap another's arithmetic.
template <typename TIn>
__device__ __forceinline__ void compress_groups(const CompressArgs& a, int64_t block, float* part,
                                                uint32_t* amax_lds, float* ss_lds) {
  const int tid = threadIdx.x;
  const int tpe = a.chunks * a.G;  // threads per entry
  const int e_local = tid / tpe;
  const int r_in = tid % tpe;
  const int g = r_in / a.chunks;
  const int c = r_in % a.chunks;
  const int64_t n_entries = a.T / a.ratio;
  const int64_t e_glob = block * a.entries_per_wg + e_local;
  const bool active = e_local < a.entries_per_wg && e_glob < a.B * n_entries;
  const int aw = amax_words(a.out.dtype, a.D);
  const int D = a.D;
  const int rpt = a.ratio / a.G;  // rows per thread, a multiple of kBatch
  for (int i = tid; i < a.entries_per_wg * aw && i < kThreads; i += kThreads) amax_lds[i] = 0u;

  int64_t b = 0, I = 0;
  const int d0 = c * kVec;
  // partial triples: part[((e_local * G + g) * D + d) * 3 + {max, sum, weighted sum}]
  float* my = part + (static_cast<int64_t>(e_local * a.G + g) * D + d0) * 3;
  if (active) {
    b = e_glob / n_entries;
    const int64_t il = e_glob % n_entries;
    I = a.t0 / a.ratio + il;
    const int64_t row0 = b * a.T + il * a.ratio + g * rpt;
    const TIn* cp = static_cast<const TIn*>(a.ca) + row0 * D + d0;
    const TIn* zp = static_cast<const TIn*>(a.za) + row0 * D + d0;
    float m[kVec], sm[kVec], ac[kVec];
#pragma unroll
    for (int ch = 0; ch < kVec; ++ch) { m[ch] = -INFINITY; sm[ch] = 0.f; ac[ch] = 0.f; }
    for (int k0 = 0; k0 < rpt; k0 += kBatch) {
      Raw8<TIn> z[kBatch], v[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        v[q].load(cp + static_cast<int64_t>(k0 + q) * D);
        z[q].load(zp + static_cast<int64_t>(k0 + q) * D);
      }
#pragma unroll
      for (int ch = 0; ch < kVec; ++ch) {
        float zc[kBatch];
        float bm = -INFINITY;
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          zc[q] = z[q].get(ch);
          if (a.bias_a) zc[q] += a.bias_a[(g * rpt + k0 + q) * D + d0 + ch];
          bm = fmaxf(bm, zc[q]);
        }
        const float nm = fmaxf(m[ch], bm);
        if (nm == -INFINITY) continue;  // every logit so far is -inf
        const float sc = __expf(m[ch] - nm);  // 0 while m is -inf
        float ss = sm[ch] * sc, aa = ac[ch] * sc;
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          const float p = __expf(zc[q] - nm);
          ss += p;
          aa = fmaf(p, v[q].get(ch), aa);
        }
        m[ch] = nm; sm[ch] = ss; ac[ch] = aa;
      }
    }
#pragma unroll
    for (int ch = 0; ch < kVec; ++ch) {
      my[3 * ch] = m[ch];
      my[3 * ch + 1] = sm[ch];
      my[3 * ch + 2] = ac[ch];
    }
  }
  __syncthreads();
  // merge the G groups of every channel in group order; the result overwrites group
  // 0's weighted-sum slot of that channel (only this thread reads that channel)
  const int nch = a.entries_per_wg * D;
  for (int idx = tid; idx < nch; idx += kThreads) {
    const int e = idx / D, d = idx % D;
    if (block * a.entries_per_wg + e >= a.B * n_entries) continue;
    float mm = -INFINITY, sum = 0.f, acc = 0.f;
    for (int gg = 0; gg < a.G; ++gg) {
      const float* o = part + (static_cast<int64_t>(e * a.G + gg) * D + d) * 3;
      const float om = o[0];
      const float nm = fmaxf(mm, om);
      if (nm == -INFINITY) continue;
      const float s1 = __expf(mm - nm), s2 = __expf(om - nm);
      sum = sum * s1 + o[1] * s2;
      acc = acc * s1 + o[2] * s2;
      mm = nm;
    }
    part[(static_cast<int64_t>(e * a.G) * D + d) * 3 + 2] = acc / sum;
  }
  __syncthreads();
  const bool owner = active && g == 0;
  float val[kVec];
  if (owner) {
#pragma unroll
    for (int ch = 0; ch < kVec; ++ch) val[ch] = my[3 * ch + 2];
  }
  finish_entry(a, owner, b, I, c, val, amax_lds + e_local * aw, ss_lds + e_local * a.chunks);
}

template <typename TIn>
__device__ __forceinline__ void compress_block(const CompressArgs& a, int64_t block, float* part, uint32_t* amax_lds,
                                               float* ss_lds) {

  const int tid = threadIdx.x;
  const int tpe = a.chunks * a.G;                       // threads per entry
  const int e_local = tid / tpe;
  const int r_in = tid % tpe;
  const int g = r_in / a.chunks;                         // row group
  const int c = r_in % a.chunks;                         // channel chunk
  const int64_t n_entries = a.T / a.ratio;
  const int64_t e_glob = block * a.entries_per_wg + e_local;
  const int64_t total = a.B * n_entries;
  const bool active = e_local < a.entries_per_wg && e_glob < total;
  const int aw = amax_words(a.out.dtype, a.D);

  for (int i = tid; i < a.entries_per_wg * aw && i < kThreads; i += kThreads) amax_lds[i] = 0u;

  float m[kVec], s[kVec], acc[kVec];
#pragma unroll
  for (int i = 0; i < kVec; ++i) { m[i] = -INFINITY; s[i] = 0.f; acc[i] = 0.f; }

  int64_t b = 0, il = 0, I = 0;
  if (active) {
    b = e_glob / n_entries;
    il = e_glob % n_entries;              // local entry index within this call
    I = a.t0 / a.ratio + il;              // absolute entry index
    const int r = a.ratio;
    // positions: [0, r) a-rows of block I; [r, 2r) b-rows of block I-1 (CSA, I >= 1)
    const int nrows = (a.overlap && I >= 1) ? 2 * r : r;
    const int d0 = c * kVec;
    // row pointers of the two branches: position pos < r reads row pos of the a-block
    // (rows [il r, il r + r) of ca / za), position r + j reads row j of the b-block
    // (the previous block of cb / zb, or the caller's prev_cb / prev_zb for the first
    // entry of the call)
    const int64_t D = a.D;
    const TIn* cA = static_cast<const TIn*>(a.ca) + (b * a.T + il * r) * D + d0;
    const TIn* zA = static_cast<const TIn*>(a.za) + (b * a.T + il * r) * D + d0;
    const TIn* cB = nullptr;
    const TIn* zB = nullptr;
    if (a.overlap) {
      cB = il >= 1 ? static_cast<const TIn*>(a.cb) + (b * a.T + (il - 1) * r) * D + d0
                   : static_cast<const TIn*>(a.prev_cb) + b * r * D + d0;
      zB = il >= 1 ? static_cast<const TIn*>(a.zb) + (b * a.T + (il - 1) * r) * D + d0
                   : static_cast<const TIn*>(a.prev_zb) + b * r * D + d0;
    }

    for (int base = g; base < nrows; base += a.G * kBatch) {
      Raw8<TIn> z[kBatch], v[kBatch];
      int nb = 0;
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const int pos = base + q * a.G;
        if (pos < nrows) {
          nb = q + 1;
          const bool in_a = pos < r;
          const int64_t off = static_cast<int64_t>(in_a ? pos : pos - r) * D;
          const TIn* cp = (in_a ? cA : cB) + off;
          const TIn* zp = (in_a ? zA : zB) + off;
          v[q].load(cp);
          z[q].load(zp);
        }
      }
#pragma unroll
      for (int ch = 0; ch < kVec; ++ch) {
        float zc[kBatch];
        float bm = -INFINITY;
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          if (q < nb) {
            zc[q] = z[q].get(ch);
            const int pos = base + q * a.G;  // bias rows: [ratio, D] per branch
            const float* bp = pos < r ? a.bias_a : a.bias_b;
            if (bp) zc[q] += bp[(pos < r ? pos : pos - r) * a.D + d0 + ch];
            bm = fmaxf(bm, zc[q]);
          }
        }
        const float nm = fmaxf(m[ch], bm);
        if (nm == -INFINITY) continue;               // every logit so far is -inf
        const float sc = __expf(m[ch] - nm);         // 0 when m was -inf
        float ss = s[ch] * sc, aa = acc[ch] * sc;
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          if (q < nb) {
            const float p = __expf(zc[q] - nm);
            ss += p;
            aa = fmaf(p, v[q].get(ch), aa);
          }
        }
        m[ch] = nm; s[ch] = ss; acc[ch] = aa;
      }
    }
  }

  // merge row groups in fixed order
  if (a.G > 1) {
    float* my = part + tid * (2 + kVec);
    // pack: m for channel 0 only is not enough (per-channel maxima) -> store all
    // channels in three passes to keep LDS at (2+8) floats per thread
    __syncthreads();
#pragma unroll
    for (int ch = 0; ch < kVec; ++ch) {
      my[0] = m[ch]; my[1] = s[ch]; my[2 + ch] = acc[ch];
      __syncthreads();
      if (active && g == 0) {
        float mm = m[ch], sum = s[ch], ac = acc[ch];
        for (int gg = 1; gg < a.G; ++gg) {
          const float* o = part + (e_local * tpe + gg * a.chunks + c) * (2 + kVec);
          const float om = o[0];
          const float nm = fmaxf(mm, om);
          if (nm == -INFINITY) continue;
          const float s1 = __expf(mm - nm), s2 = __expf(om - nm);
          sum = sum * s1 + o[1] * s2;
          ac = ac * s1 + o[2 + ch] * s2;
          mm = nm;
        }
        m[ch] = mm; s[ch] = sum; acc[ch] = ac;
      }
      __syncthreads();
    }
  }

  float val[kVec];
  const bool owner = active && g == 0;
  if (owner) {
#pragma unroll
    for (int ch = 0; ch < kVec; ++ch) val[ch] = acc[ch] / s[ch];
  }
  finish_entry(a, owner, b, I, c, val, amax_lds + e_local * aw, ss_lds + e_local * a.chunks);
}

// One launch runs up to two compressions (the KV stream and the indexer-key stream
// of a layer): blocks [0, grid0) belong to job 0, the rest to job 1.
struct CompressArgs2 {
  CompressArgs job[2];
  int64_t grid0;
};

template <int MODE>
constexpr int mode_part_floats() {
  return MODE == kModeGroups ? kThreads * kVec * 3 : (MODE == kModeSmall ? 1 : kThreads * (2 + kVec));
}

template <typename TIn, int MODE>
__global__ __launch_bounds__(kThreads) void compress_kernel(CompressArgs2 a) {
  // LDS: row-group partials and per-entry scale maxima
  __shared__ float part[mode_part_floats<MODE>()];
  __shared__ uint32_t amax_lds[kThreads];  // entries_per_wg * amax_words <= kThreads
  __shared__ double theta_lds[MODE == kModeSmall ? 64 : 1];  // RoPE angles, R <= 128
  __shared__ float ss_lds[kThreads];  // RMSNorm partial sums, entries_per_wg * chunks <= kThreads
  const int64_t blk = blockIdx.x;
  if constexpr (MODE == kModeSmall) {
    if (blk < a.grid0) compress_small<TIn>(a.job[0], blk, amax_lds, theta_lds, ss_lds);
    else compress_small<TIn>(a.job[1], blk - a.grid0, amax_lds, theta_lds, ss_lds);
  } else if constexpr (MODE == kModeGroups) {
    if (blk < a.grid0) compress_groups<TIn>(a.job[0], blk, part, amax_lds, ss_lds);
    else compress_groups<TIn>(a.job[1], blk - a.grid0, part, amax_lds, ss_lds);
  } else {
    if (blk < a.grid0) compress_block<TIn>(a.job[0], blk, part, amax_lds, ss_lds);
    else compress_block<TIn>(a.job[1], blk - a.grid0, part, amax_lds, ss_lds);
  }
}

// ------------------------------------------------------------ decode state append

// One new token per sequence into its state-pool slot ([V4-CN] §3.6.1: the sliding
// window and the compression branch's uncompressed tail are a per-sequence state of
// fixed size; a block of ratio tokens is compressed as soon as it is complete).  One
// workgroup per batch row: the token's stream rows enter the tail ring (row p mod
// RING, RING = 2 ratio with overlap, ratio without), its raw KV row enters the window
// (rolled over to the front when the buffer is full), and when p + 1 completes a block
// the entry (KV, and with overlap the indexer key) is computed from the ring exactly as
// the bulk compressor does and stored at its pool row in the paged cache.  Thread c <
// chunks(D) owns KV channels 8c .. 8c+7 and the next chunks(DI) threads the indexer's;
// a thread reads back only rows written by earlier launches and keeps the new token's
// values in registers.
struct AppendArgs {
  CompressArgs kv;      // ca.. = the new token's rows [B, D]; out / norm / RoPE of the KV entries
  CompressArgs ik;      // the indexer keys (overlap only; ik.D = DI, no RoPE)
  int has_ik;
  const int32_t* slot;  // [B]
  int64_t* length;      // [slots]
  void* tail;           // [slots, RING, NST, D] in the stream dtype (NST = 4 with overlap, else 2)
  void* itail;          // [slots, RING, 4, DI]
  // the window's row planes (one for F32 / BF16; FP8MIX: codes, RoPE dims, scale) and
  // the token's raw KV row in the same planes ([B] rows)
  const void* raw[3];
  void* win[3];
  int plane_bytes[3];   // bytes per row of each plane (0: no plane)
  int n_win;
  int64_t Ws;
  int64_t* win_pos0;    // [slots]
  PageMap pmap;         // pool rows of the caches
  int64_t* q_pos;       // [B] out: the new token's position
  int64_t* wp0_b;       // [B] out: window base of the batch row's slot
  int64_t* wp0_adj;     // [B] out: window base such that row b * Ws + (p - base) is the slot's row
  int32_t* vis_idx;     // [B, vis_K] out (no overlap): pool rows of the visible entries, -1 after
  int64_t vis_K;
};

template <typename TIn>
__device__ __forceinline__ void raw8_store(TIn* p, const Raw8<TIn>& r);
template <>
__device__ __forceinline__ void raw8_store<float>(float* p, const Raw8<float>& r) {
  reinterpret_cast<float4*>(p)[0] = r.a;
  reinterpret_cast<float4*>(p)[1] = r.b;
}
template <>
__device__ __forceinline__ void raw8_store<uint16_t>(uint16_t* p, const Raw8<uint16_t>& r) {
  *reinterpret_cast<uint4*>(p) = r.w;
}

constexpr int kAppendBatch = 8;   // ring rows loaded together by the append kernel
constexpr int kAppendGroups = 4;  // row groups of a long block (no indexer part)

template <typename TIn>
__global__ __launch_bounds__(kThreads) void state_append_kernel(AppendArgs a) {
  __shared__ uint32_t amax_lds[2][kThreads];
  __shared__ float ss_lds[2][kThreads];
  __shared__ double theta_lds[64];  // RoPE angles, R <= 128
  __shared__ float part_lds[kThreads * 3 * kVec];  // row-group partials (max, sum, weighted sum)
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const int r = a.kv.ratio;
  const bool ov = a.kv.overlap != 0;
  const int ring = ov ? 2 * r : r;
  // KV chunks on the first waves, the indexer's from the next wave on: the part a
  // thread serves is uniform in its wave, so its arguments stay scalar.  Without an
  // indexer part the waves split a block's rows into G groups instead (HCA: 128 rows).
  const int cD = a.kv.chunks, cI = a.has_ik ? a.ik.chunks : 0;
  const int ik0 = (cD + WAVE - 1) / WAVE * WAVE;
  const int G = a.has_ik ? 1 : max(1, min(kAppendGroups, kThreads / ik0));
  const int wave = __builtin_amdgcn_readfirstlane(tid / WAVE);
  const bool kv_part = wave < G * (ik0 / WAVE);
  const int g = kv_part ? wave / (ik0 / WAVE) : 0;
  const int c = kv_part ? tid - g * ik0 : tid - ik0;
  const bool mine = kv_part ? c < cD : c < cI;
  const bool ik_part = !kv_part && mine;
  const CompressArgs& A = kv_part ? a.kv : a.ik;
  const int64_t D = A.D;
  const int d0 = c * kVec;
  const int ns = (kv_part && !ov) ? 2 : 4;  // streams in ring order: (C^a, C^b, Z^a, Z^b), or (C, Z)
  // the token's rows first: they do not depend on the slot's state
  Raw8<TIn> cur[4];
  if (mine) {
    const void* src[4] = {A.ca, ns == 4 ? A.cb : A.za, A.za, A.zb};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (q < ns) cur[q].load(static_cast<const TIn*>(src[q]) + b * D + d0);
  }
  const int64_t s = a.slot[b];
  const int64_t p = a.length[s];
  const int64_t wp0 = a.win_pos0[s];
  const bool completes = (p + 1) % r == 0;
  const int64_t I = p / r;
  const int64_t out_row = completes ? paged_row(a.pmap, b, I) : 0;
  for (int i = tid; i < 2 * kThreads; i += kThreads) (&amax_lds[0][0])[i] = 0u;
  if (a.kv.R > 0 && tid < a.kv.R / 2) theta_lds[tid] = rope_theta_rev(tid, a.kv.R, a.kv.log2_base);

  // the raw KV row into the window; a full buffer first keeps its last n_win - 1 rows.
  // Each plane moves in 16-byte pieces when its rows allow, else in dwords.
  const int64_t nwp0 = p - wp0 >= a.Ws ? p - a.n_win + 1 : wp0;
#pragma unroll
  for (int pl = 0; pl < 3; ++pl) {
    const int64_t rowb = a.plane_bytes[pl];
    if (rowb == 0) continue;
    uint8_t* wb = static_cast<uint8_t*>(a.win[pl]) + s * a.Ws * rowb;
    const uint8_t* rb = static_cast<const uint8_t*>(a.raw[pl]) + b * rowb;
    if (rowb % 16 == 0) {
      const int64_t c = rowb / 16;
      if (nwp0 != wp0) {
        for (int64_t i = tid; i < static_cast<int64_t>(a.n_win - 1) * c; i += kThreads) {
          const int64_t j = i / c, q = i % c;
          reinterpret_cast<uint4*>(wb + j * rowb)[q] = reinterpret_cast<const uint4*>(wb + (nwp0 - wp0 + j) * rowb)[q];
        }
      }
      for (int64_t i = tid; i < c; i += kThreads)
        reinterpret_cast<uint4*>(wb + (p - nwp0) * rowb)[i] = reinterpret_cast<const uint4*>(rb)[i];
    } else {
      const int64_t c = rowb / 4;
      if (nwp0 != wp0) {
        for (int64_t i = tid; i < static_cast<int64_t>(a.n_win - 1) * c; i += kThreads) {
          const int64_t j = i / c, q = i % c;
          reinterpret_cast<uint32_t*>(wb + j * rowb)[q] =
              reinterpret_cast<const uint32_t*>(wb + (nwp0 - wp0 + j) * rowb)[q];
        }
      }
      for (int64_t i = tid; i < c; i += kThreads)
        reinterpret_cast<uint32_t*>(wb + (p - nwp0) * rowb)[i] = reinterpret_cast<const uint32_t*>(rb)[i];
    }
  }
  if (a.vis_idx) {
    // every entry of a block before the token's own is visible (no overlap: dense);
    // the table entries of a batch are read before its stores
    const int64_t vis = p / r;
    const int32_t* __restrict__ tbl = a.pmap.table + s * a.pmap.max_pages;
    int32_t* __restrict__ out = a.vis_idx + b * a.vis_K;
    const int64_t mask = (int64_t{1} << a.pmap.shift) - 1;
    for (int64_t j0 = tid; j0 < a.vis_K; j0 += 8 * kThreads) {
      int32_t pg[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t j = j0 + u * kThreads;
        pg[u] = j < vis ? tbl[j >> a.pmap.shift] : -1;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t j = j0 + u * kThreads;
        if (j < a.vis_K) out[j] = j < vis ? static_cast<int32_t>((static_cast<int64_t>(pg[u]) << a.pmap.shift) | (j & mask)) : -1;
      }
    }
  }

  float val[kVec];
  float m[kVec], sum[kVec], acc[kVec];
  if (mine) {
    TIn* tl = static_cast<TIn*>(kv_part ? a.tail : a.itail) + s * ring * ns * D + d0;
    if (g == 0) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (q < ns) raw8_store<TIn>(tl + ((p % ring) * ns + q) * D, cur[q]);
    }
    if (completes) {
      // online softmax per channel over the block's rows (a-branch: block I) and, with
      // overlap, the previous block's b-branch rows, kAppendBatch rows loaded at a time;
      // the token's own row comes from registers
      const int zq_a = ns == 4 ? 2 : 1;
#pragma unroll
      for (int ch = 0; ch < kVec; ++ch) {
        m[ch] = -INFINITY;
        sum[ch] = 0.f;
        acc[ch] = 0.f;
      }
      const int all_rows = (ov && I >= 1) ? 2 * r : r;
      const int q_begin = all_rows * g / G;
      const int nrows = all_rows * (g + 1) / G;  // this group's rows: [q_begin, nrows)
      for (int q0 = q_begin; q0 < nrows; q0 += kAppendBatch) {
        Raw8<TIn> cv[kAppendBatch], zv[kAppendBatch];
        float4 bz[kAppendBatch][2];
#pragma unroll
        for (int u = 0; u < kAppendBatch; ++u) {
          const int q = q0 + u;
          if (q >= nrows) break;
          const bool in_a = q < r;
          const int j = in_a ? q : q - r;
          const int64_t pos = in_a ? I * r + j : (I - 1) * r + j;
          const int cq = in_a ? 0 : 1, zq = in_a ? zq_a : 3;
          if (pos == p) {
            cv[u] = cur[cq];
            zv[u] = cur[zq];
          } else {
            cv[u].load(tl + ((pos % ring) * ns + cq) * D);
            zv[u].load(tl + ((pos % ring) * ns + zq) * D);
          }
          const float* bp = in_a ? A.bias_a : A.bias_b;
          if (bp) {
            bz[u][0] = reinterpret_cast<const float4*>(bp + j * D + d0)[0];
            bz[u][1] = reinterpret_cast<const float4*>(bp + j * D + d0)[1];
          } else {
            bz[u][0] = bz[u][1] = make_float4(0.f, 0.f, 0.f, 0.f);
          }
        }
#pragma unroll
        for (int u = 0; u < kAppendBatch; ++u) {
          if (q0 + u >= nrows) break;
          const float bb[kVec] = {bz[u][0].x, bz[u][0].y, bz[u][0].z, bz[u][0].w,
                                  bz[u][1].x, bz[u][1].y, bz[u][1].z, bz[u][1].w};
#pragma unroll
          for (int ch = 0; ch < kVec; ++ch) {
            const float z = zv[u].get(ch) + bb[ch];
            const float nm = fmaxf(m[ch], z);
            const float sc = __expf(m[ch] - nm), pz = __expf(z - nm);
            sum[ch] = sum[ch] * sc + pz;
            acc[ch] = acc[ch] * sc + pz * cv[u].get(ch);
            m[ch] = nm;
          }
        }
      }
      if (G > 1) {
        float* pp = part_lds + (g * ik0 + c) * 3 * kVec;
#pragma unroll
        for (int ch = 0; ch < kVec; ++ch) {
          pp[3 * ch] = m[ch];
          pp[3 * ch + 1] = sum[ch];
          pp[3 * ch + 2] = acc[ch];
        }
      }
    }
  }
  __syncthreads();  // the LDS maxima are cleared, the RoPE angles and the row-group partials stored
  if (completes && mine) {
    if (kv_part && G > 1 && g == 0) {
      // the groups' partials merged in group order
#pragma unroll
      for (int ch = 0; ch < kVec; ++ch) {
        m[ch] = -INFINITY;
        sum[ch] = 0.f;
        acc[ch] = 0.f;
      }
      for (int gg = 0; gg < G; ++gg) {
        const float* pp = part_lds + (gg * ik0 + c) * 3 * kVec;
#pragma unroll
        for (int ch = 0; ch < kVec; ++ch) {
          const float om = pp[3 * ch];
          const float nm = fmaxf(m[ch], om);
          if (nm == -INFINITY) continue;
          const float s1 = __expf(m[ch] - nm), s2 = __expf(om - nm);
          sum[ch] = sum[ch] * s1 + pp[3 * ch + 1] * s2;
          acc[ch] = acc[ch] * s1 + pp[3 * ch + 2] * s2;
          m[ch] = nm;
        }
      }
    }
#pragma unroll
    for (int ch = 0; ch < kVec; ++ch) val[ch] = acc[ch] / sum[ch];
  }
  if (completes) {
    finish_entry(a.kv, kv_part && mine && g == 0, 0, I, c, val, amax_lds[0], ss_lds[0],
                 a.kv.R > 0 ? theta_lds : nullptr, out_row);
    if (a.has_ik) finish_entry(a.ik, ik_part, 0, I, c, val, amax_lds[1], ss_lds[1], nullptr, out_row);
  }
  __syncthreads();  // every thread has read length[s] and win_pos0[s]
  if (tid == 0) {
    a.length[s] = p + 1;
    a.win_pos0[s] = nwp0;
    a.q_pos[b] = p;
    a.wp0_b[b] = nwp0;
    a.wp0_adj[b] = nwp0 - (s - b) * a.Ws;
  }
}

}  // namespace

int launch_state_append(const StateAppendLaunch& L, hipStream_t stream) {
  if (L.B == 0) return 0;
  AppendArgs a{};
  CompressArgs& k = a.kv;
  k.ca = L.ca; k.cb = L.cb; k.za = L.za; k.zb = L.zb;
  k.bias_a = L.bias_a; k.bias_b = L.bias_b;
  k.D = L.D; k.ratio = L.ratio; k.overlap = L.overlap; k.R = L.rope_dims;
  k.pos_offset = L.pos_offset;
  k.log2_base = L.log2_base;
  k.out = OutDesc{L.kv_out.data, L.kv_out.rope, L.kv_out.scale, L.kv_out.dtype, L.D, L.rope_dims};
  k.norm_w = L.norm_w;
  k.norm_eps = L.norm_eps;
  k.chunks = L.D / kVec;
  a.has_ik = L.overlap && L.ica;
  if (a.has_ik) {
    CompressArgs& i = a.ik;
    i = k;
    i.ca = L.ica; i.cb = L.icb; i.za = L.iza; i.zb = L.izb;
    i.bias_a = L.ibias_a; i.bias_b = L.ibias_b;
    i.D = L.DI;
    i.R = 0;
    i.out = OutDesc{L.ik_out.data, L.ik_out.rope, L.ik_out.scale, L.ik_out.dtype, L.DI, 0};
    i.norm_w = nullptr;
    i.chunks = L.DI / kVec;
  }
  if ((k.chunks + WAVE - 1) / WAVE * WAVE + (a.has_ik ? a.ik.chunks : 0) > kThreads || L.rope_dims > 128) return -2;
  a.slot = L.slot;
  a.length = L.length;
  a.tail = L.tail;
  a.itail = L.itail;
  const int R = L.rope_dims;
  if (L.win.dtype == CSA_FP8MIX) {
    const void* raw[3] = {L.kv_raw.data, L.kv_raw.rope, L.kv_raw.scale};
    void* win[3] = {L.win.data, L.win.rope, L.win.scale};
    const int bytes[3] = {L.D - R, 2 * R, 4};
    for (int i = 0; i < 3; ++i) {
      a.raw[i] = raw[i];
      a.win[i] = win[i];
      a.plane_bytes[i] = bytes[i];
      if (bytes[i] % 4) return -2;
    }
  } else {
    a.raw[0] = L.kv_raw.data;
    a.win[0] = L.win.data;
    a.plane_bytes[0] = L.D * (L.win.dtype == CSA_F32 ? 4 : 2);
  }
  a.n_win = L.n_win;
  a.Ws = L.Ws;
  a.win_pos0 = L.win_pos0;
  a.pmap = L.pmap;
  a.q_pos = L.q_pos;
  a.wp0_b = L.wp0_b;
  a.wp0_adj = L.wp0_adj;
  a.vis_idx = L.vis_idx;
  a.vis_K = L.vis_K;
  const dim3 g(static_cast<uint32_t>(L.B)), t(kThreads);
  if (L.stream_dtype == CSA_F32) hipLaunchKernelGGL(state_append_kernel<float>, g, t, 0, stream, a);
  else hipLaunchKernelGGL(state_append_kernel<uint16_t>, g, t, 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

namespace {

struct QuantArgs {
  const float* x;
  int64_t rows;
  int D, chunks, entries_per_wg;
  OutDesc out;
};

__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantArgs a) {
  __shared__ uint32_t amax_lds[kThreads];
  const int tid = threadIdx.x;
  const int e_local = tid / a.chunks;
  const int c = tid % a.chunks;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * a.entries_per_wg + e_local;
  const bool active = e_local < a.entries_per_wg && row < a.rows;
  const int aw = amax_words(a.out.dtype, a.D);
  for (int i = tid; i < a.entries_per_wg * aw && i < kThreads; i += kThreads) amax_lds[i] = 0u;
  float v[kVec];
  if (active) load8<float>(a.x + row * a.D + c * kVec, v);
  __syncthreads();
  if (active) amax_chunk(a.out, c, v, amax_lds + e_local * aw);
  __syncthreads();
  if (active) store_chunk(a.out, row, c, v, amax_lds + e_local * aw);
}

}  // namespace

namespace {

// Fill the job description of one compression and return its block count.
int64_t make_job(const CompressLaunch& L, CompressArgs& a, bool general_only = false) {
  a = CompressArgs{};
  a.ca = L.ca; a.cb = L.cb; a.za = L.za; a.zb = L.zb;
  a.bias_a = L.bias_a; a.bias_b = L.bias_b;
  a.prev_cb = L.prev_cb; a.prev_zb = L.prev_zb;
  a.B = L.B; a.T = L.T; a.t0 = L.t0; a.out_rows = L.out_rows; a.pos_offset = L.pos_offset;
  a.D = L.D; a.ratio = L.ratio; a.overlap = L.overlap; a.R = L.rope_dims;
  a.log2_base = L.log2_base;
  a.out = OutDesc{L.out.data, L.out.rope, L.out.scale, L.out.dtype, L.D, L.rope_dims};
  a.norm_w = L.norm_w;
  a.norm_eps = L.norm_eps;
  a.chunks = L.D / kVec;
  const int nrows = L.overlap ? 2 * L.ratio : L.ratio;
  if (general_only) {
    a.mode = kModeGeneral;  // set below
  } else if (nrows <= kBatch) {
    a.mode = kModeSmall;
    a.G = 1;
    a.entries_per_wg = kThreads / a.chunks;
  } else if (!L.overlap && L.ratio % kBatch == 0 && a.chunks <= kThreads) {
    // the most groups that fit the workgroup and split the block into whole batches
    int G = 1;
    while (2 * G * a.chunks <= kThreads && (L.ratio / kBatch) % (2 * G) == 0) G *= 2;
    a.mode = kModeGroups;
    a.G = G;
    a.entries_per_wg = kThreads / (a.chunks * G);
  }
  if (general_only || (a.mode != kModeSmall && a.mode != kModeGroups)) {
    // row groups: enough to keep every wave busy on long blocks
    int G = 1;
    while (G * 2 * a.chunks <= kThreads && nrows / (G * 2) >= kBatch) G *= 2;
    a.mode = kModeGeneral;
    a.G = G;
    a.entries_per_wg = kThreads / (a.chunks * G);
  }
  const int64_t n_entries = L.B * (L.T / L.ratio);
  return (n_entries + a.entries_per_wg - 1) / a.entries_per_wg;
}

template <int MODE>
void launch_mode(const CompressArgs2& a, int64_t grid, int stream_dtype, hipStream_t stream) {
  const dim3 g(static_cast<uint32_t>(grid)), t(kThreads);
  if (stream_dtype == CSA_F32) hipLaunchKernelGGL((compress_kernel<float, MODE>), g, t, 0, stream, a);
  else hipLaunchKernelGGL((compress_kernel<uint16_t, MODE>), g, t, 0, stream, a);
}

int launch(const CompressArgs2& a, int64_t grid, int stream_dtype, hipStream_t stream) {
  if (grid == 0) return 0;
  const int mode = a.job[0].mode;  // the two jobs of one launch share a path
  if (grid != a.grid0 && a.job[1].mode != mode) return -1;
  if (mode == kModeSmall) launch_mode<kModeSmall>(a, grid, stream_dtype, stream);
  else if (mode == kModeGroups) launch_mode<kModeGroups>(a, grid, stream_dtype, stream);
  else launch_mode<kModeGeneral>(a, grid, stream_dtype, stream);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_compress(const CompressLaunch& L, hipStream_t stream) {
  CompressArgs2 a{};
  a.grid0 = make_job(L, a.job[0]);
  return launch(a, a.grid0, L.stream_dtype, stream);
}

int launch_compress2(const CompressLaunch& L0, const CompressLaunch& L1, hipStream_t stream) {
  CompressArgs2 a{};
  a.grid0 = make_job(L0, a.job[0]);
  int64_t g1 = make_job(L1, a.job[1]);
  if (a.job[0].mode != a.job[1].mode) {  // both take the general path
    a.grid0 = make_job(L0, a.job[0], true);
    g1 = make_job(L1, a.job[1], true);
  }
  return launch(a, a.grid0 + g1, L0.stream_dtype, stream);
}

// Row-wise RMSNorm launches (rmsnorm.h)
__global__ __launch_bounds__(256) void rmsnorm_kernel(NormArgs a) {
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  norm_row(a.x, row, a.y, row, a.w, a.D, a.dtype, a.eps, threadIdx.x & 63);
}

int launch_rmsnorm(const csa_buf& x, int64_t rows, int D, const float* w, float eps, const csa_buf& y,
                   hipStream_t stream) {
  if (rows == 0) return 0;
  if (x.dtype != y.dtype || (x.dtype != CSA_F32 && x.dtype != CSA_BF16) || D % kVec || D > 2048) return -2;
  if ((rows + 3) / 4 >= (int64_t(1) << 31)) return -4;
  NormArgs a{x.data, y.data, w, rows, D, x.dtype, eps};
  hipLaunchKernelGGL(rmsnorm_kernel, dim3(static_cast<uint32_t>((rows + 3) / 4)), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

__global__ __launch_bounds__(256) void attn_norm_kernel(AttnNormArgs a) { attn_norm_block<4>(a, blockIdx.x); }

AttnNormArgs make_attn_norm(const csa_buf& q, const csa_buf& q_out, const float* q_w, const csa_buf& win,
                            const csa_buf& win_out, const float* kv_w, const int64_t* q_pos, const int64_t* win_pos0,
                            int64_t B, int64_t Tq, int64_t Tw, int H, int D, int n_win, float eps) {
  AttnNormArgs a{};
  a.q = NormArgs{q.data, q_out.data, q_w, B * Tq * H, D, q.dtype, eps};
  a.win = win.data;
  a.win_out = win_out.data;
  a.kv_w = kv_w;
  a.q_pos = q_pos;
  a.win_pos0 = win_pos0;
  a.B = B;
  a.Tq = Tq;
  a.Tw = Tw;
  a.win_dtype = win.dtype;
  a.n_win = n_win;
  return a;
}

int launch_attn_norm(AttnNormArgs a, hipStream_t stream) {
  if (a.q.rows == 0) return 0;
  if ((a.q.dtype != CSA_F32 && a.q.dtype != CSA_BF16) || (a.win_dtype != CSA_F32 && a.win_dtype != CSA_BF16) ||
      a.q.D % kVec || a.q.D > 2048)
    return -2;
  if ((a.q.rows + 3) / 4 + a.B * 1024 >= (int64_t(1) << 31)) return -4;
  attn_norm_shape(a, 4);
  hipLaunchKernelGGL(attn_norm_kernel, dim3(a.blocks), dim3(256), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_quantize(const float* x, int64_t rows, int D, int rope_dims, const csa_buf& out,
                    hipStream_t stream) {
  if (rows == 0) return 0;
  QuantArgs a{};
  a.x = x; a.rows = rows; a.D = D;
  a.chunks = D / kVec;
  a.entries_per_wg = kThreads / a.chunks;
  a.out = OutDesc{out.data, out.rope, out.scale, out.dtype, D, rope_dims};
  const int64_t grid = (rows + a.entries_per_wg - 1) / a.entries_per_wg;
  hipLaunchKernelGGL(quantize_kernel, dim3(static_cast<uint32_t>(grid)), dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
