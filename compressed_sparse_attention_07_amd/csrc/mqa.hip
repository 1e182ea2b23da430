// K4: shared-KV multi-query attention over (selected or all visible) compressed
// entries plus the raw sliding window, with attention sink and partial / inverse
// RoPE.  [V4-CN] "DeepSeek-V4中文翻译" §2.3.1 (shared-KV MQA: an entry is both key
// and value of every head), §2.3.2 (HCA: dense over all compressed entries),
// §2.3.3 (window branch, sink logit added to the softmax denominator, RoPE on the
// last 64 dims and the output rotated back by the query position); [NOTES]
// csa()/hca() sketches: one attention over concat(entries, window).
//
// MFMA path (bf16 queries, bf16 or FP8-mixed cache): a workgroup owns one query
// token, a group of heads (16 per wave) and a range of key slots.  Key tiles of 32
// rows are gathered into LDS twice: row-major (A operand of S^T = K Q^T) and
// transposed (A operand of O^T = V^T P^T).  Computing the transposed products
// makes every lane hold one head's column in both results, so the online-softmax
// rescale is one factor per lane and P^T feeds the PV product straight from the
// S^T registers (the contraction order over the tile's keys is permuted to match
// the lanes' own keys).  FP8-mixed entries are staged as exact bf16 codes and the
// per-entry scale is applied to the logits and to P (non-RoPE dims only).  With
// several key ranges per token, partial (max, sum, O) go to the workspace and a
// combine kernel merges them in fixed split order, so results do not depend on
// scheduling or batch composition.
#include <algorithm>
#include <cmath>

#include "device_common.h"
#include "launch.h"

namespace csa {

namespace {

struct AttnArgs {
  // what every workgroup reads first sits at the front of the argument block (three
  // 64-byte lines), so a prologue fetches it in one burst
  int H, D, n_win, hpw;
  int nsplit, sps, K, ratio;
  int sparse, R, out_dtype;
  uint32_t nblk;  // blocks in the grid of the attention launch
  float scale;
  int64_t B, Tq, N;
  int64_t kv_rows, Tw, pos_offset;
  const void* q;
  const int64_t* q_pos;
  const int64_t* win_pos0;
  const int32_t* idx;
  const void* kv;
  const void* win;
  const uint16_t* kv_rope;
  const float* kv_scale;
  const uint16_t* win_rope;
  const float* win_scale;
  const uint16_t* q_rope;  // FP8MIX queries: bf16 RoPE dims [tokens, H, R]
  const float* q_scale;    //               and the per-(token, head) scale
  const float* sink;
  void* out;
  uint16_t* part_o; // [tokens, H, nsplit, D] bf16, O / l of the split
  float2* part_ml;  // [tokens, H, nsplit] (running max, sum of exponentials)
  double log2_base;
  double theta_rev[64];  // RoPE frequency of pair j in revolutions per position
};

struct Slots {
  int64_t b, p, nsel, wstart, nslots, wp0;
};

// x / d for x >= 0, d >= 1, with 32-bit division whenever both fit in 32 bits
__device__ __forceinline__ int64_t div_nonneg(int64_t x, int64_t d) {
  if (((static_cast<uint64_t>(x) | static_cast<uint64_t>(d)) >> 32) == 0)
    return static_cast<uint32_t>(x) / static_cast<uint32_t>(d);
  return x / d;
}

// The slot ranges of token bt (sequence b, position p, window base wp0)
__device__ __forceinline__ Slots slots_of(const AttnArgs& a, int64_t b, int64_t p, int64_t wp0) {
  Slots s;
  s.b = b;
  s.p = p;
  if (a.sparse) {
    s.nsel = a.K;
  } else {
    int64_t v = s.p >= 0 ? div_nonneg(s.p, a.ratio) : s.p / a.ratio;
    s.nsel = v > a.N ? a.N : (v < 0 ? 0 : v);
  }
  s.wstart = s.p - a.n_win + 1 > 0 ? s.p - a.n_win + 1 : 0;
  s.nslots = s.nsel + (s.p - s.wstart + 1);
  s.wp0 = wp0;
  return s;
}

__device__ __forceinline__ Slots token_slots(const AttnArgs& a, int64_t bt) {
  const int64_t b = div_nonneg(bt, a.Tq);
  return slots_of(a, b, a.q_pos[bt], a.win_pos0[b]);
}

// Source row of slot `slot`: returns entry row (>= 0) in kv, or window row in win
// (is_win), or -1 if the slot is empty.
__device__ __forceinline__ int64_t slot_row(const AttnArgs& a, const Slots& s, int64_t bt, int64_t slot,
                                            bool* is_win, int64_t* wpos) {
  if (slot < s.nsel) {
    *is_win = false;
    int64_t e = a.sparse ? static_cast<int64_t>(a.idx[bt * a.K + slot]) : slot;
    return e >= 0 ? s.b * a.kv_rows + e : -1;
  }
  *is_win = true;
  const int64_t pw = s.wstart + (slot - s.nsel);
  *wpos = pw;
  return s.b * a.Tw + (pw - s.wp0);
}

// ================================================================ MFMA path

constexpr int kKT = 32;   // keys per tile

// 16 bytes of a result row.  Split partials are read once, by the combine launch:
// they are stored with the nontemporal hint.
__device__ __forceinline__ void store_row16(uint16_t* dst, uint4 v, bool partial) {
  if (partial) __builtin_nontemporal_store(u32x4_t{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4_t*>(dst));
  else *reinterpret_cast<uint4*>(dst) = v;
}

constexpr float kLog2e = 1.4426950408889634f;  // log2(e)
constexpr float kLn2 = 0.6931471805599453f;     // ln(2)
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }


// At D = 512 a wave needs ~400 registers (16 heads x 512 fp32 accumulators, the
// queries and one prefetched tile), so those workgroups are capped at 4 waves.
template <int D>
constexpr int mfma_max_waves() { return D >= 512 ? 4 : 8; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element (i mod 4)
// of the 8-byte chunks addressed by lanes 4e + i/4, e = 0..3.  With lane j of group g
// addressing row (key) base + 4g + j/4, column d0 + 4(j mod 4) of the row-major tile,
// lane i gets the four keys base + 4g + e at column d0 + i: a column of V, i.e. a row
// of V^T, which is the A operand layout of the PV product.
__device__ __forceinline__ s16x4 lds_read_tr(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)(p)));
}

template <int D, int NW, bool FP8>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KP = D + 8;            // row pitch (bf16): conflict-free 16-byte row reads
  constexpr int NS = D / 32;           // k-steps of S^T = K Q^T
  constexpr int NDB = D / 16;          // 16-row blocks of O^T = V^T P^T
  constexpr int CH = D / 8;            // 16-byte chunks per key row
  constexpr int IPT = kKT * CH / NT;   // chunks per thread per tile
  static_assert(IPT * NT == kKT * CH, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) uint16_t Krow[2][kKT * KP];
  __shared__ __attribute__((aligned(16))) uint16_t Qs[NW * 16 * KP];  // RoPE'd queries of the group
  __shared__ __attribute__((aligned(16))) float kscale[2][kKT];
  __shared__ __attribute__((aligned(16))) int kvalid[2][kKT];
  __shared__ int64_t src_row[2][kKT];  // row in kv / win, -1 = empty
  __shared__ int64_t src_pos[2][kKT];  // window position (window rows)
  __shared__ int src_win[2][kKT];
  __shared__ float2 qcs[64];           // (cos, sin) of the query position per RoPE pair
  __shared__ double theta[64];         // RoPE frequencies in revolutions per position

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;

  const int n_hg = a.H / a.hpw;
  int64_t blk = blockIdx.x;
  const int hg = static_cast<int>(blk % n_hg);
  blk /= n_hg;
  const int sp = static_cast<int>(blk % a.nsplit);
  const int64_t bt = blk / a.nsplit;
  const Slots S = token_slots(a, bt);
  const int64_t s_lo = static_cast<int64_t>(sp) * a.sps;
  const int64_t s_hi = min(S.nslots, s_lo + a.sps);
  const int ntiles = s_hi > s_lo ? static_cast<int>((s_hi - s_lo + kKT - 1) / kKT) : 0;
  const int h = hg * a.hpw + wid * 16 + col;  // head of this lane's result column
  const int nope = D - a.R;
  const double qpos = static_cast<double>(S.p + a.pos_offset);

  for (int j = tid; j < a.R / 2; j += NT) {
    const double th = a.theta_rev[j];
    theta[j] = th;
    float c, sn;
    rope_cs_rev(qpos, th, &c, &sn);
    qcs[j] = make_float2(c, sn);
  }

  // resolve the source rows of tile t into src[buf] in two halves: the entry-index
  // load is issued early (resolve_load) and consumed after the tile's MFMAs
  // (resolve_store), so its latency overlaps the compute
  auto resolve_load = [&](int t) -> int32_t {
    int32_t e = 0;
    if (tid < kKT) {
      const int64_t slot = s_lo + static_cast<int64_t>(t) * kKT + tid;
      e = (a.sparse && slot < s_hi && slot < S.nsel) ? a.idx[bt * a.K + slot] : 0;
    }
    return e;
  };
  auto resolve_store = [&](int t, int buf, int32_t r_e) {
    if (tid < kKT) {
      const int64_t slot = s_lo + static_cast<int64_t>(t) * kKT + tid;
      int64_t row = -1, wpos = 0;
      int win = 0;
      if (slot < s_hi) {
        if (slot < S.nsel) {
          const int64_t e = a.sparse ? static_cast<int64_t>(r_e) : slot;
          row = e >= 0 ? S.b * a.kv_rows + e : -1;
        } else {
          win = 1;
          wpos = S.wstart + (slot - S.nsel);
          row = S.b * a.Tw + (wpos - S.wp0);
        }
      }
      src_row[buf][tid] = row;
      src_pos[buf][tid] = wpos;
      src_win[buf][tid] = win;
    }
  };
  // issue the global loads of tile t (sources in src[buf]) into registers
  uint4 pre[IPT];
  float pre_sc[IPT];
  auto load_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int item = tid + NT * u;
      const int j = item / CH;
      const int c = item % CH;
      const int d0 = 8 * c;
      const int64_t row = src_row[buf][j];
      uint4 v = make_uint4(0, 0, 0, 0);
      float sc = 1.f;
      if (row >= 0) {
        const bool w = src_win[buf][j] != 0;
        const void* base = w ? a.win : a.kv;
        if (FP8) {
          if (c == 0) sc = (w ? a.win_scale : a.kv_scale)[row];
          if (d0 < nope) {
            const uint2 cd = *reinterpret_cast<const uint2*>(static_cast<const uint8_t*>(base) + row * nope + d0);
            v.x = cd.x;
            v.y = cd.y;
          } else {
            v = *reinterpret_cast<const uint4*>((w ? a.win_rope : a.kv_rope) + row * a.R + (d0 - nope));
          }
        } else {
          v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + row * D + d0);
        }
      }
      pre[u] = v;
      pre_sc[u] = sc;
    }
  };
  // dequantize the registers and store them as tile `buf` (row-major bf16)
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < IPT; ++u) {
      const int item = tid + NT * u;
      const int j = item / CH;
      const int c = item % CH;
      const int d0 = 8 * c;
      uint4 v = pre[u];
      if (FP8 && d0 < nope) {
        const uint2 cd = make_uint2(v.x, v.y);
        v.x = e4m3_to_bf16(cd.x & 0xff) | (static_cast<uint32_t>(e4m3_to_bf16((cd.x >> 8) & 0xff)) << 16);
        v.y = e4m3_to_bf16((cd.x >> 16) & 0xff) | (static_cast<uint32_t>(e4m3_to_bf16(cd.x >> 24)) << 16);
        v.z = e4m3_to_bf16(cd.y & 0xff) | (static_cast<uint32_t>(e4m3_to_bf16((cd.y >> 8) & 0xff)) << 16);
        v.w = e4m3_to_bf16((cd.y >> 16) & 0xff) | (static_cast<uint32_t>(e4m3_to_bf16(cd.y >> 24)) << 16);
      }
      *reinterpret_cast<uint4*>(&Krow[buf][j * KP + d0]) = v;
      if (c == 0) {
        kscale[buf][j] = pre_sc[u];
        kvalid[buf][j] = src_row[buf][j] >= 0 ? 1 : 0;
      }
    }
  };
  // window rows are raw: rotate the RoPE dims of tile `buf` to each row's own position
  // (only tiles that reach into the window run this)
  const int RCH = a.R / 8;  // 16-byte chunks of RoPE dims per row
  auto rope_window_rows = [&](int buf) {
    for (int item = tid; item < kKT * RCH; item += NT) {
      const int j = item / RCH;
      if (!src_win[buf][j] || src_row[buf][j] < 0) continue;
      const int d0 = nope + 8 * (item % RCH);
      uint4 v = *reinterpret_cast<const uint4*>(&Krow[buf][j * KP + d0]);
      float x[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                    bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
      const double kp = static_cast<double>(src_pos[buf][j] + a.pos_offset);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float cc, sn;
        rope_cs_rev(kp, theta[(d0 + e - nope) / 2], &cc, &sn);
        const float x0 = x[e], x1 = x[e + 1];
        x[e] = x0 * cc - x1 * sn;
        x[e + 1] = x0 * sn + x1 * cc;
      }
      v = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7]));
      *reinterpret_cast<uint4*>(&Krow[buf][j * KP + d0]) = v;
    }
  };
  // does tile t hold window rows?  (slots >= nsel are window positions)
  auto tile_has_window = [&](int t) {
    const int64_t first = s_lo + static_cast<int64_t>(t) * kKT;
    return min(first + kKT, s_hi) > S.nsel && first < s_hi;
  };

  // prologue: the entry indices of tiles 0 and 1 and the queries are fetched together,
  // tile 0's rows are requested as soon as its indices are known, and the query RoPE /
  // LDS staging runs while they are in flight
  constexpr int QIT = 16 * CH / 64;  // 16-byte query chunks per thread (NW*16 heads over NW*64 threads)
  uint4 qv[QIT];
  {
    const uint16_t* qg = static_cast<const uint16_t*>(a.q) + (bt * a.H + hg * a.hpw) * D;
#pragma unroll
    for (int u = 0; u < QIT; ++u) {
      const int i = tid + NT * u;
      qv[u] = *reinterpret_cast<const uint4*>(qg + (i / CH) * D + 8 * (i % CH));
    }
  }
  {
    const int32_t e0 = resolve_load(0);
    const int32_t e1 = resolve_load(1);
    resolve_store(0, 0, e0);
    resolve_store(1, 1, e1);
  }
  __syncthreads();
  if (ntiles > 0) load_tile(0);

  // queries of the head group, RoPE'd at the query position, staged once in LDS;
  // the B operand of S^T = K Q^T (q[h][32s + 8grp .. +8]) is read from there per tile,
  // which keeps the registers for the accumulators
#pragma unroll
  for (int u = 0; u < QIT; ++u) {
    const int i = tid + NT * u;
    const int hr = i / CH;
    const int d0 = 8 * (i % CH);
    uint4 raw = qv[u];
    if (d0 + 8 > nope) {
      float v[8] = {bf16lo(raw.x), bf16hi(raw.x), bf16lo(raw.y), bf16hi(raw.y),
                    bf16lo(raw.z), bf16hi(raw.z), bf16lo(raw.w), bf16hi(raw.w)};
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        if (d0 + e >= nope) {
          const float2 cs = qcs[(d0 + e - nope) / 2];
          const float x0 = v[e], x1 = v[e + 1];
          v[e] = x0 * cs.x - x1 * cs.y;
          v[e + 1] = x0 * cs.y + x1 * cs.x;
        }
      }
      raw = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7]));
    }
    *reinterpret_cast<uint4*>(&Qs[hr * KP + d0]) = raw;
  }
  const uint16_t* qrow = Qs + (wid * 16 + col) * KP + 8 * grp;
  if (ntiles > 0) store_tile(0);
  __syncthreads();
  if (ntiles > 0 && tile_has_window(0)) {
    rope_window_rows(0);
    __syncthreads();
  }

  f32x4 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    const int cur = t & 1, nxt = cur ^ 1;
    const bool more = t + 1 < ntiles;
    if (more) load_tile(nxt);  // in flight during this tile's MFMAs
    const int32_t e2 = (t + 2 < ntiles) ? resolve_load(t + 2) : 0;

    const uint16_t* K = Krow[cur];
    // ---- S^T = K Q^T for the 32 keys (two 16-key blocks)
    f32x4 sacc[2], racc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      racc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8 qf = *reinterpret_cast<const bf16x8*>(qrow + 32 * s);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(K + (16 * kb + col) * KP + 8 * grp + 32 * s);
        if (FP8 && 32 * s >= nope)
          racc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf, racc[kb], 0, 0, 0);
        else
          sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf, sacc[kb], 0, 0, 0);
      }
    }
    // ---- online softmax for head h over this lane's 8 keys (16kb + 4grp + r)
    float z[2][4], ksc[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int4 kv4 = *reinterpret_cast<const int4*>(&kvalid[cur][16 * kb + 4 * grp]);
      const float4 ks4 = *reinterpret_cast<const float4*>(&kscale[cur][16 * kb + 4 * grp]);
      const int vv[4] = {kv4.x, kv4.y, kv4.z, kv4.w};
      const float kk[4] = {ks4.x, ks4.y, ks4.z, ks4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ksc[kb][r] = kk[r];
        float v = FP8 ? fmaf(kk[r], sacc[kb][r], racc[kb][r]) : sacc[kb][r];
        v = vv[r] ? a.scale * v : -INFINITY;
        z[kb][r] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = rows4_max(mt);
    // Lazy rescaling: the exponentials use a reference max m_run that is raised only
    // when a logit exceeds it by more than kSlack (so p <= e^kSlack); O and l always
    // refer to the same m_run, so the result is exact whatever the reference.
    constexpr float kSlack = 8.f;
    const bool raise = mt > m_run + kSlack;
    const float m_ref = raise ? mt : m_run;
    if (__any(raise)) {  // wave-uniform: rescale the accumulators of the heads that moved
      const float alpha = (m_run == -INFINITY || !raise) ? (raise ? 0.f : 1.f) : __expf(m_run - m_ref);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
    m_run = m_ref;
    const bool none = (m_run == -INFINITY);
    float pn[8], pr[8];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = none ? 0.f : __expf(z[kb][r] - m_run);
        psum += p;
        pr[4 * kb + r] = p;
        pn[4 * kb + r] = FP8 ? p * ksc[kb][r] : p;
      }
    }
    l_run += psum;
    const bf16x8 pB = __builtin_bit_cast(
        bf16x8, make_uint4(pack_bf16x2(pn[0], pn[1]), pack_bf16x2(pn[2], pn[3]), pack_bf16x2(pn[4], pn[5]),
                           pack_bf16x2(pn[6], pn[7])));
    bf16x8 pR = pB;
    if (FP8)
      pR = __builtin_bit_cast(
          bf16x8, make_uint4(pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]), pack_bf16x2(pr[4], pr[5]),
                             pack_bf16x2(pr[6], pr[7])));
    // ---- O^T += V^T P^T; V^T rows come straight from the row-major tile by transpose reads:
    //      keys 4grp + (0..3) and 16 + 4grp + (0..3), matching P^T's key order
    const uint16_t* vb = K + (4 * grp + (col >> 2)) * KP + 4 * (col & 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const s16x4 lo = lds_read_tr(vb + 16 * db);
      const s16x4 hi = lds_read_tr(vb + 16 * KP + 16 * db);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, (FP8 && 16 * db >= nope) ? pR : pB, acc[db], 0, 0, 0);
    }

    if (more) store_tile(nxt);
    if (t + 2 < ntiles) resolve_store(t + 2, cur, e2);
    __syncthreads();
    if (more && tile_has_window(t + 1)) {
      rope_window_rows(nxt);
      __syncthreads();
    }
  }

  // sum of exponentials for head h: the four row groups hold disjoint keys
  float l_tot = l_run;
  l_tot = rows4_sum(l_tot);

  const int64_t th = bt * a.H + h;
  if (a.nsplit > 1) {
    // normalised partial (a convex combination of keys) stored as bf16
    uint16_t* po = a.part_o + (th * a.nsplit + sp) * D;
    const float il = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      *reinterpret_cast<uint2*>(po + 16 * db + 4 * grp) =
          make_uint2(pack_bf16x2(acc[db][0] * il, acc[db][1] * il), pack_bf16x2(acc[db][2] * il, acc[db][3] * il));
    if (grp == 0) a.part_ml[th * a.nsplit + sp] = make_float2(m_run, l_tot);
    return;
  }
  // ---- finalize: sink, normalise, inverse RoPE, store bf16
  const float sk = a.sink[h];
  float inv;
  if (sk == INFINITY) inv = 0.f;
  else if (sk == -INFINITY) inv = 1.f / l_tot;
  else inv = 1.f / (l_tot + __expf(sk - m_run));
  uint16_t* op = static_cast<uint16_t*>(a.out) + th * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d0 = 16 * db + 4 * grp;
    float v[4] = {acc[db][0] * inv, acc[db][1] * inv, acc[db][2] * inv, acc[db][3] * inv};
#pragma unroll
    for (int e = 0; e < 4; e += 2) {
      if (d0 + e >= nope) {
        // rotate back by the query position: angle -> -angle
        const float2 cs = qcs[(d0 + e - nope) / 2];
        const float x0 = v[e], x1 = v[e + 1];
        v[e] = x0 * cs.x + x1 * cs.y;
        v[e + 1] = x1 * cs.x - x0 * cs.y;
      }
    }
    *reinterpret_cast<uint2*>(op + d0) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
}

// ================================================================ LDS-DMA path (bf16, D = 512)
//
// The computation of attn_mfma_kernel, with the key rows brought into LDS by direct
// global->LDS loads: one global_load_lds_dwordx4 moves one 1 KiB row, lane i's 16
// bytes landing at M0 + 16 i.  No registers hold tiles in flight, so a ring of
// kDmaStages tiles keeps three tiles of gathered rows in flight while the fourth is
// computed on.  The queries live in registers (B operand of S^T = K Q^T), loaded and
// roped there once.  With 8 waves (128 heads) two waves share each SIMD, so one wave's
// LDS reads overlap the other's MFMAs.  Each wave issues the same number of row loads for every
// tile (an empty slot loads the query's own window row, which the softmax masks), so
// "tile t has landed" is "at most (rows per wave) x (tiles issued after t) vector
// memory operations outstanding", waited for with s_waitcnt and made visible to the
// other waves by the barrier that follows.  The compiler does not see these loads;
// the loop issues no other vector-memory operation.
//
// FP8MIX caches (FP8 = true): a row is three direct loads (448 e4m3 codes, 64 bf16
// RoPE dims, the f32 entry scale) into a ring of raw rows; once a tile has landed,
// one pass of the workgroup converts it (hardware e4m3 -> f32, times the scale,
// rounded to bf16; window rows' RoPE dims rotated) into a single bf16 tile that the
// MFMA loop reads exactly as in the bf16 case.

constexpr int kDmaStages = 4;
constexpr bool kDmaPipe = true;  // long key ranges take the software-pipelined loop
constexpr int kPipeMinSlots = 8 * 32;  // ... ranges of at least 8 tiles, or unsplit ones
constexpr int kDmaIdxCap = 2048;  // entry indices of one workgroup's slot range, staged in LDS

template <int NW, int R, bool FP8, bool PIPE = false, bool FQ = false>
__global__ __launch_bounds__(NW * 64) void attn_dma_kernel(AttnArgs a) {
  constexpr int D = 512;
  constexpr int NT = NW * 64;
  constexpr int KP = D + 16;           // row pitch (bf16): 1056 B, the S^T operand reads run at full LDS rate
  constexpr int NS = D / 32;
  constexpr int NDB = D / 16;
  constexpr int RPW = kKT / NW;        // rows each wave loads per tile
  constexpr int STAGE = kKT * KP;      // bf16 per ring stage
  constexpr int LPR = FP8 ? 3 : 1;     // direct loads per row
  constexpr int RAWROW = (D - R) + 2 * R;  // bytes of an FP8MIX row: codes, then bf16 RoPE dims
  static_assert(RPW * LPR * (kDmaStages - 2) < 64, "outstanding row loads must fit vmcnt");
  static_assert(!FP8 || STAGE * 2 + kDmaStages * kKT * RAWROW <= kDmaStages * STAGE * 2, "raw rows fit the ring");
  static_assert(!FQ || (FP8 && !PIPE && R == 64), "FP8MIX queries go with an FP8MIX cache, 64 RoPE dims");

  // bf16: kDmaStages tiles.  FP8MIX: the converted tile (the first STAGE) and the raw
  // rows of kDmaStages tiles behind it.  The epilogue reuses all of it.
  __shared__ __attribute__((aligned(16))) uint16_t ring[kDmaStages * STAGE];
  __shared__ __attribute__((aligned(16))) float rscale[FP8 ? kDmaStages : 1][kKT];  // FP8MIX entry scales
  __shared__ __attribute__((aligned(16))) int idx_s[kDmaIdxCap];
  __shared__ __attribute__((aligned(16))) float kbias[kDmaStages][kKT];  // 0, or -inf for an empty slot
  __shared__ int64_t wpos_s[kDmaStages][kKT];  // window position of a window row, -1 otherwise
  __shared__ float2 qcs[64];
  __shared__ double theta[64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15;
  const int grp = lane >> 4;

  // The argument block's scalars are all fetched before the first is used: otherwise
  // the compiler loads them a cache line at a time, each load after a full wait.
  asm volatile("" ::"s"(a.H), "s"(a.hpw), "s"(a.nsplit), "s"(a.sps), "s"(a.K), "s"(a.sparse), "s"(a.n_win),
               "s"(a.ratio), "s"(a.Tq), "s"(a.N), "s"(a.kv_rows), "s"(a.Tw), "s"(a.pos_offset), "s"(a.q),
               "s"(a.q_pos), "s"(a.win_pos0), "s"(a.idx), "s"(a.kv), "s"(a.win), "s"(a.nblk));
  // the grid has fewer than 2^32 blocks: 32-bit index arithmetic
  const uint32_t n_hg = static_cast<uint32_t>(a.H / a.hpw);
  const uint32_t blk = xcd_block(blockIdx.x, a.nblk);
  const int hg = __builtin_amdgcn_readfirstlane(static_cast<int>(blk % n_hg));
  const uint32_t blk2 = blk / n_hg;
  const int sp = __builtin_amdgcn_readfirstlane(static_cast<int>(blk2 % static_cast<uint32_t>(a.nsplit)));
  const int64_t bt = __builtin_amdgcn_readfirstlane(static_cast<int>(blk2 / static_cast<uint32_t>(a.nsplit)));
  const int64_t s_lo = static_cast<int64_t>(sp) * a.sps;
  // prologue loads, in the order they are needed: the token's position and window base
  // and the RoPE angles, the range's entry indices, then the queries (straight into the
  // B-operand registers: lane (col, grp) holds q[head col][32 s + 8 grp .. + 8]).  Loads
  // return in issue order, so the row loads the indices address go out while the
  // queries are still in flight.
  const uint32_t ring_b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
  // bt < 2^32 (the grid) and so is Tq
  const int64_t b_seq = static_cast<uint32_t>(bt) / static_cast<uint32_t>(a.Tq);
  const int64_t p_pre = a.q_pos[bt];
  const int64_t wp0_pre = a.win_pos0[b_seq];
  const double th_pre = tid < R / 2 ? a.theta_rev[tid] : 0.0;  // R <= 128 < 2 NT
  asm volatile("" ::: "memory");
  int32_t idx_pre[kDmaIdxCap / NT];
  const int64_t n_idx = a.sparse ? min(s_lo + a.sps, static_cast<int64_t>(a.K)) - s_lo : 0;
#pragma unroll
  for (int u = 0; u < kDmaIdxCap / NT; ++u) {
    const int64_t i = tid + static_cast<int64_t>(u) * NT;
    idx_pre[u] = i < n_idx ? a.idx[bt * a.K + s_lo + i] : 0;
  }
  asm volatile("" ::: "memory");  // keep the index loads ahead of the query loads
  uint4 qraw[FQ ? 1 : NS];
  // FP8MIX queries (FQ): e4m3 codes as the B operand of the 128-deep fp8 products (lane
  // (col, grp) holds codes 128 c + 32 grp .. + 32 of head col; the 64 past the D - R
  // codes are zero), the head's scale, and its bf16 RoPE dims as a bf16 B operand
  v8i32 q8[FQ ? 4 : 1];
  uint4 qrraw[FQ ? 2 : 1];
  float qsc = 0.f;
  if constexpr (FQ) {
    const int64_t qh = bt * a.H + hg * a.hpw + wid * 16 + col;
    const uint8_t* qc = static_cast<const uint8_t*>(a.q) + qh * (D - R);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
      if (128 * c + 32 * grp < D - R) {
        lo = *reinterpret_cast<const uint4*>(qc + 128 * c + 32 * grp);
        hi = *reinterpret_cast<const uint4*>(qc + 128 * c + 32 * grp + 16);
      }
      q8[c] = v8i32{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                    static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
    }
    qsc = a.q_scale[qh];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) qrraw[s2] = *reinterpret_cast<const uint4*>(a.q_rope + qh * R + 32 * s2 + 8 * grp);
  } else {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (bt * a.H + hg * a.hpw + wid * 16 + col) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < NS; ++s) qraw[s] = *reinterpret_cast<const uint4*>(qrow + 32 * s);
  }
  const Slots S = slots_of(a, b_seq, uni64(p_pre), uni64(wp0_pre));
  const int64_t s_hi = min(S.nslots, s_lo + a.sps);
  const int ntiles = s_hi > s_lo ? static_cast<int>((s_hi - s_lo + kKT - 1) / kKT) : 0;
  const int h = hg * a.hpw + wid * 16 + col;
  constexpr int nope = D - R;  // the RoPE dims are the last R
  const double qpos = static_cast<double>(S.p + a.pos_offset);
  const uint16_t* kvp = static_cast<const uint16_t*>(a.kv);
  const uint16_t* winp = static_cast<const uint16_t*>(a.win);

  if (tid < R / 2) {
    theta[tid] = th_pre;
    float c, sn;
    rope_cs_rev(qpos, th_pre, &c, &sn);
    qcs[tid] = make_float2(c, sn);
  }

#pragma unroll
  for (int u = 0; u < kDmaIdxCap / NT; ++u) {
    const int64_t i = tid + static_cast<int64_t>(u) * NT;
    if (i < n_idx) idx_s[i] = idx_pre[u];
  }
  // the LDS stores above (indices, angles) reach every wave; the query loads stay in
  // flight.  The compiler's own waits for qraw count only the loads it knows of, which
  // are issued before the row loads: such a wait can only be stricter than needed.
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  // source row of slot j of tile u; empty slots read the query's own window row (the
  // softmax masks them).  Every quantity here is wave-uniform.
  const int64_t u_lo = uni64(s_lo), u_hi = uni64(s_hi), u_nsel = uni64(S.nsel), u_wstart = uni64(S.wstart);
  const uint16_t* kv_b = kvp + uni64(S.b * a.kv_rows) * D;
  const uint16_t* win_b = winp + uni64(S.b * a.Tw - S.wp0) * D;  // row of window position p: win_b + p*D
  const uint16_t* win_self = win_b + uni64(S.p) * D;
  // issue the row loads of tile u into ring stage u % kDmaStages: lane i < RPW resolves
  // row wid*RPW + i, then each row's base address is broadcast to one row load
  auto issue = [&](int u) {
    const int st = u % kDmaStages;
    if constexpr (FP8) {
      // lane i < RPW resolves row wid*RPW + i to (row number, window or cache)
      int64_t rid = S.b * a.Tw + (S.p - S.wp0);  // empty slot: the query's own window row
      int isw = 1;
      if (lane < RPW) {
        const int j = wid * RPW + lane;
        const int64_t slot = u_lo + static_cast<int64_t>(u) * kKT + j;
        const bool live = slot < u_hi;
        const bool sel = slot < u_nsel;
        int64_t e = slot;
        if (a.sparse) e = idx_s[min(slot - u_lo, static_cast<int64_t>(kDmaIdxCap - 1))];
        const int64_t wp = u_wstart + (slot - u_nsel);
        const bool ok = live && (!sel || e >= 0);
        kbias[st][j] = ok ? 0.f : -INFINITY;
        wpos_s[st][j] = (ok && !sel) ? wp : -1;
        if (ok && sel) {
          rid = S.b * a.kv_rows + e;
          isw = 0;
        } else if (ok) {
          rid = S.b * a.Tw + (wp - S.wp0);
        }
      }
      const uint32_t raw_b = ring_b + STAGE * 2 + (st * kKT + wid * RPW) * RAWROW;
      const uint32_t sc_b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&rscale[st][wid * RPW]));
#pragma unroll
      for (int i = 0; i < RPW; ++i) {
        const int64_t r = static_cast<int64_t>((static_cast<uint64_t>(static_cast<uint32_t>(
                              __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint64_t>(rid) >> 32), i))) << 32) |
                          static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(rid), i)));
        const bool w = __builtin_amdgcn_readlane(isw, i) != 0;
        const uint8_t* codes = static_cast<const uint8_t*>(w ? a.win : a.kv) + r * (D - R);
        const uint16_t* rope = (w ? a.win_rope : a.kv_rope) + r * R;
        const float* scl = (w ? a.win_scale : a.kv_scale) + r;
        if (lane < (D - R) / 16) lds_dma16(codes + lane * 16, raw_b + i * RAWROW);
        if (lane < R / 8) lds_dma16(rope + lane * 8, raw_b + i * RAWROW + (D - R));
        if (lane == 0) lds_dma4(scl, sc_b + i * 4);
      }
      return;
    }
    const uint16_t* src = win_self;
    if (lane < RPW) {
      const int j = wid * RPW + lane;
      const int64_t slot = u_lo + static_cast<int64_t>(u) * kKT + j;
      const bool live = slot < u_hi;
      const bool sel = slot < u_nsel;
      int64_t e = slot;
      if (a.sparse) e = idx_s[min(slot - u_lo, static_cast<int64_t>(kDmaIdxCap - 1))];
      const int64_t wp = u_wstart + (slot - u_nsel);
      const bool ok = live && (!sel || e >= 0);
      kbias[st][j] = ok ? 0.f : -INFINITY;
      wpos_s[st][j] = (ok && !sel) ? wp : -1;
      src = !ok ? win_self : (sel ? kv_b + e * D : win_b + wp * D);
    }
    const uint64_t sa = reinterpret_cast<uint64_t>(src);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      // readlane returns int: widen through uint32_t so the low half is not sign-extended
      const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(sa), i));
      const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(sa >> 32), i));
      const uint16_t* row = reinterpret_cast<const uint16_t*>((hi << 32) | lo);
      // dense attention gathers with the nontemporal hint (measured: the HCA decode step
      // 3 % faster, prefill unchanged); sparse prefill lists of neighbouring queries share
      // rows through the caches and measured 8 % slower with it
      if (a.sparse) lds_dma16(row + lane * 8, ring_b + (st * STAGE + (wid * RPW + i) * KP) * 2);
      else lds_dma16_nt(row + lane * 8, ring_b + (st * STAGE + (wid * RPW + i) * KP) * 2);
    }
  };
  // window rows are raw: rotate their RoPE dims to each row's own position
  constexpr int RCH = R / 8;
  auto rope_window_rows = [&](int st) {
    uint16_t* T = ring + st * STAGE;
    for (int item = tid; item < kKT * RCH; item += NT) {
      const int j = item / RCH;
      const int64_t wpj = wpos_s[st][j];
      if (wpj < 0) continue;
      const int d0 = nope + 8 * (item % RCH);
      uint4 v = *reinterpret_cast<const uint4*>(&T[j * KP + d0]);
      float x[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                    bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
      const double kp = static_cast<double>(wpj + a.pos_offset);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float cc, sn;
        rope_cs_rev(kp, theta[(d0 + e - nope) / 2], &cc, &sn);
        const float x0 = x[e], x1 = x[e + 1];
        x[e] = x0 * cc - x1 * sn;
        x[e + 1] = x0 * sn + x1 * cc;
      }
      *reinterpret_cast<uint4*>(&T[j * KP + d0]) =
          make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7]));
    }
  };
  auto tile_has_window = [&](int t) {
    const int64_t first = s_lo + static_cast<int64_t>(t) * kKT;
    return min(first + kKT, s_hi) > S.nsel && first < s_hi;
  };
  // FP8MIX: raw rows of stage st -> the bf16 tile (codes times the entry scale; window
  // rows' RoPE dims rotated to their own position)
  auto convert = [&](int st) {
    const uint8_t* Rw = reinterpret_cast<const uint8_t*>(ring + STAGE) + st * kKT * RAWROW;
    for (int item = tid; item < kKT * (D / 8); item += NT) {
      const int j = item / (D / 8);
      const int d0 = 8 * (item % (D / 8));
      uint4 o;
      if (d0 < nope) {
        const uint2 cd = *reinterpret_cast<const uint2*>(Rw + j * RAWROW + d0);
        const float sc = rscale[st][j];
        typedef float f2_t __attribute__((ext_vector_type(2)));
        const f2_t x0 = __builtin_amdgcn_cvt_pk_f32_fp8(cd.x, false), x1 = __builtin_amdgcn_cvt_pk_f32_fp8(cd.x, true);
        const f2_t x2 = __builtin_amdgcn_cvt_pk_f32_fp8(cd.y, false), x3 = __builtin_amdgcn_cvt_pk_f32_fp8(cd.y, true);
        o = make_uint4(pack_bf16x2(x0.x * sc, x0.y * sc), pack_bf16x2(x1.x * sc, x1.y * sc),
                       pack_bf16x2(x2.x * sc, x2.y * sc), pack_bf16x2(x3.x * sc, x3.y * sc));
      } else {
        o = *reinterpret_cast<const uint4*>(Rw + j * RAWROW + nope + 2 * (d0 - nope));
        const int64_t wpj = wpos_s[st][j];
        if (wpj >= 0) {
          float x[8] = {bf16lo(o.x), bf16hi(o.x), bf16lo(o.y), bf16hi(o.y),
                        bf16lo(o.z), bf16hi(o.z), bf16lo(o.w), bf16hi(o.w)};
          const double kp = static_cast<double>(wpj + a.pos_offset);
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float cc, sn;
            rope_cs_rev(kp, theta[(d0 + e - nope) / 2], &cc, &sn);
            const float y0 = x[e], y1 = x[e + 1];
            x[e] = y0 * cc - y1 * sn;
            x[e + 1] = y0 * sn + y1 * cc;
          }
          o = make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                         pack_bf16x2(x[6], x[7]));
        }
      }
      *reinterpret_cast<uint4*>(&ring[j * KP + d0]) = o;
    }
  };

  // tiles 0..2 in flight while the queries are roped in registers
  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  if (ntiles > 2) issue(2);
  bf16x8 qf[FQ ? 2 : NS];  // FQ: the RoPE dims only (k-steps nope / 32 .. NS - 1)
#pragma unroll
  for (int s = 0; s < (FQ ? 2 : NS); ++s) {
    uint4 raw = FQ ? qrraw[FQ ? s : 0] : qraw[FQ ? 0 : s];
    const int d0 = (FQ ? nope : 0) + 32 * s + 8 * grp;
    if (d0 + 8 > nope) {
      float v[8] = {bf16lo(raw.x), bf16hi(raw.x), bf16lo(raw.y), bf16hi(raw.y),
                    bf16lo(raw.z), bf16hi(raw.z), bf16lo(raw.w), bf16hi(raw.w)};
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        if (d0 + e >= nope) {
          const float2 cs = qcs[(d0 + e - nope) / 2];
          const float x0 = v[e], x1 = v[e + 1];
          v[e] = x0 * cs.x - x1 * cs.y;
          v[e + 1] = x0 * cs.y + x1 * cs.x;
        }
      }
      raw = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7]));
    }
    qf[s] = __builtin_bit_cast(bf16x8, raw);
  }

  f32x4 acc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running max in base-2 units (logits scaled by scale * log2 e), exponentials by v_exp_f32
  const float scale2 = a.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;

  // ---- FQ: S^T from the raw rows of stage st: the D - R coded dims by 128-deep fp8
  // products (codes of key and query, exact products, fp32 sums) times the query and
  // entry scales, plus the RoPE dims by bf16 products from the converted tile K
  auto qk8 = [&](int st, const uint16_t* K, f32x4 (&sacc)[2]) {
    const uint8_t* Rw = reinterpret_cast<const uint8_t*>(ring + STAGE) + st * kKT * RAWROW;
    // codes 128 c + 32 grp .. + 32 of key row 16 kb + col (zero past the codes, where
    // the RoPE bf16 values lie)
    auto load8 = [&](int c, int kb) {
      uint4 lo = make_uint4(0u, 0u, 0u, 0u), hi = lo;
      if (128 * c + 32 * grp < D - R) {
        const uint8_t* p = Rw + (16 * kb + col) * RAWROW + 128 * c + 32 * grp;
        lo = *reinterpret_cast<const uint4*>(p);
        hi = *reinterpret_cast<const uint4*>(p + 16);
      }
      return v8i32{static_cast<int>(lo.x), static_cast<int>(lo.y), static_cast<int>(lo.z), static_cast<int>(lo.w),
                   static_cast<int>(hi.x), static_cast<int>(hi.y), static_cast<int>(hi.z), static_cast<int>(hi.w)};
    };
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    v8i32 kf[2];
    kf[0] = load8(0, 0);
    // (step c, key block kb) in order, the next one's fragment loading while this one's
    // product runs
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i + 1 < 8) kf[(i + 1) & 1] = load8((i + 1) >> 1, (i + 1) & 1);
      // formats 0 / 0: e4m3 on both sides; block scales 127 = 2^0
      sacc[i & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(kf[i & 1], q8[FQ ? (i >> 1) : 0], sacc[i & 1],
                                                                     0, 0, 0, 127, 0, 127);
      __builtin_amdgcn_sched_barrier(0);
    }
    // scaled code sums, then the RoPE dims' products accumulate onto them
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float4 es = *reinterpret_cast<const float4*>(&rscale[FP8 ? st : 0][16 * kb + 4 * grp]);
      sacc[kb][0] *= qsc * es.x;
      sacc[kb][1] *= qsc * es.y;
      sacc[kb][2] *= qsc * es.z;
      sacc[kb][3] *= qsc * es.w;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8 kr = *reinterpret_cast<const bf16x8*>(K + (16 * kb + col) * KP + nope + 32 * s2 + 8 * grp);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr, qf[s2], sacc[kb], 0, 0, 0);
      }
    }
  };
  // ---- S^T = K Q^T for the 32 keys of a tile (two 16-key blocks)
  auto qk = [&](const uint16_t* K, f32x4 (&sacc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(K + (16 * kb + col) * KP + 8 * grp + 32 * s);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[FQ ? 0 : s], sacc[kb], 0, 0, 0);
      }
    }
  };
  // ---- online softmax for head h over this lane's 8 keys (16kb + 4grp + r); returns P^T
  auto softmax = [&](int st, const f32x4 (&sacc)[2]) -> bf16x8 {
    float z[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float4 kb4 = *reinterpret_cast<const float4*>(&kbias[st][16 * kb + 4 * grp]);
      const float bias[4] = {kb4.x, kb4.y, kb4.z, kb4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = fmaf(sacc[kb][r], scale2, bias[r]);  // logit in base-2 units
        z[kb][r] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = rows4_max(mt);
    constexpr float kSlack = 8.f;  // lazy rescale, as in attn_mfma_kernel
    const bool raise = mt > m_run + kSlack;
    const float m_ref = raise ? mt : m_run;
    if (__any(raise)) {
      const float alpha = (m_run == -INFINITY || !raise) ? (raise ? 0.f : 1.f) : exp2_fast(m_run - m_ref);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
    }
    m_run = m_ref;
    const float m_use = m_run == -INFINITY ? 0.f : m_run;  // every key so far empty: each p is 2^-inf = 0
    float pn[8];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2_fast(z[kb][r] - m_use);
        psum += p;
        pn[4 * kb + r] = p;
      }
    }
    l_run += psum;
    return __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(pn[0], pn[1]), pack_bf16x2(pn[2], pn[3]),
                                                 pack_bf16x2(pn[4], pn[5]), pack_bf16x2(pn[6], pn[7])));
  };
  // ---- O^T += V^T P^T (V^T by transpose reads of the row-major tile)
  auto pv = [&](const uint16_t* K, const bf16x8 pB) {
    const uint16_t* vb = K + (4 * grp + (col >> 2)) * KP + 4 * (col & 3);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const s16x4 lo = lds_read_tr(vb + 16 * db);
      const s16x4 hi = lds_read_tr(vb + 16 * KP + 16 * db);
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pB, acc[db], 0, 0, 0);
    }
  };

  if constexpr (PIPE && !FP8) {
    // Software-pipelined: tile t+1's S^T products are issued before tile t's softmax,
    // so the softmax arithmetic runs while the matrix cores work.  Ring use at the top
    // of iteration t: t (its PV is pending), t+1 (products now), t+2 and t+3 in flight;
    // tile t+3 is issued once every wave is past tile t-1.
    f32x4 sc[2];
    if (ntiles > 0) {
      if (ntiles > 2) wait_vmcnt<2 * RPW>();
      else if (ntiles > 1) wait_vmcnt<RPW>();
      else wait_vmcnt<0>();
      __syncthreads();
      if (tile_has_window(0)) {
        rope_window_rows(0);
        __syncthreads();
      }
      qk(ring, sc);
    }
    for (int t = 0; t < ntiles; ++t) {
      const int st = t % kDmaStages;
      f32x4 sn[2];
      if (t + 1 < ntiles) {
        // issued so far: tiles 0 .. min(t + 2, ntiles - 1); wait for t+1
        if (t + 2 < ntiles) wait_vmcnt<RPW>();
        else wait_vmcnt<0>();
        __syncthreads();
        const int st1 = (t + 1) % kDmaStages;
        if (tile_has_window(t + 1)) {
          rope_window_rows(st1);
          __syncthreads();
        }
        if (t + 3 < ntiles) issue(t + 3);  // into the stage of tile t-1
        qk(ring + st1 * STAGE, sn);
      }
      const bf16x8 pB = softmax(st, sc);
      pv(ring + st * STAGE, pB);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) sc[kb] = sn[kb];
    }
  } else {
  for (int t = 0; t < ntiles; ++t) {
    const int st = t % kDmaStages;
    const int later = min(ntiles - 1 - t, kDmaStages - 2);  // tiles issued after t
    if (later >= 2) wait_vmcnt<2 * RPW * LPR>();
    else if (later == 1) wait_vmcnt<RPW * LPR>();
    else wait_vmcnt<0>();
    __syncthreads();
    if constexpr (FP8) {
      convert(st);  // the previous tile's readers are past the barrier above
      __syncthreads();
    } else if (tile_has_window(t)) {
      rope_window_rows(st);
      __syncthreads();
    }
    if (t + kDmaStages - 1 < ntiles) issue(t + kDmaStages - 1);  // into the stage freed by tile t-1

    const uint16_t* K = FP8 ? ring : ring + st * STAGE;
    f32x4 sacc[2];
    if constexpr (FQ) qk8(st, K, sacc);
    else qk(K, sacc);
    const bf16x8 pB = softmax(st, sacc);
    pv(K, pB);
  }
  }

  float l_tot = l_run;
  l_tot = rows4_sum(l_tot);

  // The result rows (normalised partials, or the final output) leave through LDS: each
  // lane holds 4 dims of one head, so direct stores would write 32-byte pieces of 16
  // rows; staged in the ring (free once every wave is past its last tile), each store
  // writes one 1 KiB row.
  const int64_t th = bt * a.H + h;
  const bool part = a.nsplit > 1;
  float scl;
  if (part) {
    scl = l_tot > 0.f ? 1.f / l_tot : 0.f;  // normalised partial: a convex combination of keys
  } else {
    const float sk = a.sink[h];
    if (sk == INFINITY) scl = 0.f;
    else if (sk == -INFINITY) scl = 1.f / l_tot;
    else scl = 1.f / (l_tot + exp2_fast(fmaf(sk, kLog2e, -m_run)));
  }
  __syncthreads();  // every wave is done reading the ring
  uint16_t* rows = ring + wid * 16 * KP;  // this wave's 16 result rows, pitch KP
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    const int d0 = 16 * db + 4 * grp;
    float v[4] = {acc[db][0] * scl, acc[db][1] * scl, acc[db][2] * scl, acc[db][3] * scl};
    if (!part && d0 >= nope) {
      // rotate back by the query position: angle -> -angle
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float2 cs = qcs[(d0 + e - nope) / 2];
        const float x0 = v[e], x1 = v[e + 1];
        v[e] = x0 * cs.x + x1 * cs.y;
        v[e + 1] = x1 * cs.x - x0 * cs.y;
      }
    }
    *reinterpret_cast<uint2*>(rows + col * KP + d0) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
  if (part && grp == 0) a.part_ml[th * a.nsplit + sp] = make_float2(m_run * kLn2, l_tot);  // natural-log units
  // lane l moves dims [8 l, 8 l + 8) of each of the wave's 16 rows (written by this wave)
  const int64_t h0 = bt * a.H + hg * a.hpw + wid * 16;  // the wave's first (token, head) row
#pragma unroll 4
  for (int r = 0; r < 16; ++r) {
    const uint4 v = *reinterpret_cast<const uint4*>(rows + r * KP + 8 * lane);
    uint16_t* dst = part ? a.part_o + ((h0 + r) * a.nsplit + sp) * D : static_cast<uint16_t*>(a.out) + (h0 + r) * D;
    store_row16(dst + 8 * lane, v, part);
  }
}

// ================================================================ wave-pair path (bf16, D = 512)
//
// The LDS-DMA kernel's tiles and row loads, with every block of 16 heads served by a
// pair of waves: wave 2p + h (h = 0, 1) of pair p takes key dims [256 h, 256 h + 256)
// of the S^T = K Q^T contraction and output dims [256 h, 256 h + 256) of
// O^T = V^T P^T.  The two halves of S^T meet through LDS (a + b is the same float in
// both waves, so both hold identical logits and take identical softmax steps).  A wave
// thereby holds half the queries and half the accumulators of the single-wave form,
// and the registers this frees hold a whole tile's operand fragments: every LDS read of
// a tile is issued before its MFMAs, where the single-wave form, at its register limit,
// waits one LDS round trip per MFMA.  Per 16 heads and tile the LDS traffic also drops
// from 64 KiB to 36 KiB (each wave reads half of every row twice and trades 2 KiB).
template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_pair_kernel(AttnArgs a) {
  constexpr int D = 512;
  constexpr int R = 64;
  constexpr int HD = D / 2;            // dims per wave
  constexpr int NT = NW * 64;
  constexpr int KP = D + 16;           // row pitch (bf16), as in attn_dma_kernel
  constexpr int NSH = HD / 32;         // k-steps of the half contraction
  constexpr int NDBH = HD / 16;        // 16-dim blocks of the half output
  constexpr int RPW = kKT / NW;        // rows each wave loads per tile
  constexpr int STAGE = kKT * KP;
  constexpr int nope = D - R;
  static_assert(NW % 2 == 0 && RPW * (kDmaStages - 2) < 64, "wave pairs; vmcnt range");

  __shared__ __attribute__((aligned(16))) uint16_t ring[kDmaStages * STAGE];
  __shared__ __attribute__((aligned(16))) int idx_s[kDmaIdxCap];
  __shared__ __attribute__((aligned(16))) float kbias[kDmaStages][kKT];  // 0, or -inf for an empty slot
  __shared__ int64_t wpos_s[kDmaStages][kKT];
  __shared__ float2 qcs[64];
  __shared__ double theta[64];
  __shared__ __attribute__((aligned(16))) f32x4 xch[NW][2][WAVE];  // S^T halves per wave and key block

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hw = wid & 1;              // dims half of this wave
  const int pr = wid >> 1;             // pair: heads 16 pr .. 16 pr + 15 of the group
  const int col = lane & 15;
  const int grp = lane >> 4;

  asm volatile("" ::"s"(a.H), "s"(a.hpw), "s"(a.nsplit), "s"(a.sps), "s"(a.K), "s"(a.sparse), "s"(a.n_win),
               "s"(a.ratio), "s"(a.Tq), "s"(a.N), "s"(a.kv_rows), "s"(a.Tw), "s"(a.pos_offset), "s"(a.q),
               "s"(a.q_pos), "s"(a.win_pos0), "s"(a.idx), "s"(a.kv), "s"(a.win), "s"(a.nblk));
  const uint32_t n_hg = static_cast<uint32_t>(a.H / a.hpw);
  const uint32_t blk = xcd_block(blockIdx.x, a.nblk);
  const int hg = __builtin_amdgcn_readfirstlane(static_cast<int>(blk % n_hg));
  const uint32_t blk2 = blk / n_hg;
  const int sp = __builtin_amdgcn_readfirstlane(static_cast<int>(blk2 % static_cast<uint32_t>(a.nsplit)));
  const int64_t bt = __builtin_amdgcn_readfirstlane(static_cast<int>(blk2 / static_cast<uint32_t>(a.nsplit)));
  const int64_t s_lo = static_cast<int64_t>(sp) * a.sps;
  const uint32_t ring_b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ring));
  const int64_t b_seq = static_cast<uint32_t>(bt) / static_cast<uint32_t>(a.Tq);
  const int64_t p_pre = a.q_pos[bt];
  const int64_t wp0_pre = a.win_pos0[b_seq];
  const double th_pre = tid < R / 2 ? a.theta_rev[tid] : 0.0;
  asm volatile("" ::: "memory");
  int32_t idx_pre[kDmaIdxCap / NT];
  const int64_t n_idx = a.sparse ? min(s_lo + a.sps, static_cast<int64_t>(a.K)) - s_lo : 0;
#pragma unroll
  for (int u = 0; u < kDmaIdxCap / NT; ++u) {
    const int64_t i = tid + static_cast<int64_t>(u) * NT;
    idx_pre[u] = i < n_idx ? a.idx[bt * a.K + s_lo + i] : 0;
  }
  asm volatile("" ::: "memory");  // keep the index loads ahead of the query loads
  const int h = hg * a.hpw + pr * 16 + col;  // head of this lane's result column
  uint4 qraw[NSH];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (bt * a.H + h) * D + HD * hw + 8 * grp;
#pragma unroll
    for (int s = 0; s < NSH; ++s) qraw[s] = *reinterpret_cast<const uint4*>(qrow + 32 * s);
  }
  const Slots S = slots_of(a, b_seq, uni64(p_pre), uni64(wp0_pre));
  const int64_t s_hi = min(S.nslots, s_lo + a.sps);
  const int ntiles = s_hi > s_lo ? static_cast<int>((s_hi - s_lo + kKT - 1) / kKT) : 0;
  const double qpos = static_cast<double>(S.p + a.pos_offset);
  const uint16_t* kvp = static_cast<const uint16_t*>(a.kv);
  const uint16_t* winp = static_cast<const uint16_t*>(a.win);

  if (tid < R / 2) {
    theta[tid] = th_pre;
    float c, sn;
    rope_cs_rev(qpos, th_pre, &c, &sn);
    qcs[tid] = make_float2(c, sn);
  }
#pragma unroll
  for (int u = 0; u < kDmaIdxCap / NT; ++u) {
    const int64_t i = tid + static_cast<int64_t>(u) * NT;
    if (i < n_idx) idx_s[i] = idx_pre[u];
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

  const int64_t u_lo = uni64(s_lo), u_hi = uni64(s_hi), u_nsel = uni64(S.nsel), u_wstart = uni64(S.wstart);
  const uint16_t* kv_b = kvp + uni64(S.b * a.kv_rows) * D;
  const uint16_t* win_b = winp + uni64(S.b * a.Tw - S.wp0) * D;
  const uint16_t* win_self = win_b + uni64(S.p) * D;
  // row loads of tile u into ring stage u % kDmaStages (one 1 KiB direct load per row;
  // an empty slot loads the query's own window row, which the softmax masks)
  auto issue = [&](int u) {
    const int st = u % kDmaStages;
    const uint16_t* src = win_self;
    if (lane < RPW) {
      const int j = wid * RPW + lane;
      const int64_t slot = u_lo + static_cast<int64_t>(u) * kKT + j;
      const bool live = slot < u_hi;
      const bool sel = slot < u_nsel;
      int64_t e = slot;
      if (a.sparse) e = idx_s[min(slot - u_lo, static_cast<int64_t>(kDmaIdxCap - 1))];
      const int64_t wp = u_wstart + (slot - u_nsel);
      const bool ok = live && (!sel || e >= 0);
      kbias[st][j] = ok ? 0.f : -INFINITY;
      wpos_s[st][j] = (ok && !sel) ? wp : -1;
      src = !ok ? win_self : (sel ? kv_b + e * D : win_b + wp * D);
    }
    const uint64_t sa = reinterpret_cast<uint64_t>(src);
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(sa), i));
      const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(sa >> 32), i));
      const uint16_t* row = reinterpret_cast<const uint16_t*>((hi << 32) | lo);
      lds_dma16(row + lane * 8, ring_b + (st * STAGE + (wid * RPW + i) * KP) * 2);
    }
  };
  constexpr int RCH = R / 8;
  auto rope_window_rows = [&](int st) {
    uint16_t* T = ring + st * STAGE;
    for (int item = tid; item < kKT * RCH; item += NT) {
      const int j = item / RCH;
      const int64_t wpj = wpos_s[st][j];
      if (wpj < 0) continue;
      const int d0 = nope + 8 * (item % RCH);
      uint4 v = *reinterpret_cast<const uint4*>(&T[j * KP + d0]);
      float x[8] = {bf16lo(v.x), bf16hi(v.x), bf16lo(v.y), bf16hi(v.y),
                    bf16lo(v.z), bf16hi(v.z), bf16lo(v.w), bf16hi(v.w)};
      const double kp = static_cast<double>(wpj + a.pos_offset);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        float cc, sn;
        rope_cs_rev(kp, theta[(d0 + e - nope) / 2], &cc, &sn);
        const float x0 = x[e], x1 = x[e + 1];
        x[e] = x0 * cc - x1 * sn;
        x[e + 1] = x0 * sn + x1 * cc;
      }
      *reinterpret_cast<uint4*>(&T[j * KP + d0]) =
          make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                     pack_bf16x2(x[6], x[7]));
    }
  };
  auto tile_has_window = [&](int t) {
    const int64_t first = s_lo + static_cast<int64_t>(t) * kKT;
    return min(first + kKT, s_hi) > S.nsel && first < s_hi;
  };

  // this wave's half of the queries, roped (only the upper half holds RoPE dims).  They
  // are complete before the first row load is issued: the compiler's waits for them
  // count only its own loads, and inside the loop such a wait would also wait for
  // every row load in flight.
  bf16x8 qf[NSH];
#pragma unroll
  for (int s = 0; s < NSH; ++s) {
    uint4 raw = qraw[s];
    const int d0 = HD * hw + 32 * s + 8 * grp;
    if (d0 + 8 > nope) {
      float v[8] = {bf16lo(raw.x), bf16hi(raw.x), bf16lo(raw.y), bf16hi(raw.y),
                    bf16lo(raw.z), bf16hi(raw.z), bf16lo(raw.w), bf16hi(raw.w)};
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        if (d0 + e >= nope) {
          const float2 cs = qcs[(d0 + e - nope) / 2];
          const float x0 = v[e], x1 = v[e + 1];
          v[e] = x0 * cs.x - x1 * cs.y;
          v[e + 1] = x0 * cs.y + x1 * cs.x;
        }
      }
      raw = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                       pack_bf16x2(v[6], v[7]));
    }
    qf[s] = __builtin_bit_cast(bf16x8, raw);
  }
#pragma unroll
  for (int s = 0; s < NSH; ++s) asm volatile("" : "+v"(qf[s]));
  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  if (ntiles > 2) issue(2);

  f32x4 acc[NDBH];
#pragma unroll
  for (int i = 0; i < NDBH; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // running max in base-2 units (logits scaled by scale * log2 e), exponentials by v_exp_f32
  const float scale2 = a.scale * kLog2e;
  float m_run = -INFINITY, l_run = 0.f;

  for (int t = 0; t < ntiles; ++t) {
    const int st = t % kDmaStages;
    const int later = min(ntiles - 1 - t, kDmaStages - 2);  // tiles issued after t
    if (later >= 2) wait_vmcnt<2 * RPW>();
    else if (later == 1) wait_vmcnt<RPW>();
    else wait_vmcnt<0>();
    __syncthreads();
    if (tile_has_window(t)) {
      rope_window_rows(st);
      __syncthreads();
    }
    if (t + kDmaStages - 1 < ntiles) issue(t + kDmaStages - 1);  // into the stage freed by tile t-1
    const uint16_t* K = ring + st * STAGE;

    // ---- this wave's half of S^T for the tile's two 16-key blocks: every K fragment is
    // read before the first product
    f32x4 sacc[2];
    {
      bf16x8 kf[2][NSH];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < NSH; ++s)
          kf[kb][s] = *reinterpret_cast<const bf16x8*>(K + (16 * kb + col) * KP + HD * hw + 8 * grp + 32 * s);
      __builtin_amdgcn_sched_barrier(0);  // keep every read ahead of the products
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NSH; ++s)
          sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][s], qf[s], sacc[kb], 0, 0, 0);
      }
    }
    // ---- the other half from the partner wave
    xch[wid][0][lane] = sacc[0];
    xch[wid][1][lane] = sacc[1];
    __syncthreads();
    {
      const f32x4 o0 = xch[wid ^ 1][0][lane], o1 = xch[wid ^ 1][1][lane];
      sacc[0] += o0;
      sacc[1] += o1;
    }
    // ---- online softmax for head h over this lane's 8 keys (16 kb + 4 grp + r); the two
    // waves of a pair compute the same values
    float z[2][4];
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float4 kb4 = *reinterpret_cast<const float4*>(&kbias[st][16 * kb + 4 * grp]);
      const float bias[4] = {kb4.x, kb4.y, kb4.z, kb4.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = fmaf(sacc[kb][r], scale2, bias[r]);  // logit in base-2 units
        z[kb][r] = v;
        mt = fmaxf(mt, v);
      }
    }
    mt = rows4_max(mt);
    constexpr float kSlack = 8.f;  // lazy rescale, as in attn_mfma_kernel
    const bool raise = mt > m_run + kSlack;
    const float m_ref = raise ? mt : m_run;
    if (__any(raise)) {
      const float alpha = (m_run == -INFINITY || !raise) ? (raise ? 0.f : 1.f) : exp2_fast(m_run - m_ref);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDBH; ++db) acc[db] *= alpha;
    }
    m_run = m_ref;
    const float m_use = m_run == -INFINITY ? 0.f : m_run;  // every key so far empty: each p is 2^-inf = 0
    float pn[8];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2_fast(z[kb][r] - m_use);
        psum += p;
        pn[4 * kb + r] = p;
      }
    }
    l_run += psum;
    const bf16x8 pB = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(pn[0], pn[1]), pack_bf16x2(pn[2], pn[3]),
                                                            pack_bf16x2(pn[4], pn[5]), pack_bf16x2(pn[6], pn[7])));
    // ---- O^T += V^T P^T over this wave's output dims (V^T by transpose reads, all
    // issued before the products)
    {
      const uint16_t* vb = K + (4 * grp + (col >> 2)) * KP + 4 * (col & 3) + HD * hw;
      s16x4 lo[NDBH], hi[NDBH];
#pragma unroll
      for (int db = 0; db < NDBH; ++db) {
        lo[db] = lds_read_tr(vb + 16 * db);
        hi[db] = lds_read_tr(vb + 16 * KP + 16 * db);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < NDBH; ++db) {
        const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo[db], hi[db], 0, 1, 2, 3, 4, 5, 6, 7));
        acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pB, acc[db], 0, 0, 0);
      }
    }
  }

  float l_tot = l_run;
  l_tot = rows4_sum(l_tot);

  const int64_t th = bt * a.H + h;
  const bool part = a.nsplit > 1;
  float scl;
  if (part) {
    scl = l_tot > 0.f ? 1.f / l_tot : 0.f;
  } else {
    const float sk = a.sink[h];
    if (sk == INFINITY) scl = 0.f;
    else if (sk == -INFINITY) scl = 1.f / l_tot;
    else scl = 1.f / (l_tot + exp2_fast(fmaf(sk, kLog2e, -m_run)));
  }
  __syncthreads();  // every wave is done reading the ring
  // result rows leave through LDS so that every store writes 512 contiguous bytes
  uint16_t* rows = ring + pr * 16 * KP + HD * hw;  // the pair's 16 rows, this wave's half
#pragma unroll
  for (int db = 0; db < NDBH; ++db) {
    const int d0 = HD * hw + 16 * db + 4 * grp;
    float v[4] = {acc[db][0] * scl, acc[db][1] * scl, acc[db][2] * scl, acc[db][3] * scl};
    if (!part && d0 >= nope) {
#pragma unroll
      for (int e = 0; e < 4; e += 2) {
        const float2 cs = qcs[(d0 + e - nope) / 2];
        const float x0 = v[e], x1 = v[e + 1];
        v[e] = x0 * cs.x + x1 * cs.y;
        v[e + 1] = x1 * cs.x - x0 * cs.y;
      }
    }
    *reinterpret_cast<uint2*>(rows + col * KP + 16 * db + 4 * grp) =
        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
  if (part && hw == 0 && grp == 0) a.part_ml[th * a.nsplit + sp] = make_float2(m_run * kLn2, l_tot);  // natural-log units
  // lanes 0-31 move row 2i, lanes 32-63 row 2i + 1: 16 bytes each of this wave's half
  const int64_t h0 = bt * a.H + hg * a.hpw + pr * 16;
  const int rsub = lane >> 5;
  const int dl = 8 * (lane & 31);
#pragma unroll 4
  for (int i = 0; i < 8; ++i) {
    const int r = 2 * i + rsub;
    const uint4 v = *reinterpret_cast<const uint4*>(rows + r * KP + dl);
    uint16_t* dst = part ? a.part_o + ((h0 + r) * a.nsplit + sp) * D : static_cast<uint16_t*>(a.out) + (h0 + r) * D;
    store_row16(dst + HD * hw + dl, v, part);
  }
}

// Merge the split partials of every (token, head) in split order: one wave per
// (token, head), lane l owns output dims [8l, 8l + 8) (D <= 512, nsplit <= 64).
// The split weights exp(m_i - M) * l_i are formed once per wave (lane i holds split
// i) and broadcast; every lane issues all its partial loads before combining.
template <int kBatchSplits>  // partial loads in flight per lane (no more than the splits when they fit)
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t th = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (th >= a.B * a.Tq * a.H) return;
  const int h = static_cast<int>(th % a.H);
  const int64_t bt = th / a.H;
  const int ns = a.nsplit;
  const int d0 = 8 * lane;
  const bool on = d0 < a.D;
  // every load this wave needs is issued before any is waited for: the sink, the
  // position, the split statistics and the first batch of partial rows.  The row loads
  // are unconditional (splits past ns re-read split 0, lanes past D re-read dims 0..7;
  // both get weight 0 or are not stored), so none waits inside a branch.
  const float sk = a.sink[h];
  const int64_t qp = a.q_pos[bt];
  const float2 ml = a.part_ml[th * ns + (lane < ns ? lane : 0)];
  const float mlx = lane < ns ? ml.x : -INFINITY;
  const uint16_t* pb = a.part_o + (th * ns) * a.D + (on ? d0 : 0);
  uint4 pv[kBatchSplits];
#pragma unroll
  for (int u = 0; u < kBatchSplits; ++u)
    pv[u] = load_stream16(pb + static_cast<int64_t>(u < ns ? u : 0) * a.D);
  const float M = wave_max_dpp(mlx);
  const float wgt = (mlx == -INFINITY) ? 0.f : __expf(mlx - M) * ml.y;
  const float L = wave_sum_dpp(wgt);
  float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < ns; i0 += kBatchSplits) {
    if (i0 > 0) {
#pragma unroll
      for (int u = 0; u < kBatchSplits; ++u)
        pv[u] = load_stream16(pb + static_cast<int64_t>(i0 + u < ns ? i0 + u : 0) * a.D);
    }
#pragma unroll
    for (int u = 0; u < kBatchSplits; ++u) {
      // splits past ns carry weight 0 (their lanes hold m = -inf) and finite rows
      const float w = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(wgt), (i0 + u) & 63));
      o[0] = fmaf(w, bf16lo(pv[u].x), o[0]); o[1] = fmaf(w, bf16hi(pv[u].x), o[1]);
      o[2] = fmaf(w, bf16lo(pv[u].y), o[2]); o[3] = fmaf(w, bf16hi(pv[u].y), o[3]);
      o[4] = fmaf(w, bf16lo(pv[u].z), o[4]); o[5] = fmaf(w, bf16hi(pv[u].z), o[5]);
      o[6] = fmaf(w, bf16lo(pv[u].w), o[6]); o[7] = fmaf(w, bf16hi(pv[u].w), o[7]);
    }
  }
  if (!on) return;
  float inv;
  if (sk == INFINITY) inv = 0.f;
  else if (sk == -INFINITY) inv = 1.f / L;
  else inv = 1.f / (L + __expf(sk - M));
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] *= inv;
  const int nope = a.D - a.R;
  if (d0 + 8 > nope) {
    const double qpos = static_cast<double>(qp + a.pos_offset);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      if (d0 + e >= nope) {
        float c, sn;
        rope_cs_rev(-qpos, a.theta_rev[(d0 + e - nope) / 2], &c, &sn);
        const float x0 = o[e], x1 = o[e + 1];
        o[e] = x0 * c - x1 * sn;
        o[e + 1] = x0 * sn + x1 * c;
      }
    }
  }
  if (a.out_dtype == CSA_F32) {
    float* op = static_cast<float*>(a.out) + th * a.D + d0;
    reinterpret_cast<float4*>(op)[0] = make_float4(o[0], o[1], o[2], o[3]);
    reinterpret_cast<float4*>(op)[1] = make_float4(o[4], o[5], o[6], o[7]);
  } else {
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + th * a.D + d0) =
        make_uint4(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7]));
  }
}

// ================================================================ SIMT path

constexpr int kSimtThreads = 256;
constexpr int kSimtHeads = 8;        // heads per workgroup, 32 lanes each
constexpr int kSimtLDS = 8192;       // floats of staged keys
constexpr int kSimtDPT = 32;         // max dims per lane (D <= 1024)

template <int KVF>
__device__ __forceinline__ float kv_elem(const AttnArgs& a, bool is_win, int64_t row, int d) {
  const void* base = is_win ? a.win : a.kv;
  if (KVF == CSA_F32) return static_cast<const float*>(base)[row * a.D + d];
  if (KVF == CSA_BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[row * a.D + d]);
  const int nope = a.D - a.R;
  if (d < nope) {
    const float* sc = is_win ? a.win_scale : a.kv_scale;
    return e4m3_to_f32(static_cast<const uint8_t*>(base)[row * nope + d]) * sc[row];
  }
  const uint16_t* rp = is_win ? a.win_rope : a.kv_rope;
  return bf16_to_f32(rp[row * a.R + (d - nope)]);
}

template <typename TQ, int KVF>
__global__ __launch_bounds__(kSimtThreads) void attn_simt_kernel(AttnArgs a) {
  __shared__ float kt[kSimtLDS];
  __shared__ int kvalid[kSimtLDS];
  const int D = a.D;
  const int KT = kSimtLDS / D;
  const int tid = threadIdx.x;
  const int hl = tid >> 5;       // head within group
  const int i = tid & 31;        // lane within head
  const int n_hg = (a.H + kSimtHeads - 1) / kSimtHeads;
  const int hg = static_cast<int>(blockIdx.x % n_hg);
  const int64_t bt = blockIdx.x / n_hg;
  const int h = hg * kSimtHeads + hl;
  const bool hok = h < a.H;
  const Slots S = token_slots(a, bt);
  const int nope = D - a.R;
  const double qpos = static_cast<double>(S.p + a.pos_offset);

  float q[kSimtDPT], acc[kSimtDPT];
  const TQ* qp = static_cast<const TQ*>(a.q) + (bt * a.H + (hok ? h : 0)) * D;
  auto ldq = [&](int d) -> float {
    if constexpr (sizeof(TQ) == 4) return reinterpret_cast<const float*>(qp)[d];
    else return bf16_to_f32(reinterpret_cast<const uint16_t*>(qp)[d]);
  };
#pragma unroll
  for (int u = 0; u < kSimtDPT; ++u) {
    const int d = i + 32 * u;
    q[u] = 0.f;
    acc[u] = 0.f;
    if (d < D) {
      float x = ldq(d);
      if (d >= nope) {
        float c, sn;
        rope_cs(qpos, (d - nope) / 2, a.R, a.log2_base, &c, &sn);
        const float xp = ldq(d ^ 1);
        x = (d & 1) ? fmaf(xp, sn, x * c) : fmaf(-xp, sn, x * c);
      }
      q[u] = x;
    }
  }
  float m_run = -INFINITY, l_run = 0.f;
  for (int64_t s0 = 0; s0 < S.nslots; s0 += KT) {
    __syncthreads();
    for (int e = tid; e < KT * D; e += kSimtThreads) {
      const int j = e / D;
      const int d = e % D;
      const int64_t slot = s0 + j;
      float v = 0.f;
      int ok = 0;
      if (slot < S.nslots) {
        bool is_win = false;
        int64_t wpos = 0;
        const int64_t row = slot_row(a, S, bt, slot, &is_win, &wpos);
        if (row >= 0) {
          ok = 1;
          v = kv_elem<KVF>(a, is_win, row, d);
          if (is_win && d >= nope) {
            float c, sn;
            rope_cs(static_cast<double>(wpos + a.pos_offset), (d - nope) / 2, a.R, a.log2_base, &c, &sn);
            const float vp = kv_elem<KVF>(a, is_win, row, d ^ 1);
            v = (d & 1) ? fmaf(vp, sn, v * c) : fmaf(-vp, sn, v * c);
          }
        }
      }
      kt[e] = v;
      if (d == 0) kvalid[j] = ok;
    }
    __syncthreads();
    const int nk = static_cast<int>(min(static_cast<int64_t>(KT), S.nslots - s0));
    for (int j = 0; j < nk; ++j) {
      float part = 0.f;
#pragma unroll
      for (int u = 0; u < kSimtDPT; ++u) {
        const int d = i + 32 * u;
        if (d < D) part = fmaf(q[u], kt[j * D + d], part);
      }
#pragma unroll
      for (int o = 16; o >= 1; o >>= 1) part += __shfl_xor(part, o, 32);
      if (!kvalid[j]) continue;
      const float z = a.scale * part;
      const float m_new = fmaxf(m_run, z);
      const float alpha = __expf(m_run - m_new);
      const float p = __expf(z - m_new);
      l_run = l_run * alpha + p;
#pragma unroll
      for (int u = 0; u < kSimtDPT; ++u) {
        const int d = i + 32 * u;
        if (d < D) acc[u] = fmaf(p, kt[j * D + d], acc[u] * alpha);
      }
      m_run = m_new;
    }
  }
  if (!hok) return;
  const float sk = a.sink[h];
  float inv;
  if (sk == INFINITY) inv = 0.f;
  else if (sk == -INFINITY) inv = 1.f / l_run;
  else inv = 1.f / (l_run + __expf(sk - m_run));
  TQ* op = static_cast<TQ*>(a.out) + (bt * a.H + h) * D;
#pragma unroll
  for (int u = 0; u < kSimtDPT; ++u) {
    const int d = i + 32 * u;
    float v = acc[u] * inv;
    // partner of the RoPE pair lives in lane i^1 (same u)
    const float vp = __shfl_xor(v, 1, 32);
    if (d < D) {
      if (d >= nope) {
        float c, sn;
        rope_cs(-qpos, (d - nope) / 2, a.R, a.log2_base, &c, &sn);
        v = (d & 1) ? fmaf(vp, sn, v * c) : fmaf(-vp, sn, v * c);
      }
      if constexpr (sizeof(TQ) == 4) reinterpret_cast<float*>(op)[d] = v;
      else reinterpret_cast<uint16_t*>(op)[d] = f32_to_bf16(v);
    }
  }
}

// ================================================================ planning

struct Plan {
  bool mfma;
  int hpw, nsplit, sps;
};

constexpr int kDmaMaxWaves = 8;

// Largest head group (multiple of 16 dividing H) of at most max_waves waves.
int head_group(int H, int max_waves) {
  int hpw = H;
  while (hpw > 16 * max_waves && (hpw / 2) % 16 == 0 && H % (hpw / 2) == 0) hpw /= 2;
  return hpw <= 16 * max_waves ? hpw : 0;
}

// Head group of attn_mfma_kernel.
int base_hpw(int H, int D) {
  return head_group(H, D >= 512 ? mfma_max_waves<512>() : mfma_max_waves<128>());
}

// Key-slot splits.  They depend on the per-sequence shape only (query tokens, heads,
// slots) and never on B, and the combine reads the splits in order, so a sequence's
// output is bitwise the same whatever else shares its batch (the pages ask decode to
// be batch-invariant and deterministic).  Decode-shaped launches (fewer than 256
// (token, head group) units per sequence) cut every query's slots into splits of at
// least kMinSplit slots, at most kMaxSplits of them; prefill-shaped ones do not split.
constexpr int64_t kMinSplitDma = 96;    // three 32-key tiles
constexpr int64_t kMinSplitMfma = 128;
constexpr int64_t kMaxSplitsSparse = 12;
constexpr int64_t kMaxSplitsDense = 8;  // long dense key lists: fewer, longer splits

// Which MFMA kernel a launch takes: the register-staged one, the LDS-DMA one (16 heads
// per wave) or the wave-pair one (16 heads per pair of waves).
enum class Kern { kReg, kDma, kPair };

constexpr int kPairMaxBlocks = 4;       // 16-head blocks per wave-pair workgroup (8 waves)
constexpr int64_t kMinSplitPair = 96;
constexpr int64_t kMaxSplitsSparsePair = 8;
// Longer key lists per query take the DMA kernel: the wave-pair kernel's head groups
// each load every key row, which costs more than its shorter chain saves once the
// rows, not the chain, set the time (an HCA decode query over all 8192 entries).
constexpr int64_t kPairMaxSlots = 4096;

Plan make_plan(int64_t B, int64_t Tq, int H, int D, int64_t max_slots, bool mfma, bool sparse, Kern kern) {
  Plan p{mfma, 0, 1, 0};
  if (!mfma) return p;
  const bool dma = kern != Kern::kReg;
  int hpw = kern == Kern::kPair ? head_group(H, kPairMaxBlocks)
                                : (kern == Kern::kDma ? head_group(H, kDmaMaxWaves) : base_hpw(H, D));
  if (hpw <= 0 || H % hpw != 0) {
    // no head group of an instantiated size: the SIMT kernel, which needs no workspace
    p.mfma = false;
    return p;
  }
  if (B * Tq == 0) {
    p.hpw = hpw;
    p.sps = kKT;
    return p;
  }
  int64_t units = Tq * (H / hpw);  // per sequence
  if (!dma) {
    // smaller head groups give more workgroups without split partials, but below these
    // sizes the prefetch registers no longer fit next to the accumulators
    const int min_hpw = D >= 512 ? 64 : (D >= 256 ? 32 : 16);
    while (units < 256 && hpw > min_hpw && (hpw / 2) % 16 == 0 && H % (hpw / 2) == 0) {
      hpw /= 2;
      units *= 2;
    }
  }
  int64_t ns = 1;
  if (units < 256) {
    const int64_t min_split = kern == Kern::kPair ? kMinSplitPair : (dma ? kMinSplitDma : kMinSplitMfma);
    // a long sparse list (every entry of an HCA decode query) splits like a dense one
    const int64_t mx = kern == Kern::kPair
                           ? kMaxSplitsSparsePair
                           : ((sparse && max_slots <= kPairMaxSlots) ? kMaxSplitsSparse : kMaxSplitsDense);
    ns = (max_slots + min_split - 1) / min_split;
    if (ns > mx) ns = mx;
    if (ns < 1) ns = 1;
  }
  // a sparse range's entry indices are staged in LDS by the DMA kernels
  if (sparse && max_slots <= 64 * kDmaIdxCap && ns < (max_slots + kDmaIdxCap - 1) / kDmaIdxCap)
    ns = (max_slots + kDmaIdxCap - 1) / kDmaIdxCap;
  int64_t sps = ((max_slots + ns - 1) / ns + kKT - 1) / kKT * kKT;
  if (sps < kKT) sps = kKT;
  ns = (max_slots + sps - 1) / sps;
  if (ns < 1) ns = 1;
  p.hpw = hpw;
  p.nsplit = static_cast<int>(ns);
  p.sps = static_cast<int>(sps);
  return p;
}

bool mfma_ok(const AttnLaunch& L) {
  if (L.q.dtype == CSA_FP8MIX) {
    // FP8MIX queries: only the LDS-DMA kernel's fp8 products (the entry points reject
    // every other shape before a launch)
    return L.kv.dtype == CSA_FP8MIX && L.D == 512 && L.rope_dims == 64 && L.H % 64 == 0 &&
           (head_group(L.H, kDmaMaxWaves) == 64 || head_group(L.H, kDmaMaxWaves) == 128);
  }
  if (L.q.dtype != CSA_BF16) return false;
  if (L.kv.dtype != CSA_BF16 && L.kv.dtype != CSA_FP8MIX) return false;
  if (L.win.dtype != L.kv.dtype) return false;
  if (L.H % 16 != 0) return false;
  if (L.D != 128 && L.D != 256 && L.D != 512) return false;
  const int nw = base_hpw(L.H, L.D) / 16;
  if (nw != 1 && nw != 2 && nw != 4 && nw != 8) return false;  // instantiated workgroup sizes
  if (L.rope_dims > 128) return false;
  if (L.kv.dtype == CSA_FP8MIX && ((L.D - L.rope_dims) % 32 != 0)) return false;
  return true;
}

int64_t max_slots_of(const AttnLaunch& L) {
  return (L.sparse ? static_cast<int64_t>(L.K) : L.N) + L.n_win;
}

// bf16 or FP8MIX cache, D = 512 with RoPE on the last 64 dims, 2, 4 or 8 waves: the
// LDS-DMA kernel (its row loads move 16-byte chunks of 16-byte aligned rows)
bool dma_ok(const AttnLaunch& L) {
  if (!mfma_ok(L) || L.D != 512 || L.rope_dims != 64) return false;
  if (L.kv.dtype == CSA_FP8MIX) {
    auto al = [](const void* p, uintptr_t m) { return (reinterpret_cast<uintptr_t>(p) & (m - 1)) == 0; };
    if (!al(L.kv.data, 16) || !al(L.win.data, 16) || !al(L.kv.rope, 16) || !al(L.win.rope, 16) ||
        !al(L.kv.scale, 4) || !al(L.win.scale, 4))
      return false;
  } else if (L.kv.dtype != CSA_BF16) {
    return false;
  }
  if (L.sparse && max_slots_of(L) > 64 * kDmaIdxCap) return false;
  const int nw = head_group(L.H, kDmaMaxWaves) / 16;
  if (L.kv.dtype == CSA_FP8MIX) return nw == 4 || nw == 8;  // three loads per row: 16 rows per wave would overflow vmcnt
  return nw == 2 || nw == 4 || nw == 8;
}

// bf16 cache, D = 512 with RoPE on the last 64 dims, 16, 32 or 64 heads per group: the
// wave-pair kernel
bool pair_ok(const AttnLaunch& L) {
  if (!dma_ok(L) || L.kv.dtype != CSA_BF16) return false;
  const int hpw = head_group(L.H, kPairMaxBlocks);
  return hpw == 16 || hpw == 32 || hpw == 64;
}

// The wave-pair kernel serves sparse decode-shaped launches (fewer than 256 (token,
// 128-head group) units per sequence, so the key slots are split): there its shorter
// per-tile chain wins.  Prefill and dense launches keep 128 heads per workgroup, which
// loads each key tile once per token.  The choice depends on the per-sequence shape only.
Kern kern_of(const AttnLaunch& L) {
  if (!dma_ok(L)) return Kern::kReg;
  const int hpw = head_group(L.H, kDmaMaxWaves);
  if (L.sparse && pair_ok(L) && hpw > 0 && L.Tq * (L.H / hpw) < 256 && max_slots_of(L) <= kPairMaxSlots)
    return Kern::kPair;
  return Kern::kDma;
}

AttnArgs make_args(const AttnLaunch& L, const Plan& P, void* ws) {
  AttnArgs a{};
  a.q = L.q.data;
  a.q_rope = static_cast<const uint16_t*>(L.q.rope);
  a.q_scale = static_cast<const float*>(L.q.scale);
  a.q_pos = L.q_pos;
  a.kv = L.kv.data;
  a.kv_rope = static_cast<const uint16_t*>(L.kv.rope);
  a.kv_scale = static_cast<const float*>(L.kv.scale);
  a.kv_rows = L.kv_rows;
  a.win = L.win.data;
  a.win_rope = static_cast<const uint16_t*>(L.win.rope);
  a.win_scale = static_cast<const float*>(L.win.scale);
  a.win_pos0 = L.win_pos0;
  a.Tw = L.Tw;
  a.idx = L.idx;
  a.K = L.K;
  a.ratio = L.ratio;
  a.sparse = L.sparse;
  a.sink = L.sink;
  a.scale = L.scale;
  a.R = L.rope_dims;
  a.log2_base = L.log2_base;
  for (int j = 0; j < 64; ++j)
    a.theta_rev[j] = j < L.rope_dims / 2
                         ? std::exp2(-2.0 * j / L.rope_dims * L.log2_base) * 0.15915494309189533576888376337251
                         : 0.0;
  a.pos_offset = L.pos_offset;
  a.B = L.B;
  a.Tq = L.Tq;
  a.N = L.N;
  a.H = L.H;
  a.D = L.D;
  a.n_win = L.n_win;
  a.hpw = P.hpw;
  a.nsplit = P.nsplit;
  a.sps = P.sps;
  a.out = L.out.data;
  a.out_dtype = L.out.dtype;
  if (P.mfma && P.nsplit > 1) {
    const int64_t th = L.B * L.Tq * L.H;
    a.part_o = static_cast<uint16_t*>(ws);
    a.part_ml = reinterpret_cast<float2*>(static_cast<char*>(ws) + th * P.nsplit * L.D * sizeof(uint16_t));
  }
  return a;
}

}  // namespace

bool attn_uses_mfma(const AttnLaunch& L) { return mfma_ok(L); }

size_t attn_workspace_bytes(int64_t B, int64_t Tq, int H, int D, int64_t max_slots, bool sparse) {
  // the larger of the two MFMA kernels' needs (which one runs depends on the cache dtype)
  if (H < 1 || D < 1) return 0;
  int64_t ns = make_plan(B, Tq, H, D, max_slots, true, sparse, Kern::kReg).nsplit;
  if (D == 512) {
    ns = std::max<int64_t>(ns, make_plan(B, Tq, H, D, max_slots, true, sparse, Kern::kDma).nsplit);
    ns = std::max<int64_t>(ns, make_plan(B, Tq, H, D, max_slots, true, sparse, Kern::kPair).nsplit);
  }
  if (ns <= 1) return 0;
  const int64_t th = B * Tq * H;
  return static_cast<size_t>(th * ns) * (static_cast<size_t>(D) * sizeof(uint16_t) + sizeof(float2));
}

int launch_attn(const AttnLaunch& L, void* ws, size_t ws_bytes, hipStream_t stream) {
  const int64_t tokens = L.B * L.Tq;
  if (tokens == 0) return 0;
  const Kern kern = kern_of(L);
  // FP8MIX queries run only on the LDS-DMA kernel's fp8 products (its alignment and
  // staged-index limits included)
  if (L.q.dtype == CSA_FP8MIX && kern != Kern::kDma) return -2;
  const bool dma = mfma_ok(L) && kern != Kern::kReg;
  const Plan P = make_plan(L.B, L.Tq, L.H, L.D, max_slots_of(L), mfma_ok(L), L.sparse != 0, kern);
  const bool mfma = P.mfma;
  if (mfma && P.nsplit > 1 && ws_bytes < attn_workspace_bytes(L.B, L.Tq, L.H, L.D, max_slots_of(L), L.sparse != 0))
    return -3;
  AttnArgs a = make_args(L, P, ws);
  if (mfma) {
    const int64_t grid = tokens * (L.H / P.hpw) * P.nsplit;
    if (grid >= (static_cast<int64_t>(1) << 32)) return -4;  // the kernels index blocks in 32 bits
    a.nblk = static_cast<uint32_t>(grid);
    const dim3 block(P.hpw / 16 * WAVE);
    const bool fp8 = L.kv.dtype == CSA_FP8MIX;
#define CSA_LAUNCH_MFMA_W(DD, NWV)                                                                     \
  if (L.D == DD && nw == NWV) {                                                                        \
    if (fp8) hipLaunchKernelGGL((attn_mfma_kernel<DD, NWV, true>), dim3(static_cast<uint32_t>(grid)), block, 0, stream, a); \
    else hipLaunchKernelGGL((attn_mfma_kernel<DD, NWV, false>), dim3(static_cast<uint32_t>(grid)), block, 0, stream, a);    \
  }
#define CSA_LAUNCH_MFMA(DD) CSA_LAUNCH_MFMA_W(DD, 1) CSA_LAUNCH_MFMA_W(DD, 2) CSA_LAUNCH_MFMA_W(DD, 4)
    const int nw = P.hpw / 16;
    if (dma) {
      if (L.sparse && P.sps > kDmaIdxCap) return -1;  // excluded by the plan
      const dim3 g(static_cast<uint32_t>(grid));
      if (kern == Kern::kPair) {  // two waves per 16 heads
        const dim3 pb(P.hpw / 8 * WAVE);
        if (P.hpw == 64) hipLaunchKernelGGL(attn_pair_kernel<8>, g, pb, 0, stream, a);
        else if (P.hpw == 32) hipLaunchKernelGGL(attn_pair_kernel<4>, g, pb, 0, stream, a);
        else hipLaunchKernelGGL(attn_pair_kernel<2>, g, pb, 0, stream, a);
      } else if (fp8 && L.q.dtype == CSA_FP8MIX) {  // fp8 query products, 4 or 8 waves
        if (nw == 8) hipLaunchKernelGGL((attn_dma_kernel<8, 64, true, false, true>), g, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_dma_kernel<4, 64, true, false, true>), g, block, 0, stream, a);
      } else if (fp8) {  // 4 or 8 waves (dma_ok)
        if (nw == 8) hipLaunchKernelGGL((attn_dma_kernel<8, 64, true>), g, block, 0, stream, a);
        else hipLaunchKernelGGL((attn_dma_kernel<4, 64, true>), g, block, 0, stream, a);
      } else {
        if (kDmaPipe && (P.nsplit == 1 || P.sps >= kPipeMinSlots)) {  // long ranges: the pipelined loop
          if (nw == 8) hipLaunchKernelGGL((attn_dma_kernel<8, 64, false, true>), g, block, 0, stream, a);
          else if (nw == 4) hipLaunchKernelGGL((attn_dma_kernel<4, 64, false, true>), g, block, 0, stream, a);
          else hipLaunchKernelGGL((attn_dma_kernel<2, 64, false, true>), g, block, 0, stream, a);
        } else {
          if (nw == 8) hipLaunchKernelGGL((attn_dma_kernel<8, 64, false>), g, block, 0, stream, a);
          else if (nw == 4) hipLaunchKernelGGL((attn_dma_kernel<4, 64, false>), g, block, 0, stream, a);
          else hipLaunchKernelGGL((attn_dma_kernel<2, 64, false>), g, block, 0, stream, a);
        }
      }
    } else {
    CSA_LAUNCH_MFMA(128)
    CSA_LAUNCH_MFMA(256)
    CSA_LAUNCH_MFMA(512)
    CSA_LAUNCH_MFMA_W(128, 8)
    CSA_LAUNCH_MFMA_W(256, 8)
    }
#undef CSA_LAUNCH_MFMA
#undef CSA_LAUNCH_MFMA_W
    if (hipGetLastError() != hipSuccess) return -1;
    if (P.nsplit > 1) {
      const int64_t waves = tokens * L.H;
      const dim3 cg(static_cast<uint32_t>((waves + 3) / 4));
      if (P.nsplit <= 8) hipLaunchKernelGGL(attn_combine_kernel<8>, cg, dim3(256), 0, stream, a);
      else hipLaunchKernelGGL(attn_combine_kernel<16>, cg, dim3(256), 0, stream, a);
      if (hipGetLastError() != hipSuccess) return -1;
    }
    return 0;
  }
  const int n_hg = (L.H + kSimtHeads - 1) / kSimtHeads;
  const dim3 grid(static_cast<uint32_t>(tokens * n_hg));
  const bool qf32 = L.q.dtype == CSA_F32;
#define CSA_LAUNCH_SIMT(KVF)                                                                                \
  if (L.kv.dtype == KVF) {                                                                                  \
    if (qf32) hipLaunchKernelGGL((attn_simt_kernel<float, KVF>), grid, dim3(kSimtThreads), 0, stream, a);   \
    else hipLaunchKernelGGL((attn_simt_kernel<uint16_t, KVF>), grid, dim3(kSimtThreads), 0, stream, a);     \
  }
  CSA_LAUNCH_SIMT(CSA_F32)
  CSA_LAUNCH_SIMT(CSA_BF16)
  CSA_LAUNCH_SIMT(CSA_FP8MIX)
#undef CSA_LAUNCH_SIMT
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
